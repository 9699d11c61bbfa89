"""Seeded synthetic inputs for the Qwen3-0.6B-shaped KV-cache decoder.

This module only draws numbers: weights, prompt ids, audio embedding rows and
forced token streams. It holds none of the decoder's arithmetic, so both the
CPU oracle (through the tests) and the HIP path consume exactly the same bits.

Shapes follow the decoder described on the audio.cpp "Fun-ASR-Nano Native
Runtime Implementation Plan" page (Task 1 Step 1 and Task 6 Step 4: hidden 1024,
FFN 3072, 28 layers, 16 query / 8 KV heads, head_dim 128, vocab 151936,
RoPE theta 1e6, tied embeddings) and on the transcribe.cpp "Forward map -
funasr_nano" page (LLM decoder table: per-head Q/K-RMSNorm, packed gate_up).
No checkpoint exists here, so weights are random: matrices 0.02*N(0,1), norm
gains 1 + 0.02*N(0,1), drawn in one fixed tensor order.

RNG contract: numpy Generator(PCG64(SeedSequence([seed_id, stream]))).
stream 0 = weights, 1 = prompt ids, 2 = audio rows, 10+b = forced stream of
branch b. The 0.6B workloads share one weight set (seed_id 2).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

# Canonical per-layer tensor order (also the order of the C-ABI weight table).
LAYER_TENSORS = (
    "in_norm", "wq", "wk", "wv", "q_norm", "k_norm",
    "wo", "post_norm", "w_gate", "w_up", "w_down",
)
NORM_TENSORS = ("in_norm", "q_norm", "k_norm", "post_norm")


@dataclasses.dataclass(frozen=True)
class ModelShape:
    hidden: int
    n_layer: int
    n_q_head: int
    n_kv_head: int
    head_dim: int
    ffn: int
    vocab: int
    rms_eps: float = 1e-6
    rope_theta: float = 1e6
    bf16: bool = True  # weights stored as bf16 (RNE); False = fp32


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    shape: ModelShape
    weight_seed: int
    prompt_seed: int
    prompt_len: int
    audio_begin: int
    audio_len: int
    n_decode: int
    n_branch: int = 1  # >1: the prompt is prefilled once and cloned

    @property
    def max_ctx(self) -> int:
        return self.prompt_len + self.n_decode


TINY = ModelShape(hidden=128, n_layer=2, n_q_head=4, n_kv_head=2, head_dim=32,
                  ffn=384, vocab=1024, bf16=False)
QWEN3_0P6B = ModelShape(hidden=1024, n_layer=28, n_q_head=16, n_kv_head=8,
                        head_dim=128, ffn=3072, vocab=151936, bf16=True)

WORKLOADS: Dict[str, Workload] = {
    # tiny fp32 decoder: 32-token prompt, rows 8..15 audio, 8 forced steps
    "tiny": Workload("tiny", TINY, 1, 1, 32, 8, 8, 8),
    # 0.6B: 48-token prompt, 23 audio rows, 64 greedy steps
    "short": Workload("short", QWEN3_0P6B, 2, 2, 48, 8, 23, 64),
    # 0.6B: 1024-token prompt, 750 audio rows, 256 steps
    "long": Workload("long", QWEN3_0P6B, 2, 3, 1024, 8, 750, 256),
    # 0.6B: 512-token shared prefix, 128 audio rows, 16 branches x 128 steps
    "branch16": Workload("branch16", QWEN3_0P6B, 2, 4, 512, 8, 128, 128, n_branch=16),
    # 0.6B: 8192-token prompt, 6000 audio rows, 64 steps
    "prefill8k": Workload("prefill8k", QWEN3_0P6B, 2, 5, 8192, 8, 6000, 64),
    # 0.6B: 3001-token prompt (ragged against every tile size), 2000 audio rows, 16 steps
    "ragged3k": Workload("ragged3k", QWEN3_0P6B, 2, 6, 3001, 8, 2000, 16),
    # tiny fp32 decoder at the decode kernel's position limit: a 16381-token
    # prompt, then greedy steps at positions 16381, 16382 and 16383 (the last)
    "tiny_maxpos": Workload("tiny_maxpos", TINY, 1, 7, 16381, 8, 8, 3),
}


def _rng(seed_id: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed_id, stream])))


def layer_shapes(s: ModelShape) -> Dict[str, tuple]:
    H, D, F = s.hidden, s.head_dim, s.ffn
    return {
        "in_norm": (H,), "wq": (s.n_q_head * D, H), "wk": (s.n_kv_head * D, H),
        "wv": (s.n_kv_head * D, H), "q_norm": (D,), "k_norm": (D,),
        "wo": (H, s.n_q_head * D), "post_norm": (H,), "w_gate": (F, H),
        "w_up": (F, H), "w_down": (H, F),
    }


def _round_bf16(a: np.ndarray):
    """Round float32 -> bf16 (round to nearest even, torch on the CPU).
    Returns (uint16 bit patterns, exact float32 upcast)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16), t.float().numpy()


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact upcast of bf16 bit patterns (uint16) to float32."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


class Weights:
    """One weight set. ``f32[name]`` holds float32 arrays whose values are
    exactly representable in the storage type; ``bits[name]`` holds the bf16
    bit patterns (uint16) for bf16 shapes (None for fp32 shapes).
    Names: "embed", "final_norm", and "L{i}.{tensor}" per layer."""

    def __init__(self, shape: ModelShape, f32: Dict[str, np.ndarray],
                 bits: Optional[Dict[str, np.ndarray]]):
        self.shape = shape
        self.f32 = f32
        self.bits = bits

    def names(self) -> List[str]:
        out = ["embed"]
        for i in range(self.shape.n_layer):
            out += [f"L{i}.{t}" for t in LAYER_TENSORS]
        out.append("final_norm")
        return out

    def layer(self, i: int) -> Dict[str, np.ndarray]:
        return {t: self.f32[f"L{i}.{t}"] for t in LAYER_TENSORS}


_WEIGHT_CACHE: Dict[tuple, Weights] = {}


def make_weights(shape: ModelShape, seed_id: int, cache: bool = True) -> Weights:
    """Draw one weight set in canonical order from stream 0."""
    key = (shape, seed_id)
    if cache and key in _WEIGHT_CACHE:
        return _WEIGHT_CACHE[key]
    rng = _rng(seed_id, 0)
    scale = np.float32(0.02)
    order = [("embed", (shape.vocab, shape.hidden), False)]
    shp = layer_shapes(shape)
    for i in range(shape.n_layer):
        for t in LAYER_TENSORS:
            order.append((f"L{i}.{t}", shp[t], t in NORM_TENSORS))
    order.append(("final_norm", (shape.hidden,), True))
    f32: Dict[str, np.ndarray] = {}
    bits: Optional[Dict[str, np.ndarray]] = {} if shape.bf16 else None
    for name, shp_, is_gain in order:
        z = rng.standard_normal(shp_, dtype=np.float32)
        w = (np.float32(1.0) + scale * z) if is_gain else (scale * z)
        w = w.astype(np.float32, copy=False)
        if shape.bf16:
            bits[name], f32[name] = _round_bf16(w)
        else:
            f32[name] = w
    out = Weights(shape, f32, bits)
    if cache:
        _WEIGHT_CACHE[key] = out
    return out


def make_prompt(w: Workload):
    """Prompt ids (int32[T], uniform over the vocabulary, stream 1) and audio
    rows (float32[La, H], N(0,1), stream 2) for span [audio_begin, +audio_len)."""
    s = w.shape
    ids = _rng(w.prompt_seed, 1).integers(0, s.vocab, size=w.prompt_len).astype(np.int32)
    audio = _rng(w.prompt_seed, 2).standard_normal((w.audio_len, s.hidden), dtype=np.float32)
    return ids, audio, w.audio_begin


def branch_stream(w: Workload, b: int, n: Optional[int] = None) -> np.ndarray:
    """Forced token stream of branch b (uniform ids, stream 10+b)."""
    n = w.n_decode if n is None else n
    return _rng(w.prompt_seed, 10 + b).integers(0, w.shape.vocab, size=n).astype(np.int32)


@dataclasses.dataclass(frozen=True)
class AdaptorShape:
    """Sizes of the audio adaptor (linear1, linear2, pre-norm blocks)."""
    enc_dim: int = 512
    mid_dim: int = 2048
    dim: int = 1024
    ffn_dim: int = 256
    n_block: int = 2
    n_head: int = 8


def adaptor_params(a: AdaptorShape) -> List[tuple]:
    """(name, shape, kind) in draw order; kind "w" matrix [out, in], "b" bias,
    "g" LayerNorm gain."""
    D, F = a.dim, a.ffn_dim
    out = [("linear1.w", (a.mid_dim, a.enc_dim), "w"), ("linear1.b", (a.mid_dim,), "b"),
           ("linear2.w", (D, a.mid_dim), "w"), ("linear2.b", (D,), "b")]
    for i in range(a.n_block):
        p = f"blocks.{i}."
        out += [(p + "norm1.g", (D,), "g"), (p + "norm1.b", (D,), "b")]
        for t in ("q", "k", "v", "o"):
            out += [(p + t + ".w", (D, D), "w"), (p + t + ".b", (D,), "b")]
        out += [(p + "norm2.g", (D,), "g"), (p + "norm2.b", (D,), "b"),
                (p + "fc1.w", (F, D), "w"), (p + "fc1.b", (F,), "b"),
                (p + "fc2.w", (D, F), "w"), (p + "fc2.b", (D,), "b")]
    return out


def make_adaptor_weights(a: AdaptorShape, seed_id: int):
    """Adaptor parameters from stream 3, in adaptor_params order: matrices and
    biases 0.02 N(0,1), gains 1 + 0.02 N(0,1), rounded to bf16. Returns
    (float32 values, bf16 bit patterns), both keyed by name."""
    rng = _rng(seed_id, 3)
    scale = np.float32(0.02)
    f32: Dict[str, np.ndarray] = {}
    bits: Dict[str, np.ndarray] = {}
    for name, shp, kind in adaptor_params(a):
        z = rng.standard_normal(shp, dtype=np.float32)
        w = (np.float32(1.0) + scale * z) if kind == "g" else (scale * z)
        bits[name], f32[name] = _round_bf16(w.astype(np.float32, copy=False))
    return f32, bits


@dataclasses.dataclass(frozen=True)
class EncoderShape:
    """Sizes of the SAN-M speech encoder (stem, main blocks, tp blocks)."""
    in_dim: int = 560
    dim: int = 512
    n_head: int = 4
    ffn_dim: int = 2048
    kernel: int = 11
    n_main: int = 49
    n_tp: int = 20

    def block_names(self) -> List[str]:
        return (["encoders0.0."] + [f"encoders.{i}." for i in range(self.n_main)]
                + [f"tp_encoders.{i}." for i in range(self.n_tp)])


def encoder_params(e: EncoderShape) -> List[tuple]:
    """(name, shape, kind) in draw order; kind "w" matrix [out, in], "b" bias,
    "g" LayerNorm gain, "f" FSMN taps [dim, kernel]."""
    D, F = e.dim, e.ffn_dim
    out = []
    for b, p in enumerate(e.block_names()):
        n_in = e.in_dim if b == 0 else D
        out += [(p + "norm1.g", (n_in,), "g"), (p + "norm1.b", (n_in,), "b")]
        for t in ("q", "k", "v"):
            out += [(p + t + ".w", (D, n_in), "w"), (p + t + ".b", (D,), "b")]
        out += [(p + "fsmn.w", (D, e.kernel), "f"), (p + "o.w", (D, D), "w"), (p + "o.b", (D,), "b"),
                (p + "norm2.g", (D,), "g"), (p + "norm2.b", (D,), "b"),
                (p + "ffn1.w", (F, D), "w"), (p + "ffn1.b", (F,), "b"),
                (p + "ffn2.w", (D, F), "w"), (p + "ffn2.b", (D,), "b")]
    out += [("after_norm.g", (D,), "g"), ("after_norm.b", (D,), "b"),
            ("tp_norm.g", (D,), "g"), ("tp_norm.b", (D,), "b")]
    return out


def make_encoder_weights(e: EncoderShape, seed_id: int):
    """Encoder parameters from stream 6, in encoder_params order: matrices and
    biases 0.02 N(0,1), gains 1 + 0.02 N(0,1), FSMN taps 0.1 N(0,1), rounded
    to bf16. Returns (float32 values, bf16 bit patterns), keyed by name."""
    rng = _rng(seed_id, 6)
    f32: Dict[str, np.ndarray] = {}
    bits: Dict[str, np.ndarray] = {}
    for name, shp, kind in encoder_params(e):
        z = rng.standard_normal(shp, dtype=np.float32)
        if kind == "g":
            w = np.float32(1.0) + np.float32(0.02) * z
        else:
            w = (np.float32(0.1) if kind == "f" else np.float32(0.02)) * z
        bits[name], f32[name] = _round_bf16(w.astype(np.float32, copy=False))
    return f32, bits


SAMPLE_RATE = 16000


def pcm(kind: str, n: int, seed_id: int = 0) -> np.ndarray:
    """Synthetic 16 kHz PCM float32[n] at 16-bit sample scale: "silence";
    "impulse" (one sample of 10000 at n // 2); "sine440" (amplitude 8000);
    "voiced" (stream 7): a harmonic tone whose pitch glides between 100 and
    250 Hz, five harmonics with 1/h amplitudes, a 4 Hz syllable envelope and
    white noise, peak about 10000 -- a speech-like spectrum, not speech."""
    t = np.arange(n, dtype=np.float64) / SAMPLE_RATE
    if kind == "silence":
        x = np.zeros(n)
    elif kind == "impulse":
        x = np.zeros(n)
        x[n // 2] = 10000.0
    elif kind == "sine440":
        x = 8000.0 * np.sin(2 * np.pi * 440.0 * t)
    elif kind == "voiced":
        rng = _rng(seed_id, 7)
        f0 = 175.0 + 75.0 * np.sin(2 * np.pi * rng.uniform(0.3, 0.8) * t + rng.uniform(0, 2 * np.pi))
        phase = 2 * np.pi * np.cumsum(f0) / SAMPLE_RATE
        x = sum(np.sin(h * phase) / h for h in range(1, 6))
        x *= 0.55 + 0.45 * np.sin(2 * np.pi * 4.0 * t + rng.uniform(0, 2 * np.pi))
        x = 4000.0 * x + 300.0 * rng.standard_normal(n)
    else:
        raise ValueError(kind)
    return x.astype(np.float32)


def encoder_frames(seed_id: int, n: int, width: int) -> np.ndarray:
    """Encoder output frames float32[n, width], N(0,1), stream 4."""
    return _rng(seed_id, 4).standard_normal((n, width), dtype=np.float32)


def random_ids(seed: int, n: int, vocab: int) -> np.ndarray:
    return _rng(1000 + seed, 1).integers(0, vocab, size=n).astype(np.int32)


def random_rows(seed: int, n: int, width: int) -> np.ndarray:
    return _rng(1000 + seed, 2).standard_normal((n, width), dtype=np.float32)


def custom_shape(**kw) -> ModelShape:
    return dataclasses.replace(TINY, **kw)


# ------------------------------------------------------------------ Q8_0

# The matrices a Q8_0 weight set stores as blocks, besides the embedding
# (the norm gains stay float).
Q8_MATRICES = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")
Q8_BLOCK = 32          # inputs per block
Q8_BLOCK_BYTES = 34    # fp16 scale, then 32 int8 codes


class Q8Weights:
    """A Q8_0 weight set. ``codes[name]`` int8 [out, in] and ``scales[name]``
    float16 [out, in / 32] for the embedding ("embed") and the seven matrices
    of each layer, ``blocks[name]`` the same data as bytes, one row of in / 32
    blocks of 34 bytes each (the block's fp16 scale, then its 32 codes);
    ``base`` is the weight set of the same seed whose norm gains (float32
    values) the Q8_0 set shares."""

    def __init__(self, base: Weights, codes, scales, blocks):
        self.shape = base.shape
        self.base = base
        self.codes = codes
        self.scales = scales
        self.blocks = blocks

    def abi_arrays(self) -> Dict[str, np.ndarray]:
        """The mapping the C ABI takes for Q8_0: blocks for the matrices and
        the embedding, float32 norm gains."""
        out = dict(self.blocks)
        for name in self.base.names():
            if name not in out:
                out[name] = self.base.f32[name]
        return out


def pack_q8_blocks(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Byte layout of Q8_0 rows: block b of a row is scales[:, b] (fp16, little
    endian) followed by codes[:, 32 b : 32 b + 32]."""
    out, n = codes.shape
    nb = n // Q8_BLOCK
    blk = np.empty((out, nb, Q8_BLOCK_BYTES), np.uint8)
    blk[:, :, :2] = np.ascontiguousarray(scales.astype("<f2")).view(np.uint8).reshape(out, nb, 2)
    blk[:, :, 2:] = codes.reshape(out, nb, Q8_BLOCK).view(np.uint8)
    return blk.reshape(out, nb * Q8_BLOCK_BYTES)


_Q8_CACHE: Dict[tuple, Q8Weights] = {}


def make_q8_weights(shape: ModelShape, seed_id: int) -> Q8Weights:
    """Draw a Q8_0 weight set (stream 5): for the embedding, then each layer's
    matrices in order, codes
    clip(rint(8 N(0, 1)), -127, 127) (a bell with standard deviation about 8),
    1% of them replaced by uniform codes over [-127, 127] so that every code
    value occurs, and per-block fp16 scales 0.002 U(0.8, 1.2), so the weights
    q d have a standard deviation near 0.022, like the bf16 sets' 0.02. No
    quantizer is involved: codes and scales are the drawn data."""
    key = (shape, seed_id)
    if key in _Q8_CACHE:
        return _Q8_CACHE[key]
    base = make_weights(shape, seed_id)
    rng = _rng(seed_id, 5)
    shp = layer_shapes(shape)
    order = [("embed", (shape.vocab, shape.hidden))]
    order += [(f"L{i}.{t}", shp[t]) for i in range(shape.n_layer) for t in Q8_MATRICES]
    codes, scales, blocks = {}, {}, {}
    for name, (out, n) in order:
        g = rng.standard_normal((out, n), dtype=np.float32)
        q = np.clip(np.rint(np.float32(8.0) * g), -127, 127).astype(np.int8)
        wide = np.flatnonzero(rng.random((out, n), dtype=np.float32) < np.float32(0.01))
        q.reshape(-1)[wide] = rng.integers(-127, 128, size=wide.size).astype(np.int8)
        d = (np.float32(0.002) * rng.uniform(0.8, 1.2, size=(out, n // Q8_BLOCK))).astype(np.float16)
        codes[name], scales[name] = q, d
        blocks[name] = pack_q8_blocks(q, d)
    out_w = Q8Weights(base, codes, scales, blocks)
    _Q8_CACHE[key] = out_w
    return out_w
