"""CPU oracle of the SAN-M speech encoder (test infrastructure: imported by
tests/ and bench.py's baseline leg only, never by the product path; numpy,
float64).

Sources:
  * audio.cpp "Fun-ASR-Nano Native Runtime Implementation Plan", Task 3 Step 3
    (the SAN-M block: Q/K/V projection, scaled dot-product attention, a
    depthwise FSMN over V, residual addition, affine LayerNorm, ReLU FFN) and
    Task 4 Step 3 (the encoder: sqrt(512) scaling, sinusoidal positions, one
    560 -> 512 stem, 49 main blocks, a normalisation, 20 timestamp blocks and
    a final normalisation).
  * transcribe.cpp "Forward map - funasr_nano", table "Encoder
    (SenseVoiceEncoderSmall, frozen)": PE added to the [T, 560] input, the
    projection block encoders0 without the attention residual, encoders 0..48
    (residual SAN-M), after_norm (LayerNorm eps 1e-12), tp_encoders 0..19,
    tp_norm (LayerNorm eps 1e-12); no CTC head, the result is tp_norm's output.

Readings where the pages are silent (each listed in the design doc):
  * the scaling multiplies the 560-wide LFR rows by sqrt(512) before the
    positions are added;
  * the positions are the textbook sinusoid over the input width d = 560:
    PE[t, 2i] = sin(t / 10000^(2i/d)), PE[t, 2i+1] = cos(t / 10000^(2i/d)),
    t = 0, 1, ...;
  * a block is pre-norm: h = LN1(x); q, k, v = h Wq^T + bq, h Wk^T + bk,
    h Wv^T + bv; per head softmax(q k^T / sqrt(d_head)) v (every frame sees
    every frame), then the output projection Wo, bo; the FSMN memory is
    v + (depthwise convolution of v over time, one kernel of width K per
    channel, zero padding (K-1)/2 on both sides, no bias); the block output is
    y = attention + memory, added to x in residual blocks and taken alone in
    the stem; then x + W2 relu(W1 LN2(x) + b1) + b2;
  * every LayerNorm has a gain and a bias, the population variance and eps
    1e-12 (the value the page gives for after_norm and tp_norm);
  * head count, FFN width and FSMN kernel width are not given for the real
    encoder: parameters, 4 heads (d_head 128), FFN 2048 and K = 11 in the
    workloads (the page's block probe uses 2 heads, FFN 16, K = 3).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict

import numpy as np

from .adaptor import layer_norm, linear, relu


@dataclass(frozen=True)
class EncoderConfig:
    in_dim: int = 560        # n_mels * lfr_m
    dim: int = 512
    n_head: int = 4
    ffn_dim: int = 2048
    kernel: int = 11         # FSMN width (odd)
    n_main: int = 49         # residual blocks after the stem
    n_tp: int = 20
    ln_eps: float = 1e-12

    def block_names(self):
        """Parameter prefixes in run order: the stem, the main blocks, the tp blocks."""
        return (["encoders0.0."] + [f"encoders.{i}." for i in range(self.n_main)]
                + [f"tp_encoders.{i}." for i in range(self.n_tp)])


def positions(t: int, d: int) -> np.ndarray:
    """[t, d] sinusoid: even columns sin, odd columns cos of pos / 10000^(2i/d)."""
    pos = np.arange(t, dtype=np.float64)[:, None]
    i = np.arange(d // 2, dtype=np.float64)[None, :]
    ang = pos / np.power(10000.0, 2.0 * i / d)
    pe = np.zeros((t, d))
    pe[:, 0::2] = np.sin(ang)
    pe[:, 1::2] = np.cos(ang)
    return pe


def fsmn(v: np.ndarray, w: np.ndarray) -> np.ndarray:
    """v + depthwise conv over time: out[t, c] = v[t, c] + sum_j w[c, j] v[t + j - (K-1)/2, c]."""
    T, _ = v.shape
    K = w.shape[1]
    half = (K - 1) // 2
    vp = np.concatenate([np.zeros((half, v.shape[1])), v, np.zeros((K - 1 - half, v.shape[1]))], axis=0)
    out = v.copy()
    for j in range(K):
        out += w[:, j][None, :] * vp[j: j + T]
    return out


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, n_head: int) -> np.ndarray:
    """Bidirectional scaled dot-product attention per head; [T, d] each."""
    T, d = q.shape
    hd = d // n_head
    o = np.empty((T, d))
    for h in range(n_head):
        sl = slice(h * hd, (h + 1) * hd)
        s = q[:, sl] @ k[:, sl].T / np.sqrt(hd)
        s = s - s.max(axis=1, keepdims=True)
        e = np.exp(s)
        o[:, sl] = (e / e.sum(axis=1, keepdims=True)) @ v[:, sl]
    return o


def sanm_block(x: np.ndarray, p: Dict[str, np.ndarray], pre: str, cfg: EncoderConfig, residual: bool) -> np.ndarray:
    h = layer_norm(x, p[pre + "norm1.g"], p[pre + "norm1.b"], cfg.ln_eps)
    q = linear(h, p[pre + "q.w"], p[pre + "q.b"])
    k = linear(h, p[pre + "k.w"], p[pre + "k.b"])
    v = linear(h, p[pre + "v.w"], p[pre + "v.b"])
    y = linear(attention(q, k, v, cfg.n_head), p[pre + "o.w"], p[pre + "o.b"]) + fsmn(v, p[pre + "fsmn.w"])
    x = x + y if residual else y
    h = layer_norm(x, p[pre + "norm2.g"], p[pre + "norm2.b"], cfg.ln_eps)
    return x + linear(relu(linear(h, p[pre + "ffn1.w"], p[pre + "ffn1.b"])), p[pre + "ffn2.w"], p[pre + "ffn2.b"])


def embed(feats: np.ndarray, cfg: EncoderConfig) -> np.ndarray:
    """LFR rows [T, in_dim] scaled by sqrt(dim) plus positions (gate enc.embed.out)."""
    x = np.asarray(feats, dtype=np.float64)
    return x * np.sqrt(cfg.dim) + positions(x.shape[0], cfg.in_dim)


def encoder(feats: np.ndarray, p: Dict[str, np.ndarray], cfg: EncoderConfig, stages=None) -> np.ndarray:
    """LFR rows [T, in_dim] -> encoder output [T, dim] (tp_norm's output).
    `stages`, a dict, receives the gate tensors of the page's table by name."""
    q = {k: np.asarray(v, dtype=np.float64) for k, v in p.items()}
    x = embed(feats, cfg)
    if stages is not None:
        stages["enc.embed.out"] = x
    names = cfg.block_names()
    for b, pre in enumerate(names):
        x = sanm_block(x, q, pre, cfg, residual=b > 0)
        if stages is not None:
            stages["enc." + pre + "out"] = x
        if b == cfg.n_main:
            x = layer_norm(x, q["after_norm.g"], q["after_norm.b"], cfg.ln_eps)
            if stages is not None:
                stages["enc.after_norm.out"] = x
    x = layer_norm(x, q["tp_norm.g"], q["tp_norm.b"], cfg.ln_eps)
    if stages is not None:
        stages["enc.tp_norm.out"] = x
    return x
