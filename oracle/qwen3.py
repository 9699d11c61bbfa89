"""CPU oracle for the Qwen3-0.6B-shaped KV-cache decoder (test infrastructure).

This is the plain, slow, obviously-correct reference the HIP path is checked
against. Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import it; the product path never does. It shares no
code with the HIP library: numpy only, computing in float64 by default.

Sources (cited by page title and section/table):
  [P1] audio.cpp "Fun-ASR-Nano Native Runtime Implementation Plan", Task 6
       Step 4 (decoder dimensions, RoPE theta 1e6, tied embeddings) and
       Task 6 Step 5 (prefill + decode + KV-cache logit parity).
  [P2] transcribe.cpp "Forward map - funasr_nano", table "LLM decoder"
       (token embed get_rows; audio-row override of inputs_embeds; Qwen3 block
       = rms_norm + GQA 16/8 + per-head Q/K-RMSNorm + NeoX RoPE + SwiGLU with
       packed gate_up; final rms_norm * w; tied lm_head on the last position)
       and table "Generation / KV Path" (prefill writes KV for [0, T); one
       single-token step per position n_past >= T).
  [P3] NCNN "Qwen3ASR ncnn多平台移植", section 4 (audio rows replace the
       audio-pad rows; length/position/modality order unchanged) and section 5
       (prefill with upper-triangular causal mask; per-step: embed, RoPE at the
       absolute position, one-row mask over history, append current K/V, full
       vocabulary logits, greedy pick; the context is cloned, not mutated).

Readings where the pages are silent (each listed in the design doc):
  * RMSNorm: x / sqrt(mean(x^2) + eps) * g, eps = 1e-6 (pages give only
    "rms_norm * w").
  * Q/K norm: one gain vector of length head_dim per layer for Q and one for
    K, shared by all heads, applied per head before RoPE.
  * RoPE: NeoX rotate-half pairs (j, j + D/2), frequency theta^(-2j/D),
    angle pos * freq evaluated in float64; the cache keeps rotated K, raw V.
  * Attention: scale 1/sqrt(D), no bias, window or soft-cap; query head h
    reads KV head h // (n_q / n_kv).
  * No biases in the decoder linears; SwiGLU = down(silu(gate x) * up x).
  * Token decision: argmax of the logits rounded to float32, lowest index on
    ties (the precision the GPU path decides in).
"""
from __future__ import annotations

import copy
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

import numpy as np


@dataclass(frozen=True)
class OracleConfig:
    hidden: int
    n_layer: int
    n_q_head: int
    n_kv_head: int
    head_dim: int
    ffn: int
    vocab: int
    rms_eps: float = 1e-6
    rope_theta: float = 1e6

    @staticmethod
    def from_shape(s) -> "OracleConfig":
        return OracleConfig(s.hidden, s.n_layer, s.n_q_head, s.n_kv_head, s.head_dim,
                            s.ffn, s.vocab, s.rms_eps, s.rope_theta)


# ---------------------------------------------------------------- primitives

def rms_norm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """[P2] LLM decoder table: "rms_norm * w". Normalises over the last axis:
    x_i / sqrt(mean_j x_j^2 + eps) * g_i."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def rope_angles(pos: np.ndarray, head_dim: int, theta: float) -> np.ndarray:
    """[P1] Task 6 Step 4 (theta 1e6), [P2] "NeoX RoPE @ 1e6": angle[p, j] =
    p * theta^(-2j/D) for j < D/2, in float64."""
    j = np.arange(head_dim // 2, dtype=np.float64)
    freq = np.power(np.float64(theta), -2.0 * j / head_dim)
    return np.asarray(pos, dtype=np.float64)[:, None] * freq[None, :]


def apply_rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """NeoX rotate-half: for j < D/2 the pair (x_j, x_{j+D/2}) is rotated by
    angle[p, j]. x: [T, heads, D]; pos: [T] absolute positions ([P3] section 5
    step 2: RoPE at the current absolute position)."""
    D = x.shape[-1]
    half = D // 2
    ang = rope_angles(pos, D, theta)
    c = np.cos(ang).astype(x.dtype)[:, None, :]
    s = np.sin(ang).astype(x.dtype)[:, None, :]
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def silu(z: np.ndarray) -> np.ndarray:
    """SwiGLU activation of the gate branch: z / (1 + exp(-z))."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Max-subtracted softmax over the last axis; -inf entries get weight 0."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_pos: np.ndarray,
              n_kv_valid: int, block: int = 512) -> np.ndarray:
    """Causal GQA attention ([P3] section 5: upper-triangular mask in prefill,
    one-row mask over the history in decode).

    q: [T, n_q, D] at absolute positions q_pos; k, v: [n_kv, >=n_kv_valid, D]
    cache rows 0..n_kv_valid-1 (position u is row u). Query at position p
    sees keys u <= p. Query rows are processed in blocks so a long prompt's
    score matrix is never held whole."""
    T, n_q, D = q.shape
    n_kv = k.shape[0]
    group = n_q // n_kv
    scale = 1.0 / np.sqrt(np.float64(D))
    out = np.empty_like(q)
    u = np.arange(n_kv_valid)
    for h in range(n_q):
        g = h // group
        kh = k[g, :n_kv_valid]
        vh = v[g, :n_kv_valid]
        for t0 in range(0, T, block):
            t1 = min(T, t0 + block)
            s = (q[t0:t1, h, :] @ kh.T) * scale
            s = np.where(u[None, :] <= q_pos[t0:t1, None], s, -np.inf)
            out[t0:t1, h, :] = softmax_rows(s) @ vh
    return out


# --------------------------------------------------------------------- state

class OracleState:
    """KV cache of one sequence: rotated K and raw V per layer, row u holding
    position u ([P2] "Generation / KV Path"; [P3] section 5 context)."""

    def __init__(self, cfg: OracleConfig, dtype, capacity: int = 64):
        self.cfg = cfg
        self.n_past = 0
        self.k = [np.zeros((cfg.n_kv_head, capacity, cfg.head_dim), dtype) for _ in range(cfg.n_layer)]
        self.v = [np.zeros((cfg.n_kv_head, capacity, cfg.head_dim), dtype) for _ in range(cfg.n_layer)]

    def _reserve(self, n: int) -> None:
        cap = self.k[0].shape[1]
        if n <= cap:
            return
        new = max(n, 2 * cap)
        for lst in (self.k, self.v):
            for i, a in enumerate(lst):
                b = np.zeros((a.shape[0], new, a.shape[2]), a.dtype)
                b[:, :cap] = a
                lst[i] = b

    def append(self, layer: int, k_new: np.ndarray, v_new: np.ndarray, pos0: int) -> None:
        """Write K/V rows for positions pos0..pos0+T-1 (k_new: [T, n_kv, D])."""
        T = k_new.shape[0]
        self._reserve(pos0 + T)
        self.k[layer][:, pos0:pos0 + T] = np.transpose(k_new, (1, 0, 2))
        self.v[layer][:, pos0:pos0 + T] = np.transpose(v_new, (1, 0, 2))

    def clone(self) -> "OracleState":
        """[P3] section 5: generation works on a clone of the context."""
        return copy.deepcopy(self)


# --------------------------------------------------------------------- model

class Qwen3Oracle:
    """Qwen3 causal decoder with a KV cache ([P1] Task 6 Step 4, [P2] LLM
    decoder table). Parameters: dict with "embed" [V,H], "final_norm" [H] and
    per layer "L{i}.{in_norm,wq,wk,wv,q_norm,k_norm,wo,post_norm,w_gate,w_up,
    w_down}" with linear weights stored [out, in]."""

    def __init__(self, cfg: OracleConfig, params: Dict[str, np.ndarray], dtype=np.float64):
        self.cfg = cfg
        self.dtype = np.dtype(dtype)
        self.p = {k: np.asarray(v).astype(self.dtype) for k, v in params.items()}
        c = cfg
        assert self.p["embed"].shape == (c.vocab, c.hidden)
        assert self.p["L0.wq"].shape == (c.n_q_head * c.head_dim, c.hidden)

    def new_state(self) -> OracleState:
        return OracleState(self.cfg, self.dtype)

    # [P2] "Token embed" + "Audio-row override"; [P3] section 4.
    def embed(self, ids: np.ndarray, audio: Optional[np.ndarray], audio_begin: int) -> np.ndarray:
        """X[t] = E[ids[t]]; rows [a0, a0+La) are replaced by the audio rows
        (replace, not add; the ids under the span are not used)."""
        ids = np.asarray(ids, dtype=np.int64)
        T = len(ids)
        x = np.empty((T, self.cfg.hidden), self.dtype)
        n_audio = 0 if audio is None else len(audio)
        from_table = np.ones(T, bool)
        from_table[audio_begin:audio_begin + n_audio] = False
        x[from_table] = self.p["embed"][ids[from_table]]
        if n_audio:
            x[audio_begin:audio_begin + n_audio] = np.asarray(audio, dtype=self.dtype)
        return x

    def qkv(self, i: int, x: np.ndarray, pos: np.ndarray):
        """Row-wise first half of a Qwen3 block ([P2]: rms_norm, Q/K/V
        projections, per-head Q/K-RMSNorm, NeoX RoPE at each row's absolute
        position). Returns q [T,n_q,D], k, v [T,n_kv,D]."""
        c, p = self.cfg, self.p
        T, D = x.shape[0], c.head_dim
        xn = rms_norm(x, p[f"L{i}.in_norm"], c.rms_eps)
        q = (xn @ p[f"L{i}.wq"].T).reshape(T, c.n_q_head, D)
        k = (xn @ p[f"L{i}.wk"].T).reshape(T, c.n_kv_head, D)
        v = (xn @ p[f"L{i}.wv"].T).reshape(T, c.n_kv_head, D)
        q = rms_norm(q, p[f"L{i}.q_norm"], c.rms_eps)
        k = rms_norm(k, p[f"L{i}.k_norm"], c.rms_eps)
        return apply_rope(q, pos, c.rope_theta), apply_rope(k, pos, c.rope_theta), v

    def out_mlp(self, i: int, x: np.ndarray, o: np.ndarray) -> np.ndarray:
        """Row-wise second half: X += O Wo^T; X += down(silu(gate Xn) * up Xn)
        with Xn = rms_norm(X; post_norm) ([P2] "SwiGLU (packed gate_up)")."""
        c, p = self.cfg, self.p
        x = x + o.reshape(x.shape[0], c.n_q_head * c.head_dim) @ p[f"L{i}.wo"].T
        xn = rms_norm(x, p[f"L{i}.post_norm"], c.rms_eps)
        z = silu(xn @ p[f"L{i}.w_gate"].T) * (xn @ p[f"L{i}.w_up"].T)
        return x + z @ p[f"L{i}.w_down"].T

    def block(self, i: int, x: np.ndarray, state: OracleState, pos0: int) -> np.ndarray:
        """One Qwen3 block over rows at positions pos0..pos0+T-1. This layer's
        K/V are appended to the cache before attending ([P3] section 5 step 4)."""
        pos = np.arange(pos0, pos0 + x.shape[0])
        q, k, v = self.qkv(i, x, pos)
        state.append(i, k, v, pos0)
        o = attention(q, state.k[i], state.v[i], pos, pos0 + x.shape[0])
        return self.out_mlp(i, x, o)

    def head(self, x_last: np.ndarray) -> np.ndarray:
        """[P2] "Final RMSNorm" + "Tied lm_head": logits = E . rms_norm(x)."""
        xn = rms_norm(x_last, self.p["final_norm"], self.cfg.rms_eps)
        return xn @ self.p["embed"].T

    def forward(self, state: OracleState, x: np.ndarray, pos0: int) -> np.ndarray:
        for i in range(self.cfg.n_layer):
            x = self.block(i, x, state, pos0)
        state.n_past = pos0 + x.shape[0]
        return x

    # [P3] section 5: prefill over the whole prompt, last-position logits.
    def prefill(self, state: OracleState, ids: np.ndarray, audio: Optional[np.ndarray] = None,
                audio_begin: int = 0) -> np.ndarray:
        if state.n_past != 0:
            raise ValueError("prefill needs an empty state")
        x = self.embed(ids, audio, audio_begin)
        x = self.forward(state, x, 0)
        return self.head(x[-1])

    # [P3] section 5 steps 1-5; [P2] single-step decode at n_past.
    def decode(self, state: OracleState, token: int, pos: int) -> np.ndarray:
        if pos != state.n_past:
            raise ValueError("decode position must equal n_past")
        x = self.embed(np.array([token]), None, 0)
        x = self.forward(state, x, pos)
        return self.head(x[0])

    def decode_many(self, states: Sequence[OracleState], tokens: Sequence[int]) -> np.ndarray:
        """Independent single-token steps for several sequences, each at its own
        n_past. The row-wise parts run on the stacked rows; attention runs per
        sequence over its own cache, so each row equals a separate decode()."""
        B = len(states)
        pos = np.array([s.n_past for s in states])
        x = self.embed(np.asarray(tokens), None, 0)
        for i in range(self.cfg.n_layer):
            q, k, v = self.qkv(i, x, pos)
            o = np.empty_like(q)
            for b, st in enumerate(states):
                st.append(i, k[b:b + 1], v[b:b + 1], int(pos[b]))
                o[b:b + 1] = attention(q[b:b + 1], st.k[i], st.v[i], pos[b:b + 1], int(pos[b]) + 1)
            x = self.out_mlp(i, x, o)
        for b, st in enumerate(states):
            st.n_past = int(pos[b]) + 1
        return self.head(x)


def pick_token(logits: np.ndarray) -> int:
    """Greedy pick ([P3] section 5 step 6, temperature 0 default): argmax of
    the logits rounded to float32, lowest index on ties."""
    l32 = np.asarray(logits, dtype=np.float32)
    if not np.all(np.isfinite(l32)):
        raise FloatingPointError("non-finite logits")
    return int(np.argmax(l32))


def greedy_trajectory(model: Qwen3Oracle, ids, audio, audio_begin: int, n_decode: int):
    """Teacher trajectory ([P3] section 7.1): prefill, then n_decode greedy
    steps. Returns (tokens int32[n_decode + 1], logits [n_decode + 1, V]):
    logits[0] is the prefill logit, tokens[i] = pick_token(logits[i]), and
    logits[s] for s >= 1 comes from the step that consumed tokens[s-1] at
    position len(ids) + s - 1."""
    st = model.new_state()
    out = [model.prefill(st, ids, audio, audio_begin)]
    toks = [pick_token(out[0])]
    T = len(ids)
    for s in range(n_decode):
        out.append(model.decode(st, toks[-1], T + s))
        toks.append(pick_token(out[-1]))
    return np.array(toks, dtype=np.int32), np.stack(out)
