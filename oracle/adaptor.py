"""CPU oracle of the audio adaptor (test infrastructure: imported by tests/
and bench.py's baseline leg only, never by the product path; numpy, float64).

The adaptor turns encoder frames [T, 512] into the 1024-wide rows that replace
the audio span of the decoder prompt. Source: transcribe.cpp "Forward map -
funasr_nano", section "Adaptor" (stage table and the list of deviations from
the encoder block):
  * linear1 512 -> 2048 with bias, then ReLU; linear2 2048 -> 1024 with bias;
  * two blocks, each: LayerNorm (gain and bias, eps 1e-12) -> multi-head
    attention with biased Q/K/V/O projections -> residual add; LayerNorm ->
    fc1 1024 -> 256 with bias, ReLU, fc2 256 -> 1024 with bias -> residual;
  * no Q/K norm, no RoPE; the output of the second block is the result (the
    caller keeps its first rows as the audio span).

Readings where the page is silent (each listed in the design doc):
  * pre-norm blocks (the norm feeds the sub-layer, the residual adds the raw
    input), as the order "norm1 -> q/k/v/out -> residual" reads;
  * the attention is bidirectional (every frame sees every frame), scale
    1/sqrt(head_dim), softmax with the row maximum subtracted;
  * the number of heads is not given: a parameter, 8 (head_dim 128) in the
    workloads;
  * LayerNorm uses the biased (population) variance of the row;
  * no final LayerNorm after the second block (the table lists none).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict

import numpy as np


@dataclass(frozen=True)
class AdaptorConfig:
    enc_dim: int = 512
    mid_dim: int = 2048      # linear1 output
    dim: int = 1024          # linear2 output = decoder hidden size
    ffn_dim: int = 256       # block FFN bottleneck (dim // 4)
    n_block: int = 2
    n_head: int = 8
    ln_eps: float = 1e-12


def linear(x: np.ndarray, w: np.ndarray, b: np.ndarray) -> np.ndarray:
    """nn.Linear: x W^T + b, W stored [out, in]."""
    return x @ w.T + b


def relu(x: np.ndarray) -> np.ndarray:
    return np.maximum(x, 0.0)


def layer_norm(x: np.ndarray, g: np.ndarray, b: np.ndarray, eps: float) -> np.ndarray:
    """(x - mean) / sqrt(var + eps) * g + b over the last axis, population variance."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * g + b


def mha(x: np.ndarray, p: Dict[str, np.ndarray], pre: str, n_head: int) -> np.ndarray:
    """Bidirectional multi-head attention with biased projections; x [T, D]."""
    T, D = x.shape
    hd = D // n_head
    q = linear(x, p[pre + "q.w"], p[pre + "q.b"]).reshape(T, n_head, hd)
    k = linear(x, p[pre + "k.w"], p[pre + "k.b"]).reshape(T, n_head, hd)
    v = linear(x, p[pre + "v.w"], p[pre + "v.b"]).reshape(T, n_head, hd)
    o = np.empty((T, n_head, hd), dtype=x.dtype)
    for h in range(n_head):
        s = q[:, h, :] @ k[:, h, :].T / np.sqrt(hd)
        s = s - s.max(axis=1, keepdims=True)
        e = np.exp(s)
        o[:, h, :] = (e / e.sum(axis=1, keepdims=True)) @ v[:, h, :]
    return linear(o.reshape(T, D), p[pre + "o.w"], p[pre + "o.b"])


def block(x: np.ndarray, p: Dict[str, np.ndarray], i: int, cfg: AdaptorConfig) -> np.ndarray:
    pre = f"blocks.{i}."
    x = x + mha(layer_norm(x, p[pre + "norm1.g"], p[pre + "norm1.b"], cfg.ln_eps), p, pre, cfg.n_head)
    h = layer_norm(x, p[pre + "norm2.g"], p[pre + "norm2.b"], cfg.ln_eps)
    return x + linear(relu(linear(h, p[pre + "fc1.w"], p[pre + "fc1.b"])), p[pre + "fc2.w"], p[pre + "fc2.b"])


def adaptor(enc: np.ndarray, p: Dict[str, np.ndarray], cfg: AdaptorConfig, dtype=np.float64) -> np.ndarray:
    """Encoder frames [T, enc_dim] -> adaptor rows [T, dim]."""
    q = {k: np.asarray(v, dtype=dtype) for k, v in p.items()}
    x = np.asarray(enc, dtype=dtype)
    x = relu(linear(x, q["linear1.w"], q["linear1.b"]))
    x = linear(x, q["linear2.w"], q["linear2.b"])
    for i in range(cfg.n_block):
        x = block(x, q, i, cfg)
    return x
