"""Block-int8 weights (Q8_0) for the quantized-decode oracle (test
infrastructure: imported by tests/ only; numpy).

The audio.cpp page "Fun-ASR-Nano Native Runtime Implementation Plan", Task 8,
names Q8_0 as one of the packaged weight types (the default package) and asks
for the same greedy transcript as the F16 weights; it does not define the
format. Reading (listed in the design doc), the common block format:
  * a row of an [out, in] matrix is cut into blocks of 32 consecutive inputs;
  * per block, d = max|w| / 127 in float32, stored rounded to float16;
  * q = w / d: one IEEE float32 division by that float32 d (not a product
    with a rounded reciprocal), then rounded half away from zero, evaluated
    exactly (float64), |q| <= 127 (q = 0 and d = 0 for an all-zero block);
  * the decoder uses w' = q * float32(fp16 d), exact in float32 (8-bit by
    11-bit significands), so a quantized model is the float oracle fed w'.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32


def quantize(w: np.ndarray):
    """w float32 [out, in] (in % 32 == 0) -> (q int8 [out, in], d float16 [out, in / 32])."""
    w = np.asarray(w, dtype=np.float32)
    out, n = w.shape
    if n % BLOCK:
        raise ValueError("input width must be a multiple of 32")
    blocks = w.reshape(out, n // BLOCK, BLOCK)
    amax = np.abs(blocks).max(axis=2)
    d = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(d > 0, d, np.float32(1.0)).astype(np.float32)
    x = (blocks / safe[:, :, None]).astype(np.float32)  # float32 division, one rounding
    x = np.where(d[:, :, None] > 0, x, np.float32(0.0)).astype(np.float64)
    q = np.sign(x) * np.floor(np.abs(x) + 0.5)  # half away from zero, exact for float32 x
    q = np.clip(q, -127, 127).astype(np.int8)
    return q.reshape(out, n), d.astype(np.float16)


def dequantize(q: np.ndarray, d: np.ndarray) -> np.ndarray:
    """(q, d) -> float32 [out, in], q * d exactly."""
    out, n = q.shape
    scale = np.asarray(d, dtype=np.float16).astype(np.float32)
    return (q.reshape(out, n // BLOCK, BLOCK).astype(np.float32) * scale[:, :, None]).reshape(out, n)
