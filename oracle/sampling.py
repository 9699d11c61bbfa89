"""CPU oracle of the sampling step after the LM head (test infrastructure).

The NCNN page "Qwen3ASR ncnn多平台移植" lists, in section 1, greedy,
temperature, top-k, top-p and repetition-penalty sampling among the runtime's
abilities, and in section 6 keeps greedy as the default with the other four
"for non-deterministic generation experiments". The page gives no formulas or
order, so this oracle takes the common reading (each listed in the design doc):

  1. repetition penalty rho on every distinct token id of the row's history:
     z = z / rho where z > 0, z * rho otherwise;
  2. temperature 0 is greedy: the lowest index of the maximum;
  3. z = z / T;
  4. candidates ordered by (z descending, index ascending); top-k keeps the
     first k;
  5. probabilities over the kept candidates, softmax with the maximum
     subtracted;
  6. top-p keeps the shortest prefix whose probability mass reaches top_p
     (at least one candidate), renormalised;
  7. with a caller-supplied uniform u in [0, 1): the first candidate whose
     cumulative probability exceeds u times the kept mass.

Precision, matching the decisions the device makes: steps 1 and 3 in float32
(one rounded operation per value, so both sides get the same bits); steps 5-7
in float64, with the cumulative sums taken in candidate order.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np


@dataclass(frozen=True)
class SamplingParams:
    temperature: float = 0.0
    top_k: int = 0            # 0: off
    top_p: float = 1.0        # 1: off
    repetition_penalty: float = 1.0  # 1: off


def penalize(logits: np.ndarray, history: Sequence[int], rho: float) -> np.ndarray:
    """Step 1, in float32: each distinct history id once."""
    z = np.array(logits, dtype=np.float32, copy=True)
    if rho == 1.0:
        return z
    r = np.float32(rho)
    for t in sorted(set(int(h) for h in history if 0 <= int(h) < z.size)):
        z[t] = z[t] / r if z[t] > 0 else z[t] * r
    return z


def candidates(z: np.ndarray, top_k: int) -> np.ndarray:
    """Step 4: indices ordered by (value descending, index ascending), the
    first top_k of them (all when top_k is 0). numpy's stable lexsort: the
    last key (-value) is the primary one, the index breaks ties."""
    order = np.lexsort((np.arange(z.size), -z.astype(np.float64)))
    if top_k > 0:
        order = order[:top_k]
    return order.astype(np.int64)


def kept_distribution(logits: np.ndarray, params: SamplingParams, history: Sequence[int] = ()):
    """Steps 1 and 3-6: the kept candidates (in order) and their cumulative
    probability mass in float64 (not yet renormalised)."""
    z = penalize(logits, history, params.repetition_penalty)
    z = z / np.float32(params.temperature)
    cand = candidates(z, params.top_k)
    zc = z[cand].astype(np.float64)
    e = np.exp(zc - zc[0])
    cum = np.zeros(e.size)
    acc = 0.0
    for i in range(e.size):
        acc += e[i]
        cum[i] = acc
    total = cum[-1]
    n = e.size
    if params.top_p < 1.0:
        n = 1
        while n < e.size and cum[n - 1] < params.top_p * total:
            n += 1
    return cand[:n], cum[:n]


def sample(logits: np.ndarray, params: SamplingParams, u: float, history: Sequence[int] = ()) -> int:
    """The sampled token id for one row of logits and one uniform u."""
    if not np.all(np.isfinite(np.asarray(logits, dtype=np.float32))):
        raise FloatingPointError("non-finite logits")
    if params.temperature == 0.0:
        return int(np.argmax(penalize(logits, history, params.repetition_penalty)))
    cand, cum = kept_distribution(logits, params, history)
    target = u * cum[-1]
    for i in range(cand.size):
        if cum[i] > target:
            return int(cand[i])
    return int(cand[-1])


def boundary_margin(logits: np.ndarray, params: SamplingParams, u: float, history: Sequence[int] = ()) -> float:
    """Distance of u * mass to the nearest cumulative boundary, relative to
    the mass: a pick closer than rounding can decide is reported, not
    failed (float64 sums in another order differ by ~1e-16)."""
    if params.temperature == 0.0:
        return 1.0
    _, cum = kept_distribution(logits, params, history)
    target = u * cum[-1]
    return float(np.min(np.abs(cum - target)) / cum[-1])
