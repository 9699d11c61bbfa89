"""Per-step logits comparison metrics (test infrastructure).

NCNN "Qwen3ASR ncnn多平台移植", section 7.2 lists the per-step measures used to
compare a candidate's full-vocabulary logits with the teacher's: maximum and
mean absolute error, RMSE, mean relative error with denominator max(|t|, 1e-6),
cosine similarity of the whole vector, and argmax agreement. Relative error
alone is unreliable near zero logits, so acceptance uses the others.
"""
from __future__ import annotations

import numpy as np


def step_metrics(candidate, teacher) -> dict:
    c = np.asarray(candidate, dtype=np.float64).ravel()
    t = np.asarray(teacher, dtype=np.float64).ravel()
    d = c - t
    ad = np.abs(d)
    t32 = t.astype(np.float32)
    top2 = np.partition(t32, -2)[-2:] if t32.size >= 2 else np.array([0.0, 0.0])
    denom = np.linalg.norm(c) * np.linalg.norm(t)
    return {
        "max_abs": float(ad.max()) if ad.size else 0.0,
        "mean_abs": float(ad.mean()) if ad.size else 0.0,
        "rmse": float(np.sqrt(np.mean(d * d))) if ad.size else 0.0,
        "mean_rel": float(np.mean(ad / np.maximum(np.abs(t), 1e-6))) if ad.size else 0.0,
        "cosine": float(np.dot(c, t) / denom) if denom > 0 else float("nan"),
        "argmax_equal": bool(np.argmax(c.astype(np.float32)) == np.argmax(t32)),
        "teacher_top2_margin": float(top2[1] - top2[0]) if t32.size >= 2 else float("inf"),
    }
