"""Helpers shared by the GPU tests: run the HIP path through the C ABI on
seeded synthetic inputs and compare with the oracle (NCNN page section 7:
teacher-forced per-step logits, the metrics of section 7.2).

Every per-step comparison is also recorded; at the end of the session the
records are written as JSON to $QDEC_PARITY_REPORT (default
gpu_parity_report.json at the repository root): test label, step, and the
section 7.2 metrics (max abs, mean abs, RMSE, mean relative error, cosine,
argmax agreement) with the oracle's top-2 margin."""
from __future__ import annotations

import json
import os

import numpy as np

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
REPORT = []


def write_report():
    if not REPORT:
        return
    path = os.environ.get("QDEC_PARITY_REPORT", os.path.join(ROOT, "gpu_parity_report.json"))
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        json.dump({"records": REPORT}, f)


def record(label, step, metrics, kind="full"):
    REPORT.append({"label": label, "step": int(step), "kind": kind,
                   **{k: (bool(v) if isinstance(v, (bool, np.bool_)) else float(v)) for k, v in metrics.items()}})


def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU test without a GPU"
    return torch, torch.device("cuda:0")


def device_model(shape, W):
    from qwen3_kv_cache_amd.device import Model
    return Model(shape, W.bits if shape.bf16 else W.f32, bf16=shape.bf16)


_CACHE = {}


def weights_06b():
    """The 0.6B-shape weight set every full-size workload shares (seed 2)."""
    if "W" not in _CACHE:
        _CACHE["W"] = synth.make_weights(synth.QWEN3_0P6B, 2)
    return _CACHE["W"]


def model_06b():
    if "m" not in _CACHE:
        _CACHE["m"] = device_model(synth.QWEN3_0P6B, weights_06b())
    return _CACHE["m"]


def oracle_06b():
    """The float64 oracle on the same 0.6B weights (about 4.8 GB of host memory)."""
    if "o" not in _CACHE:
        _CACHE["o"] = oracle.Qwen3Oracle(oracle.OracleConfig.from_shape(synth.QWEN3_0P6B), weights_06b().f32)
    return _CACHE["o"]


def run_forced(model, ids, audio, a0, forced, max_ctx=None, state=None, keep_state=False):
    """Prefill (ids, audio rows at a0) then decode `forced` tokens one step at
    a time. Returns (logits [1 + n, V] float32, argmax [1 + n] int32)."""
    from qwen3_kv_cache_amd import qdec
    torch, dev = torch_dev()
    V = model.shape.vocab
    n = len(forced)
    T = len(ids)
    st = state or qdec.qdec_state_create(model.handle, max_ctx or (T + n))
    logits = torch.full((n + 1, V), float("nan"), dtype=torch.float32, device=dev)
    amax = torch.full((n + 1,), -1, dtype=torch.int32, device=dev)
    audio_d = torch.from_numpy(np.ascontiguousarray(audio, dtype=np.float32)).to(dev) if audio is not None and len(audio) else None
    qdec.qdec_prefill(st, ids, T, audio_d.data_ptr() if audio_d is not None else None, a0,
                      0 if audio_d is None else len(audio), logits[0].data_ptr(), amax[0].data_ptr())
    for s, tok in enumerate(forced):
        qdec.qdec_decode_step(st, int(tok), T + s, logits[s + 1].data_ptr(), amax[s + 1].data_ptr())
    torch.cuda.synchronize()
    qdec.qdec_model_status(model.handle)
    out = logits.cpu().numpy(), amax.cpu().numpy()
    if keep_state:
        return out + (st,)
    qdec.qdec_state_destroy(st)
    return out


def oracle_forced(orc, ids, audio, a0, forced):
    st = orc.new_state()
    res = [orc.prefill(st, ids, audio, a0)]
    for s, tok in enumerate(forced):
        res.append(orc.decode(st, int(tok), len(ids) + s))
    return np.stack(res)


def check_steps(gpu, amax, ref, fp32: bool, label: str):
    """Per-step acceptance on the full vocabulary vector: fp32 weights max abs
    <= 1e-4; bf16 weights cosine >= 0.9999 and max abs <= 5e-2; argmax equal
    to the oracle's pick (lowest index of the fp32-rounded maximum) on every
    step. Every step's metrics go to the parity report."""
    worst = {"max_abs": 0.0, "cos_min": 1.0}
    for s in range(len(ref)):
        m = oracle.step_metrics(gpu[s], ref[s])
        record(label, s, m)
        worst["max_abs"] = max(worst["max_abs"], m["max_abs"])
        worst["cos_min"] = min(worst["cos_min"], m["cosine"])
        assert np.all(np.isfinite(gpu[s])), f"{label} step {s}: non-finite logits"
        if fp32:
            assert m["max_abs"] <= 1e-4, f"{label} step {s}: max abs {m['max_abs']:.3g}"
        else:
            assert m["cosine"] >= 0.9999, f"{label} step {s}: cosine {m['cosine']:.6f}"
            assert m["max_abs"] <= 5e-2, f"{label} step {s}: max abs {m['max_abs']:.3g}"
        pick = oracle.pick_token(ref[s])
        assert int(amax[s]) == pick, (f"{label} step {s}: argmax {int(amax[s])} != oracle {pick} "
                                      f"(oracle top-2 margin {m['teacher_top2_margin']:.3g}, max abs {m['max_abs']:.3g})")
        # the device argmax agrees with the logits it wrote
        assert int(amax[s]) == int(np.argmax(gpu[s])), f"{label} step {s}: argmax inconsistent with logits"
    return worst


def mid_workload(shape, seed, T, a0, La, n_decode):
    W = synth.make_weights(shape, seed)
    ids = synth.random_ids(seed, T, shape.vocab)
    audio = synth.random_rows(seed, La, shape.hidden)
    forced = synth.random_ids(seed + 100, n_decode, shape.vocab)
    return W, ids, audio, a0, forced
