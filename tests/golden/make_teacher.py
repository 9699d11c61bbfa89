"""Write the oracle's teacher data for the full-size 0.6B workloads.

Calls only oracle/ (float64) and the seeded input generators in synth/. The
GPU parity tests compare the HIP path against these stored values because the
float64 oracle needs minutes per workload at full size. Stored per logits
vector (step 0 = prefill, step s = the step that consumed token s-1):
  * the oracle's greedy token (teacher trajectory; branch workloads are forced
    on their seeded streams instead),
  * values at a fixed seeded sample of vocabulary indices plus the oracle's
    top-k indices and values,
  * top-1/top-2 margin (float32 domain) and the full-vector L2 norm,
  * the full float32 logits at several steps spread over the run (greedy
    workloads: 9 steps from the prefill logit to the last step; branch
    workloads: the prefill and branch 0's last step).

Usage: python tests/golden/make_teacher.py prefill8k ragged3k branch16
"""
import argparse
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import synth  # noqa: E402

SAMPLE_SEED = 20261202


def summarize(logits: np.ndarray, sample_idx: np.ndarray, k: int):
    l32 = logits.astype(np.float32)
    top = np.argsort(-l32, kind="stable")[:k]
    srt = np.sort(l32)
    return {
        "sample": l32[sample_idx],
        "top_idx": top.astype(np.int32),
        "top_val": l32[top],
        "margin": float(srt[-1]) - float(srt[-2]),
        "norm": float(np.linalg.norm(logits)),
        "token": oracle.pick_token(logits),
    }


def run_greedy(w, model, n_sample=8192, k=32, n_full=9):
    ids, audio, a0 = synth.make_prompt(w)
    if n_sample >= w.shape.vocab:  # small vocabularies: every entry
        sample_idx = np.arange(w.shape.vocab)
    else:
        sample_idx = np.sort(np.random.default_rng(SAMPLE_SEED).choice(w.shape.vocab, n_sample, replace=False))
    full_steps = np.unique(np.round(np.linspace(0, w.n_decode, n_full)).astype(np.int32))
    full = []
    st = model.new_state()
    t0 = time.perf_counter()
    lg = model.prefill(st, ids, audio, a0)
    t_prefill = time.perf_counter() - t0
    rows = [summarize(lg, sample_idx, k)]
    full.append(lg.astype(np.float32))
    full_first = lg.astype(np.float32)
    t0 = time.perf_counter()
    for s in range(w.n_decode):
        lg = model.decode(st, rows[-1]["token"], w.prompt_len + s)
        rows.append(summarize(lg, sample_idx, k))
        if s + 1 in full_steps:
            full.append(lg.astype(np.float32))
        print(f"  step {s + 1}/{w.n_decode} token {rows[-1]['token']} margin {rows[-1]['margin']:.4g}", flush=True)
    t_decode = time.perf_counter() - t0
    return dict(
        tokens=np.array([r["token"] for r in rows], np.int32),
        sample_idx=sample_idx.astype(np.int32),
        sample_vals=np.stack([r["sample"] for r in rows]),
        top_idx=np.stack([r["top_idx"] for r in rows]),
        top_vals=np.stack([r["top_val"] for r in rows]),
        margin=np.array([r["margin"] for r in rows]),
        norm=np.array([r["norm"] for r in rows]),
        full_first=full_first,
        full_last=lg.astype(np.float32),
        full_steps=full_steps,
        full_vals=np.stack(full),
        oracle_prefill_s=np.float64(t_prefill),
        oracle_decode_s=np.float64(t_decode),
    )


def run_branches(w, model, n_sample=256, k=16):
    ids, audio, a0 = synth.make_prompt(w)
    sample_idx = np.sort(np.random.default_rng(SAMPLE_SEED).choice(w.shape.vocab, n_sample, replace=False))
    base = model.new_state()
    t0 = time.perf_counter()
    lg0 = model.prefill(base, ids, audio, a0)
    t_prefill = time.perf_counter() - t0
    states = [base.clone() for _ in range(w.n_branch)]
    streams = np.stack([synth.branch_stream(w, b) for b in range(w.n_branch)])
    per = []
    t0 = time.perf_counter()
    for s in range(w.n_decode):
        lgs = model.decode_many(states, streams[:, s])
        per.append([summarize(lgs[b], sample_idx, k) for b in range(w.n_branch)])
        print(f"  step {s + 1}/{w.n_decode}", flush=True)
    t_decode = time.perf_counter() - t0
    first = summarize(lg0, sample_idx, k)

    def col(key):
        return np.stack([np.stack([per[s][b][key] for s in range(w.n_decode)]) for b in range(w.n_branch)])
    return dict(
        streams=streams.astype(np.int32),
        sample_idx=sample_idx.astype(np.int32),
        prefill_sample=first["sample"], prefill_top_idx=first["top_idx"], prefill_top_val=first["top_val"],
        prefill_margin=np.float64(first["margin"]), prefill_token=np.int32(first["token"]),
        full_first=lg0.astype(np.float32),
        tokens=col("token").astype(np.int32),
        sample_vals=col("sample"), top_idx=col("top_idx"), top_vals=col("top_val"),
        margin=col("margin"), norm=col("norm"),
        full_last_b0=lgs[0].astype(np.float32),
        oracle_prefill_s=np.float64(t_prefill),
        oracle_decode_s=np.float64(t_decode),
    )


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("workloads", nargs="+")
    ap.add_argument("--out", default=HERE)
    a = ap.parse_args()
    for name in a.workloads:
        w = synth.WORKLOADS[name]
        print(f"[teacher] {name}: generating weights", flush=True)
        W = synth.make_weights(w.shape, w.weight_seed)
        model = oracle.Qwen3Oracle(oracle.OracleConfig.from_shape(w.shape), W.f32, dtype=np.float64)
        print(f"[teacher] {name}: running oracle", flush=True)
        res = run_branches(w, model) if w.n_branch > 1 else run_greedy(w, model)
        path = os.path.join(a.out, f"teacher_{name}.npz")
        np.savez_compressed(path, **res)
        print(f"[teacher] wrote {path} ({os.path.getsize(path) / 1e6:.1f} MB)", flush=True)
        del model


if __name__ == "__main__":
    main()
