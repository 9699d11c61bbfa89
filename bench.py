"""Benchmark: decode tok/s (B=1) and prefill tok/s of the Qwen3-0.6B-shaped
KV-cache decoder on one MI355X, with a roofline figure and the CPU oracle
timed on the host as a reported baseline.

One step = one pass of the whole path over one synthetic request of the
default workload: prefill a 48-token prompt whose rows 8..30 are audio
embedding rows, then 64 greedy decode steps, each feeding the previous
step's device argmax (no host round trip). The 64 steps run as one
multi-step launch (qdec_decode_greedy); --per-step launches once per token.
Inputs and weights are resident in HBM before timing; states are created
before the timed region.

The default run also reports, under "other_workloads", the rest of the
metric with the same weights and fewer repetitions: B=16 batched decode of
16 clones of a 512-token prefill (branch16), the 1024- and 8192-token
prompts (long, prefill8k), and the default workload on Q8_0 weights of the
same shape (short_q8_0); under "sampling" the time of one sampling step
(qdec_sample) over 1 and 16 rows of logits; under "adaptor" the audio
adaptor that makes the audio rows (qdec_adaptor_run) at 183 and 6000 encoder
frames; and under "encoder" the frontend + SAN-M encoder (qdec_encoder_run)
on 11 s and 60 s of 16 kHz audio. --no-others skips them.

Usage: python bench.py [--steps K] [--warmup W] [--workload short|long|prefill8k|branch16]
       python bench.py --copy-probe   (plain copy kernel for counter calibration)
       python bench.py --adaptor-only (the audio adaptor alone)
       python bench.py --encoder-only (the frontend + encoder alone)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
METRIC = "decode tok/s (B=1,B=16) + prefill tok/s, Qwen3-0.6B bf16; % HBM peak"


def decode_bytes(shape, ctx_lens) -> float:
    """Algorithmic HBM bytes of one decode token at each attended length p:
    every bf16 weight once (layers + tied head), the fp32 K and V of p
    positions, the new K/V row, and the embedding row."""
    H, L, D = shape.hidden, shape.n_layer, shape.head_dim
    layer_w = (shape.n_q_head * D * H + 2 * shape.n_kv_head * D * H + H * shape.n_q_head * D + 3 * shape.ffn * H) * 2
    norms = (2 * H + 2 * D) * 2
    head = shape.vocab * H * 2
    kv_row = 2 * shape.n_kv_head * D * 4
    w = L * (layer_w + norms) + head + H * 2
    return float(np.mean([w + L * kv_row * p + L * kv_row for p in ctx_lens]))


def decode_bytes_q8(shape, ctx_lens) -> float:
    """The same byte model for Q8_0 weights: every matrix weight (layers and
    the tied head) at 34/32 bytes, its int8 code and its share of the block's
    fp16 scale; fp32 norm gains; the embedding row as Q8_0 blocks."""
    H, L, D = shape.hidden, shape.n_layer, shape.head_dim
    q8 = 34.0 / 32.0
    layer_w = (shape.n_q_head * D * H + 2 * shape.n_kv_head * D * H + H * shape.n_q_head * D + 3 * shape.ffn * H) * q8
    norms = (2 * H + 2 * D) * 4
    head = shape.vocab * H * q8
    kv_row = 2 * shape.n_kv_head * D * 4
    w = L * (layer_w + norms) + head + H * q8
    return float(np.mean([w + L * kv_row * p + L * kv_row for p in ctx_lens]))


def batch_decode_bytes(shape, prefix: int, B: int, s: int):
    """Algorithmic HBM bytes of batched decode step s (0-based) of B branches
    cloned from a prefix of `prefix` positions: (unique, per sequence).
    Unique: every weight once, the shared prefix K/V once, each branch's own
    s + 1 positions, the B new K/V rows and embedding rows. Per sequence:
    each branch reading the whole history, as B separate decodes would."""
    H, L = shape.hidden, shape.n_layer
    kv_row = 2 * shape.n_kv_head * shape.head_dim * 4
    w = decode_bytes(shape, [0]) - L * kv_row - H * 2  # weights, norms and head only
    unique = w + L * kv_row * (prefix + B * (s + 1)) + B * L * kv_row + B * H * 2
    per_seq = w + B * L * kv_row * (prefix + s + 1) + B * L * kv_row + B * H * 2
    return float(unique), float(per_seq)


def decode_roofline(shape, wl, dec_ms_mean: float):
    """Achieved GB/s of a workload's decode from the byte model above."""
    n, B = wl.n_decode, wl.n_branch
    t_step = dec_ms_mean / 1e3 / n
    if B == 1:
        b = decode_bytes(shape, [wl.prompt_len + s + 1 for s in range(n)])
        return {"bytes_per_step": round(b), "achieved": round(b / t_step / 1e9, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(b / t_step / 1e9 / HBM_PEAK_GBS, 4)}
    u = np.mean([batch_decode_bytes(shape, wl.prompt_len, B, s)[0] for s in range(n)])
    q = np.mean([batch_decode_bytes(shape, wl.prompt_len, B, s)[1] for s in range(n)])
    return {"bytes_per_step_unique": round(u), "bytes_per_step_per_sequence": round(q),
            "achieved_unique": round(u / t_step / 1e9, 1), "achieved_per_sequence": round(q / t_step / 1e9, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac_unique": round(u / t_step / 1e9 / HBM_PEAK_GBS, 4)}


def prefill_flops(shape, T: int) -> float:
    """Useful FLOPs of a T-token prefill, each counted once: 2 per weight per
    row for the layer projections, 4 D per (query head, attended key) pair for
    QK and PV with causal masking, and the LM head on the last row."""
    H, L, D, NQ, NKV, F = shape.hidden, shape.n_layer, shape.head_dim, shape.n_q_head, shape.n_kv_head, shape.ffn
    layer_w = H * (NQ + 2 * NKV) * D + NQ * D * H + 3 * F * H
    return 2.0 * L * layer_w * T + L * 4.0 * NQ * D * T * (T + 1) / 2 + 2.0 * shape.vocab * H


def read_profile_values(name: str, source: str):
    """The key: value lines of a committed profile summary, or None when the
    named source file has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", name)
    src = os.path.join(ROOT, "qwen3_kv_cache_amd", "csrc", source)
    try:
        kv = {}
        for line in open(path):
            if ":" in line and not line.startswith((" ", "#")):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
        if kv.get("source_sha256") != hashlib.sha256(open(src, "rb").read()).hexdigest():
            return None
        return kv
    except OSError:
        return None


def prefill_mfma(shape, T: int, ms: float, workload: str):
    """MFMA roofline of the prefill: useful FLOP/s against the dense bf16
    peak, with the counter-measured MFMA busy share of the prefill kernels
    when a matching summary is committed (taken at T = 8192)."""
    f = prefill_flops(shape, T)
    tf = f / (ms / 1e3) / 1e12
    out = {"bound": "mfma", "useful_flops": f, "achieved": round(tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
           "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "counters": None}
    kv = read_profile_values("prefill_mfma_counters_8k.txt", "qdec_kernels.hip") if workload == "prefill8k" else None
    if kv is not None:
        try:
            out["counters"] = {"mfma_busy_pct_prefill_kernels": float(kv["mfma_busy_pct_prefill_kernels"]),
                               "mfma_flops_issued_per_prefill": float(kv["mfma_flops_issued_per_prefill"])}
        except (KeyError, ValueError):
            pass
    return out


def adaptor_flops(a, T: int) -> float:
    """Useful FLOPs of the audio adaptor over T frames: 2 per weight per frame
    for every linear, and 4 dim per (frame, frame) pair per block for QK and PV."""
    lin = a.enc_dim * a.mid_dim + a.mid_dim * a.dim
    blk = 4 * a.dim * a.dim + 2 * a.dim * a.ffn_dim
    return 2.0 * T * lin + a.n_block * (2.0 * T * blk + 4.0 * T * T * a.dim)


def measure_adaptor(frames=(183, 6000), reps=5):
    """Time qdec_adaptor_run (seeded bf16 weights of the 512/2048/1024/256
    adaptor, 2 blocks, 8 heads) on N(0,1) frames, inputs resident on the GPU."""
    import torch

    import synth
    from qwen3_kv_cache_amd.device import Adaptor
    shape = synth.AdaptorShape()
    _, bits = synth.make_adaptor_weights(shape, 1)
    a = Adaptor(shape, bits)
    out = {}
    try:
        for T in frames:
            x = torch.from_numpy(synth.encoder_frames(1, T, shape.enc_dim)).cuda()
            y = torch.empty((T, shape.dim), dtype=torch.float32, device="cuda")
            a.run(x, y)
            torch.cuda.synchronize()
            st = torch.cuda.current_stream()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            for _ in range(reps):
                a.run(x, y)
            e1.record(st)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            tf = adaptor_flops(shape, T) / (ms / 1e3) / 1e12
            out[f"T{T}"] = {"ms": round(ms, 4), "frames_per_s": round(T / (ms / 1e3), 1),
                            "useful_tflops": round(tf, 1), "frac_bf16_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
    finally:
        a.close()
    return out


def encoder_flops(e, T: int) -> float:
    """Useful FLOPs of the SAN-M encoder over T LFR rows: 2 per weight per row
    for every projection (the stem's q/k/v take 560 inputs), 4 dim per (row,
    row) pair per block for QK and PV, 2 K dim per row per block for the FSMN."""
    D, F, nb = e.dim, e.ffn_dim, 1 + e.n_main + e.n_tp
    per_block = 3 * D * D + D * D + 2 * D * F
    lin = nb * per_block + 3 * D * (e.in_dim - D)
    return 2.0 * T * lin + nb * (4.0 * T * T * D + 2.0 * e.kernel * T * D)


def measure_encoder(seconds=(11.0, 60.0), reps=3):
    """Time qdec_encoder_run (frontend + 70 SAN-M blocks, seeded bf16 weights
    of the 512-wide encoder) on speech-like 16 kHz PCM resident on the GPU,
    and the frontend alone (qdec_frontend_run); 11 s of audio is the 183
    LFR rows the adaptor receives in the pages' example."""
    import torch

    import synth
    from qwen3_kv_cache_amd.device import Encoder
    shape = synth.EncoderShape()
    _, bits = synth.make_encoder_weights(shape, 1)
    enc = Encoder(shape, bits)
    out = {}
    try:
        for sec in seconds:
            n = int(sec * 16000)
            x = torch.from_numpy(synth.pcm("voiced", n, 1)).cuda()
            T = enc.rows(n)
            y = torch.empty((T, shape.dim), dtype=torch.float32, device="cuda")
            lfr = enc.frontend(x)
            enc.run(x, y)
            torch.cuda.synchronize()
            st = torch.cuda.current_stream()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            ev[0].record(st)
            for _ in range(reps):
                enc.run(x, y)
            ev[1].record(st)
            for _ in range(reps):
                enc.frontend(x)
            ev[2].record(st)
            torch.cuda.synchronize()
            ms = ev[0].elapsed_time(ev[1]) / reps
            fe_ms = ev[1].elapsed_time(ev[2]) / reps
            tf = encoder_flops(shape, T) / (ms / 1e3) / 1e12
            out[f"{sec:g}s"] = {"rows": T, "ms": round(ms, 3), "frontend_ms": round(fe_ms, 4),
                                "audio_s_per_s": round(sec / (ms / 1e3), 1), "useful_tflops": round(tf, 1),
                                "frac_bf16_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
            del lfr
    finally:
        enc.close()
    return out


def counter_traffic():
    """HBM bytes per decode launch from the committed rocprofv3 counter summary,
    or None when the decode kernel's source has changed since it was taken."""
    kv = read_profile_values("decode_kernel_short_traffic.txt", "qdec_decode.hip")
    try:
        return int(float(kv["hbm_bytes_per_launch"])) if kv is not None else None
    except (KeyError, ValueError):
        return None


def copy_probe():
    import torch
    n = 1 << 28  # 1 GiB of fp32
    a = torch.empty(n, dtype=torch.float32, device="cuda:0").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4, "launches": 5}))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, W, n_decode_sample: int):
    """The oracle in float32 (the plain fp32 CPU reference of the decoder) on
    the host: prefill of the same prompt and a bounded number of greedy decode
    steps, with the BLAS thread pool set to the cores this process may run on.
    Returns decode tok/s, with prefill tok/s and the host described in
    `sample`."""
    import oracle
    import synth
    cores = len(os.sched_getaffinity(0))
    limit = None
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        limit = threadpool_limits(limits=cores, user_api="blas")
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [cores])
    except Exception:
        threads = cores
    try:
        orc = oracle.Qwen3Oracle(oracle.OracleConfig.from_shape(w.shape), W.f32, dtype=np.float32)
        ids, audio, a0 = synth.make_prompt(w)
        st = orc.new_state()
        t0 = time.perf_counter()
        lg = orc.prefill(st, ids, audio, a0)
        t_pre = time.perf_counter() - t0
        tok = oracle.pick_token(lg)
        t0 = time.perf_counter()
        for s in range(n_decode_sample):
            lg = orc.decode(st, tok, w.prompt_len + s)
            tok = oracle.pick_token(lg)
        t_dec = time.perf_counter() - t0
    finally:
        if limit is not None:
            limit.restore_original_limits()
    return {"value": round(n_decode_sample / t_dec, 2), "unit": "decode tok/s", "cores": int(threads), "kind": "oracle",
            "dtype": "f32", "prefill_tok_s": round(w.prompt_len / t_pre, 1),
            "host": {"cpu_model": cpu_model(), "affinity_cores": cores, "blas_threads": int(threads),
                     "OPENBLAS_NUM_THREADS": os.environ.get("OPENBLAS_NUM_THREADS")},
            "sample": f"float32 numpy oracle: prefill of the {w.prompt_len}-token prompt "
                      f"({w.prompt_len / t_pre:.1f} prefill tok/s) then {n_decode_sample} greedy decode steps, B=1"}


def measure(w, model, steps, warmup, per_step=False):
    """Prefill of the workload's prompt then its decode (greedy in one launch
    for B=1; B=16 clones of the prefilled state stepping through
    qdec_decode_batch), `warmup` untimed and `steps` timed repetitions.
    Returns per-repetition prefill and decode milliseconds (HIP events on the
    library's stream) and the wall time of the timed repetitions."""
    import torch

    import synth
    from qwen3_kv_cache_amd import qdec

    dev = torch.device("cuda:0")
    ids, audio, a0 = synth.make_prompt(w)
    audio_d = torch.from_numpy(audio).to(dev)
    B = w.n_branch
    n = w.n_decode
    toks = torch.zeros((n + 1, B), dtype=torch.int32, device=dev)
    streams = np.stack([synth.branch_stream(w, b) for b in range(B)]) if B > 1 else None
    total = warmup + steps
    states = [qdec.qdec_state_create(model.handle, w.max_ctx) for _ in range(total)]
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(total)]
    torch.cuda.synchronize()

    def one_step(i):
        st = states[i]
        e0, e1, e1d, e2 = ev[i]
        e0.record()
        qdec.qdec_prefill(st, ids, len(ids), audio_d.data_ptr(), a0, len(audio), None, toks[0].data_ptr())
        e1.record()
        if B == 1:
            e1d.record()
            if per_step:
                for s in range(n):
                    qdec.qdec_decode_step_dev(st, toks[s].data_ptr(), w.prompt_len + s, None, toks[s + 1].data_ptr())
            else:
                qdec.qdec_decode_greedy(st, toks[0].data_ptr(), w.prompt_len, n, None, toks[1].data_ptr())
        else:
            # the clones (host work and a page-table upload each) stay outside
            # the timed decode
            br = [qdec.qdec_clone_state(st) for _ in range(B)]
            e1d.record()
            for s in range(n):
                qdec.qdec_decode_batch(br, streams[:, s], None, toks[s + 1].data_ptr())
            e2.record()
            torch.cuda.synchronize()
            for b in br:
                qdec.qdec_state_destroy(b)
            return
        e2.record()

    for i in range(warmup):
        one_step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(warmup, total):
        one_step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_ms = np.array([ev[i][0].elapsed_time(ev[i][1]) for i in range(warmup, total)])
    dec_ms = np.array([ev[i][2].elapsed_time(ev[i][3]) for i in range(warmup, total)])
    for st in states:
        qdec.qdec_state_destroy(st)
    return pre_ms, dec_ms, wall


def measure_sampling(model, V, calls=20, groups=7):
    """qdec_sample on 1 and 16 rows of seeded N(0, 3^2) logits (temperature
    0.8, top-k 50, top-p 0.95, repetition penalty 1.1 over 64 history ids):
    microseconds per call as the median of `groups` timed groups of `calls`
    calls each (HIP events on the library's stream), with every group's value."""
    import torch

    from qwen3_kv_cache_amd import qdec

    dev = torch.device("cuda:0")
    rng = np.random.default_rng(7)
    out = {"temperature": 0.8, "top_k": 50, "top_p": 0.95, "repetition_penalty": 1.1, "history": 64}
    for n in (1, 16):
        z = torch.from_numpy((3.0 * rng.standard_normal((n, V))).astype(np.float32)).to(dev)
        h = torch.from_numpy(rng.integers(0, V, size=(n, 64)).astype(np.int32)).to(dev)
        tok = torch.zeros(n, dtype=torch.int32, device=dev)
        u = rng.random(n).astype(np.float32)

        def call():
            qdec.qdec_sample(model.handle, z.data_ptr(), n, 0.8, 50, 0.95, 1.1, h.data_ptr(), 64, u, tok.data_ptr())

        for _ in range(3):
            call()
        torch.cuda.synchronize()
        per = []
        for _ in range(groups):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(calls):
                call()
            e1.record()
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) * 1e3 / calls)
        out[f"rows{n}_us"] = round(float(np.median(per)), 2)
        out[f"rows{n}_us_groups"] = [round(x, 2) for x in per]
    return out


# Stamp slots of the diagnostic decode build (first decode step of a launch,
# first exchange thread of each workgroup): slot 1 + 10 l + i is boundary i of
# layer l, 1 + 10 L is the final residual, 300-302 close the LM head and the
# argmax exchange.
TRACE_PHASES = ("A  input norm + QKV dot", "E1 q/k/v rows exchange (group)", "B  QK-norm, RoPE, attention",
                "M  attention merge (+ split exchange)", "C  O dot + publish", "E3 O partials exchange (chip)",
                "D  post norm + gate/up dot + SwiGLU", "E4 z exchange (group)", "E  down dot + publish",
                "E5 down partials exchange (chip)")


def decode_trace(w, model, n_steps: int = 8):
    """Per-phase time of one decode step from the diagnostic library's
    realtime-counter stamps (100 MHz): median and 90th percentile over
    workgroups and layers 1 .. L-2 of each phase, plus the LM head."""
    import ctypes

    import torch

    import synth
    from qwen3_kv_cache_amd import qdec

    L = w.shape.n_layer
    dev = torch.device("cuda:0")
    ids, audio, a0 = synth.make_prompt(w)
    audio_d = torch.from_numpy(audio).to(dev)
    toks = torch.zeros(n_steps + 1, dtype=torch.int32, device=dev)
    for rep in range(2):  # the second launch is the one read back
        st = qdec.qdec_state_create(model.handle, w.max_ctx)
        qdec.qdec_prefill(st, ids, len(ids), audio_d.data_ptr(), a0, len(audio), None, toks[0].data_ptr())
        qdec.qdec_decode_greedy(st, toks[0].data_ptr(), w.prompt_len, n_steps, None, toks[1].data_ptr())
        torch.cuda.synchronize()
        qdec.qdec_state_destroy(st)
    nb = torch.cuda.get_device_properties(0).multi_processor_count
    n = nb * 512
    buf = (ctypes.c_ulonglong * n)()
    if qdec.lib().qdec_debug_trace(buf, n) != 0:
        raise RuntimeError("qdec_debug_trace failed")
    t = np.frombuffer(buf, dtype=np.uint64).reshape(nb, 512).astype(np.int64)
    us = 0.01  # one realtime tick = 10 ns
    rows = {}
    for i, name in enumerate(TRACE_PHASES):
        d = []
        for l in range(1, L - 1):
            a = t[:, 1 + 10 * l + i]
            b = t[:, 1 + 10 * (l + 1)] if i == 9 else t[:, 1 + 10 * l + i + 1]
            d.append((b - a) * us)
        d = np.concatenate(d)
        rows[name] = {"median_us": round(float(np.median(d)), 3), "p90_us": round(float(np.percentile(d, 90)), 3)}
    layer = np.concatenate([(t[:, 1 + 10 * (l + 1)] - t[:, 1 + 10 * l]) * us for l in range(1, L - 1)])
    head = (t[:, 300] - t[:, 1 + 10 * L]) * us
    key = (t[:, 302] - t[:, 300]) * us
    step = (t[:, 302] - t[:, 0]) * us
    # Exchanges: the realtime counter is chip-wide, so a consumer's completion
    # can be set against its producers' publish stamps: "skew" is how long the
    # consumer waited for the last producer, "latency" the time from the last
    # publish to the consumer seeing every word.
    grp = np.arange(nb) % 8

    def xch(pub_i, done_i, nxt, local):
        lat, skew = [], []
        for l in range(1, L - 1):
            pub = t[:, 1 + 10 * l + pub_i]
            done = t[:, 1 + 10 * (l + nxt) + done_i]
            last = np.array([pub[grp == g].max() for g in range(8)])[grp] if local else np.full(nb, pub.max())
            lat.append((done - last) * us)
            skew.append((last - pub) * us)
        lat, skew = np.concatenate(lat), np.concatenate(skew)
        return {"latency_after_last_publish_us": round(float(np.median(lat)), 3),
                "wait_for_last_producer_us": round(float(np.median(skew)), 3)}
    exchanges = {"E3 O partials (chip)": xch(5, 6, 0, False), "E4 z (group)": xch(7, 8, 0, True),
                 "E5 down partials (chip)": xch(9, 0, 1, False)}
    # inside the FFN phases (layers 1 .. 7): D = input norm | bars + dot | SwiGLU + publish,
    # E = bars + dot | publish + attention prefetch
    sub = {}
    for name, a_i, b_i in (("D norm_input", 6, 401), ("D bars+dot", 401, 402), ("D swiglu+publish", 402, 7),
                           ("E bars+dot", 8, 403), ("E publish+prefetch", 403, 9)):
        d = []
        for l in range(1, 8):
            ia = 1 + 10 * l + a_i if a_i < 10 else 400 + l * 4 + (a_i - 400)
            ib = 1 + 10 * l + b_i if b_i < 10 else 400 + l * 4 + (b_i - 400)
            d.append((t[:, ib] - t[:, ia]) * us)
        sub[name] = round(float(np.median(np.concatenate(d))), 3)
    out = {"phases": rows, "exchanges": exchanges, "ffn_detail_us": sub, "layer_us_median": round(float(np.median(layer)), 3),
           "head_dot_us_median": round(float(np.median(head)), 3),
           "argmax_exchange_us_median": round(float(np.median(key)), 3),
           "step_us_median": round(float(np.median(step)), 3), "workgroups": nb,
           "workload": w.name, "context": w.prompt_len}
    # attention stages of layers 1 .. 3 (slots 464 + 8 (l - 1) + i): A publish
    # done, block 0 started, QK-norm + RoPE done, exchange-wave sync, partial
    # done, second sync; and block 0's scores done, end of the partial
    att = {}
    for name, i0, i1 in (("qkv gather", None, 0), ("qk-norm+rope", 0, 2), ("sync1", 2, 3), ("partial", 3, 4),
                         ("sync2", 4, 5), ("partial: to scores", 1, 6), ("partial: scores..end", 6, 7),
                         ("block0: key select", 1, 101), ("block0: head0 scores", 101, 103),
                         ("block0: head0 softmax..head1 start", 103, 102), ("block0: head1..softmax end", 102, 6)):
        d = []
        for l in range(1, 4):
            def slot(i):  # 0..7: attention stages; 101..103: block-0 details
                return 432 + 8 * (l - 1) + (i - 100) if i >= 100 else 464 + 8 * (l - 1) + i
            b = t[:, slot(i1)]
            a = t[:, 1 + 10 * l + 1] if i0 is None else t[:, slot(i0)]
            d.append((b - a) * us)
        att[name] = round(float(np.median(np.concatenate(d))), 3)
    # memory wave 0 of each workgroup: units 4 .. 15 of the step (6 stamps each:
    # start, input ready, ring filled, dot done, partials ready, next issued)
    m = t[:, 320:392].reshape(nb, 12, 6)
    out["memory_wave"] = {k: round(float(np.median((m[:, :, j + 1] - m[:, :, j]) * us)), 3) for j, k in
                          enumerate(("wait input", "ring wait", "dot", "wait partials barrier", "issue"))}
    out["memory_wave_by_unit"] = {
        u: {k: round(float(np.median((m[:, ui::4, j + 1] - m[:, ui::4, j]) * us)), 3) for j, k in
            enumerate(("wait input", "ring wait", "dot", "wait partials barrier", "issue"))}
        for ui, u in enumerate(("A qkv", "C o", "D gate/up", "E down"))}
    out["attention_detail_us"] = att
    return out


def _csv_rows(directory: str, suffix: str):
    import csv
    import glob
    paths = sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))
    if not paths:
        raise SystemExit(f"no *{suffix} under {directory}")
    return list(csv.DictReader(open(paths[0])))


def profile_summary(kind: str, directory: str, bench_log: str = None, copy_dir: str = None) -> str:
    """Text summary of rocprofv3 output for profiles/: `stats` reads the
    kernel-trace statistics (time per kernel); `traffic` reads the FETCH_SIZE
    and WRITE_SIZE counter runs of the decode kernel (directory holds both)
    and of the 1 GiB copy probe (copy_dir), and converts the counters to HBM
    bytes per launch with the copy's known bytes as the scale."""
    import hashlib
    src = os.path.join(ROOT, "qwen3_kv_cache_amd", "csrc")
    shas = {f: hashlib.sha256(open(os.path.join(src, f), "rb").read()).hexdigest()
            for f in ("qdec_decode.hip", "qdec_kernels.hip", "qdec_encoder.hip")}
    out = []
    if kind == "stats":
        rows = _csv_rows(directory, "kernel_stats.csv")
        out.append(f"{'kernel':66s} {'calls':>6s} {'total_us':>11s} {'avg_us':>10s} {'pct':>6s}")
        for r in rows:
            name = r["Name"].replace("void ", "").replace("qdec::(anonymous namespace)::", "")[:64]
            out.append(f"{name:66s} {int(r['Calls']):6d} {float(r['TotalDurationNs']) / 1e3:11.1f} "
                       f"{float(r['AverageNs']) / 1e3:10.2f} {float(r['Percentage']):6.2f}")
        dec = [r for r in rows if "decode_kernel" in r["Name"]]
        if dec:
            avg = float(dec[0]["AverageNs"]) / 1e3
            out.append("")
            out.append(f"decode_kernel_avg_us_per_launch: {avg:.2f}")
        if bench_log:
            line = [ln for ln in open(bench_log) if ln.startswith("{")]
            if line:
                b = json.loads(line[-1])
                if "config" in b and "roofline" in b:
                    n = b["config"]["decode_steps"]
                    out.append(f"decode_us_per_token_from_profile: {avg / n:.2f}" if dec else "")
                    out.append(f"bench line of the same run (under the profiler): decode {b['value']} tok/s, "
                               f"roofline {b['roofline']['achieved']} GB/s = {100 * b['roofline']['frac']:.1f}% "
                               "of 8 TB/s")
                elif "config" in b:
                    out.append("")
                    out.append(f"bench line of the same run (under the profiler): {b['value']} {b['unit']}, "
                               f"prefill {b['prefill_ms']} ms")
                else:
                    out.append("")
                    out.append("bench line of the same run (under the profiler): " + json.dumps(b))
    elif kind == "mfma":
        # two counter runs of the prefill8k bench (one warm-up and one timed
        # prefill each): MfmaUtil under <dir>/util, SQ_INSTS_VALU_MFMA_MOPS_BF16
        # under <dir>/mops; the prefill kernels are every dispatch except the
        # decode kernel, copies and set-up
        def rows_of(d, counter):
            return [r for r in _csv_rows(d, "counter_collection.csv") if r["Counter_Name"] == counter]
        skip = ("decode_kernel", "__amd_rocclr", "clear_words", "to_f32", "q8_unpack", "xcc_probe")
        util = [r for r in rows_of(os.path.join(directory, "util"), "MfmaUtil") if not any(k in r["Kernel_Name"] for k in skip)]
        mops = [r for r in rows_of(os.path.join(directory, "mops"), "SQ_INSTS_VALU_MFMA_MOPS_BF16")
                if not any(k in r["Kernel_Name"] for k in skip)]
        short = lambda n: n.replace("void ", "").replace("qdec::(anonymous namespace)::", "").split("(")[0][:40]
        per = {}
        for r in util:
            k = short(r["Kernel_Name"])
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            e = per.setdefault(k, {"n": 0, "us": 0.0, "busy": 0.0, "mops": 0.0})
            e["n"] += 1
            e["us"] += dur
            e["busy"] += float(r["Counter_Value"]) * dur
        for r in mops:
            per.setdefault(short(r["Kernel_Name"]), {"n": 0, "us": 0.0, "busy": 0.0, "mops": 0.0})["mops"] += float(
                r["Counter_Value"])
        n_prefill = 2
        out.append(f"{'kernel':40s} {'dispatches':>10s} {'avg_us':>9s} {'MfmaUtil%':>10s} {'issued_TFLOP':>13s}")
        for k, e in sorted(per.items(), key=lambda kv: -kv[1]["us"]):
            if not e["n"]:
                continue
            out.append(f"{k:40s} {e['n']:10d} {e['us'] / e['n']:9.2f} {e['busy'] / max(e['us'], 1e-9):10.2f} "
                       f"{e['mops'] * 512 / 1e12:13.3f}")
        tot_us = sum(e["us"] for e in per.values())
        busy = sum(e["busy"] for e in per.values()) / max(tot_us, 1e-9)
        issued = sum(e["mops"] for e in per.values()) * 512 / n_prefill
        import synth
        useful = prefill_flops(synth.QWEN3_0P6B, 8192)
        out += ["", "Values below are machine-readable by bench.py (key: value).",
                f"source_sha256: {shas['qdec_kernels.hip']}", f"mfma_busy_pct_prefill_kernels: {busy:.2f}",
                f"mfma_flops_issued_per_prefill: {issued:.4e}", f"useful_flops_per_prefill: {useful:.4e}", "",
                f"Issued / useful MFMA FLOPs = {issued / useful:.3f}. Time-weighted MfmaUtil over the prefill kernels "
                f"= {busy:.2f}%."]
    else:
        def per_dispatch(d, counter, kernel):
            rows = [r for r in _csv_rows(d, "counter_collection.csv") if r["Counter_Name"] == counter and kernel in r["Kernel_Name"]]
            vals = [float(r["Counter_Value"]) for r in rows]
            return (sum(vals) / len(vals), len(vals)) if vals else (float("nan"), 0)
        f_dec, nf = per_dispatch(os.path.join(directory, "fetch"), "FETCH_SIZE", "decode_kernel")
        w_dec, nw = per_dispatch(os.path.join(directory, "write"), "WRITE_SIZE", "decode_kernel")
        f_cp, _ = per_dispatch(os.path.join(copy_dir, "fetch"), "FETCH_SIZE", "copyBuffer")
        w_cp, _ = per_dispatch(os.path.join(copy_dir, "write"), "WRITE_SIZE", "copyBuffer")
        gib_kib = (1 << 30) / 1024
        fs, ws = gib_kib / f_cp, gib_kib / w_cp
        hbm = (f_dec * fs + w_dec * ws) * 1024
        import synth
        w = synth.WORKLOADS["short"]
        alg = decode_bytes(w.shape, [w.prompt_len + s + 1 for s in range(w.n_decode)]) * w.n_decode
        out += [f"source_sha256: {shas['qdec_decode.hip']}", f"fetch_kib_per_dispatch: {f_dec:.1f}",
                f"write_kib_per_dispatch: {w_dec:.1f}", f"copy_fetch_kib: {f_cp:.1f}", f"copy_write_kib: {w_cp:.1f}",
                f"fetch_scale: {fs:.4f}", f"write_scale: {ws:.4f}", f"hbm_bytes_per_launch: {hbm:.0f}",
                f"algorithmic_bytes_per_launch: {alg:.0f}", "",
                f"Traffic / algorithmic bytes = {hbm / alg:.4f} (dispatches averaged: {nf} fetch, {nw} write)."]
    out.append("")
    out.append("Source sha256 (qwen3_kv_cache_amd/csrc): " + "; ".join(f"{k} {v}" for k, v in shas.items()))
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="short")
    ap.add_argument("--cpu-sample", type=int, default=64,
                    help="greedy decode steps the CPU oracle runs for the baseline (0 = skip)")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--adaptor-only", action="store_true",
                    help="time only the audio adaptor (qdec_adaptor_run) and print its JSON")
    ap.add_argument("--encoder-only", action="store_true",
                    help="time only the frontend + SAN-M encoder (qdec_encoder_run) and print its JSON")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the other workloads the default run also reports (B=16, long and 8k prompts)")
    ap.add_argument("--trace", action="store_true",
                    help="per-phase time of a decode step from the diagnostic build libqdec_trace.so "
                         "(python -m qwen3_kv_cache_amd.build --trace)")
    ap.add_argument("--q8", action="store_true",
                    help="the main measurement on Q8_0 weights (int8 codes, fp16 block scales) of the same shape")
    ap.add_argument("--per-step", action="store_true",
                    help="decode with one launch per token (qdec_decode_step_dev) instead of one launch for all steps")
    ap.add_argument("--profile-summary", choices=("stats", "traffic", "mfma"),
                    help="print the profiles/ summary of rocprofv3 output under --profile-dir (no GPU use)")
    ap.add_argument("--profile-dir")
    ap.add_argument("--copy-dir", help="counter runs of --copy-probe (traffic summaries)")
    ap.add_argument("--bench-log", help="bench output of the profiled run (stats summaries)")
    a = ap.parse_args()
    if a.profile_summary:
        print(profile_summary(a.profile_summary, a.profile_dir, a.bench_log, a.copy_dir))
        return
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {a.gpus}); the decoder is single-GPU by design.",
              file=sys.stderr)
        sys.exit(2)
    if a.copy_probe:
        copy_probe()
        return
    if a.adaptor_only:
        print(json.dumps({"adaptor": measure_adaptor()}), flush=True)
        return
    if a.encoder_only:
        print(json.dumps({"encoder": measure_encoder()}), flush=True)
        return

    import torch

    import synth
    from qwen3_kv_cache_amd import qdec
    from qwen3_kv_cache_amd.device import Model

    if a.trace:
        from qwen3_kv_cache_amd.build import TRACE_LIB
        qdec.use_library(TRACE_LIB)
    w = synth.WORKLOADS[a.workload]
    dev = torch.device("cuda:0")
    W = synth.make_weights(w.shape, w.weight_seed)
    if a.q8:
        model = Model(w.shape, synth.make_q8_weights(w.shape, w.weight_seed).abi_arrays(), bf16=False, q8=True)
    else:
        model = Model(w.shape, W.bits if w.shape.bf16 else W.f32, bf16=w.shape.bf16)
    if a.trace:
        res = decode_trace(w, model)
        model.close()
        for k, v in res["phases"].items():
            print(f"{k:42s} median {v['median_us']:7.3f} us   p90 {v['p90_us']:7.3f} us", flush=True)
        for k, v in res["exchanges"].items():
            print(f"{k:42s} latency {v['latency_after_last_publish_us']:7.3f} us   "
                  f"producer skew {v['wait_for_last_producer_us']:7.3f} us", flush=True)
        print(json.dumps(res["ffn_detail_us"]), flush=True)
        print(json.dumps({"decode_trace": res}), flush=True)
        return
    pre_ms, dec_ms, wall = measure(w, model, a.steps, a.warmup, a.per_step)
    n, B = w.n_decode, w.n_branch
    decode_tok_s = n * B * a.steps / (dec_ms.sum() / 1e3)
    prefill_tok_s = w.prompt_len * a.steps / (pre_ms.sum() / 1e3)
    ctx = [w.prompt_len + s + 1 for s in range(n)]
    bytes_tok = (decode_bytes_q8 if a.q8 else decode_bytes)(w.shape, ctx)
    per_tok_s = dec_ms.mean() / 1e3 / n
    achieved = bytes_tok / per_tok_s / 1e9 if B == 1 else None
    line = {
        "metric": METRIC,
        "value": round(decode_tok_s, 2),
        "unit": "decode tok/s" if B == 1 else "decode tok/s (B=16, summed over branches)",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(wall / a.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("Q8_0 weights (int8 codes, fp16 block scales)" if a.q8 else "bf16 weights")
                 + ", fp32 activations/KV",
        "data": "synthetic (seeded random-init weights of the Qwen3-0.6B shape, uniform ids, N(0,1) audio rows)",
        "config": {"workload": f"{w.name}: Qwen3-0.6B shape, {w.prompt_len}-token prompt with {w.audio_len} audio rows, "
                               f"prefill then {n} greedy decode steps" + (f" x {B} cloned branches" if B > 1 else ", B=1"),
                   "prompt_len": w.prompt_len, "audio_rows": w.audio_len, "decode_steps": n, "batch": B},
        "prefill_tok_s": round(prefill_tok_s, 1),
        "prefill_ms": round(float(pre_ms.mean()), 4),
        "decode_ms_per_token": round(float(dec_ms.mean()) / n, 5),
        "prefill_mfma": prefill_mfma(w.shape, w.prompt_len, float(pre_ms.mean()), w.name),
    }
    if achieved is not None:
        # counters were taken on the short workload's 64-step launch
        traffic = counter_traffic() if (w.name == "short" and not a.per_step and not a.q8) else None
        line["roofline"] = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                            "kernel": "decode_kernel (%d steps per launch)" % (1 if a.per_step else n),
                            "bytes_per_unit": round(bytes_tok)}
    if a.workload == "short" and not a.no_others and not a.q8:
        # the rest of the metric (B=16 decode, prefill of long prompts), same
        # weights, fewer repetitions
        others = {}
        for name in ("branch16", "long", "prefill8k"):
            wo = synth.WORKLOADS[name]
            assert wo.shape == w.shape and wo.weight_seed == w.weight_seed, name
            p_ms, d_ms, _ = measure(wo, model, 2, 1)
            others[name] = {"decode_tok_s": round(wo.n_decode * wo.n_branch * len(d_ms) / (d_ms.sum() / 1e3), 1),
                            "batch": wo.n_branch, "prompt_len": wo.prompt_len, "decode_steps": wo.n_decode,
                            "prefill_tok_s": round(wo.prompt_len * len(p_ms) / (p_ms.sum() / 1e3), 1),
                            "prefill_ms": round(float(p_ms.mean()), 3),
                            "prefill_mfma": prefill_mfma(wo.shape, wo.prompt_len, float(p_ms.mean()), name),
                            "decode_roofline": decode_roofline(wo.shape, wo, float(d_ms.mean()))}
        # the short workload on Q8_0 weights of the same shape and seed: the
        # decode kernel streams int8 codes and fp16 scales; prefill runs on the
        # exactly dequantized fp32 weights
        Q = synth.make_q8_weights(w.shape, w.weight_seed)
        m8 = Model(w.shape, Q.abi_arrays(), bf16=False, q8=True)
        p_ms, d_ms, _ = measure(w, m8, 3, 1)
        m8.close()
        t_tok = float(d_ms.mean()) / 1e3 / n
        b8 = decode_bytes_q8(w.shape, ctx)
        others["short_q8_0"] = {"decode_tok_s": round(n * len(d_ms) / (d_ms.sum() / 1e3), 1), "batch": 1,
                                "prompt_len": w.prompt_len, "decode_steps": n,
                                "decode_ms_per_token": round(t_tok * 1e3, 5),
                                "prefill_tok_s": round(w.prompt_len * len(p_ms) / (p_ms.sum() / 1e3), 1),
                                "decode_roofline": {"bytes_per_step": round(b8), "achieved": round(b8 / t_tok / 1e9, 1),
                                                    "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                                    "frac": round(b8 / t_tok / 1e9 / HBM_PEAK_GBS, 4)}}
        line["other_workloads"] = others
        line["sampling"] = measure_sampling(model, w.shape.vocab)
        line["adaptor"] = measure_adaptor()
        line["encoder"] = measure_encoder()
    if a.cpu_sample > 0 and not a.q8:
        line["cpu_baseline"] = cpu_baseline(w, W, a.cpu_sample)
    model.close()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
