"""GPU parity of block-int8 (Q8_0) weights (audio.cpp "Fun-ASR-Nano Native
Runtime Implementation Plan", Task 8: a Q8_0 package must give the same greedy
transcript as the float weights). The library is fed Q8_0 blocks; the oracle
is the float64 decoder fed the exact dequantized weights q * d
(oracle.quant.dequantize). Prefill and the batched path compute on those fp32
weights inside the library, the single-sequence decode kernel on the int8
codes and fp16 scales, so both are held to the fp32-weight bar."""
import numpy as np
import pytest

import oracle
import synth
from oracle.quant import dequantize

from .gpu_harness import check_steps, oracle_forced, record, run_forced, torch_dev

pytestmark = pytest.mark.gpu


def oracle_params(Q):
    """Float weights of a Q8_0 set: q * d for the matrices and the embedding,
    the float32 norm gains as they are."""
    out = {}
    for name in Q.base.names():
        out[name] = dequantize(Q.codes[name], Q.scales[name]) if name in Q.codes else Q.base.f32[name]
    return out


def q8_model(Q):
    from qwen3_kv_cache_amd.device import Model
    return Model(Q.shape, Q.abi_arrays(), bf16=False, q8=True)


def workload(shape, seed, T, La, n_decode):
    ids = synth.random_ids(seed, T, shape.vocab)
    audio = synth.random_rows(seed, La, shape.hidden)
    forced = synth.random_ids(seed + 100, n_decode, shape.vocab)
    return ids, audio, forced


SHAPES = {
    # D=64, GQA 2; T=300 leaves ragged tiles, V=5003 a ragged LM-head block
    "d64_g2": (synth.custom_shape(hidden=256, n_layer=2, n_q_head=4, n_kv_head=2, head_dim=64, ffn=768,
                                  vocab=5003), 300, 17, 100, 12),
    # the 0.6B head geometry (D=128, GQA 2): rows of 512 inputs (16 scale blocks)
    "d128_g2": (synth.custom_shape(hidden=512, n_layer=3, n_q_head=8, n_kv_head=4, head_dim=128, ffn=1536,
                                   vocab=4099), 77, 8, 20, 10),
    # GQA 4, D=32: the O projection's per-group slices are 256 inputs wide,
    # the down projection's 64 (two scale blocks, padded scale segments)
    "d32_g4": (synth.custom_shape(hidden=128, n_layer=2, n_q_head=8, n_kv_head=2, head_dim=32, ffn=512,
                                  vocab=777), 45, 3, 9, 6),
    # MHA, hidden 1024 (rows of 64 scale blocks, the decode kernel's widest)
    "h1024_g1": (synth.custom_shape(hidden=1024, n_layer=1, n_q_head=8, n_kv_head=8, head_dim=128, ffn=1024,
                                    vocab=1500), 33, 0, 0, 8),
}


@pytest.mark.parametrize("name", sorted(SHAPES))
def test_q8_teacher_forced(name):
    shape, T, a0, La, n = SHAPES[name]
    Q = synth.make_q8_weights(shape, 21)
    ids, audio, forced = workload(shape, 21, T, La, n)
    orc = oracle.Qwen3Oracle(oracle.OracleConfig.from_shape(shape), oracle_params(Q))
    ref = oracle_forced(orc, ids, audio, a0, forced)
    print(f"[q8 {name}] prefill {T} + {n} steps", flush=True)
    m = q8_model(Q)
    try:
        gpu, amax = run_forced(m, ids, audio, a0, forced)
    finally:
        m.close()
    print(name, check_steps(gpu, amax, ref, fp32=True, label=f"q8 {name}"))


def test_q8_greedy_one_launch():
    """16 greedy steps in one decode launch, crossing the 128-position point
    where the kernel's attention switches from whole-per-rank to split."""
    from qwen3_kv_cache_amd import qdec
    shape, _, a0, La, _ = SHAPES["d128_g2"]
    T, n = 120, 16
    Q = synth.make_q8_weights(shape, 22)
    ids, audio, _ = workload(shape, 22, T, La, 1)
    orc = oracle.Qwen3Oracle(oracle.OracleConfig.from_shape(shape), oracle_params(Q))
    toks, ref = oracle.greedy_trajectory(orc, ids, audio, a0, n)
    torch, dev = torch_dev()
    m = q8_model(Q)
    try:
        st = qdec.qdec_state_create(m.handle, T + n)
        l0 = torch.full((shape.vocab,), float("nan"), dtype=torch.float32, device=dev)
        t0 = torch.full((1,), -1, dtype=torch.int32, device=dev)
        audio_d = torch.from_numpy(audio).to(dev)
        qdec.qdec_prefill(st, ids, T, audio_d.data_ptr(), a0, len(audio), l0.data_ptr(), t0.data_ptr())
        logits = torch.full((n, shape.vocab), float("nan"), dtype=torch.float32, device=dev)
        out = torch.full((n,), -1, dtype=torch.int32, device=dev)
        print(f"[q8 greedy] {n} steps from pos {T}", flush=True)
        qdec.qdec_decode_greedy(st, t0.data_ptr(), T, n, logits.data_ptr(), out.data_ptr())
        torch.cuda.synchronize()
        qdec.qdec_model_status(m.handle)
        qdec.qdec_state_destroy(st)
    finally:
        m.close()
    got = np.concatenate([t0.cpu().numpy(), out.cpu().numpy()])
    assert list(got) == list(toks), f"tokens {got} != oracle {toks}"
    gpu = np.concatenate([l0.cpu().numpy()[None], logits.cpu().numpy()])
    check_steps(gpu, got, ref, fp32=True, label="q8 greedy d128_g2")


def test_q8_batch_rows():
    """Four clones of one prompt decoded together through the batched path
    (which runs on the dequantized fp32 weights), against the oracle."""
    from qwen3_kv_cache_amd import qdec
    shape, T, a0, La, _ = SHAPES["d64_g2"]
    B, n = 4, 3
    Q = synth.make_q8_weights(shape, 23)
    ids, audio, _ = workload(shape, 23, T, La, 1)
    feed = np.stack([synth.random_ids(500 + b, n, shape.vocab) for b in range(B)])
    orc = oracle.Qwen3Oracle(oracle.OracleConfig.from_shape(shape), oracle_params(Q))
    st0 = orc.new_state()
    orc.prefill(st0, ids, audio, a0)
    ref = np.zeros((n, B, shape.vocab))
    for b in range(B):
        sb = st0.clone()
        for s in range(n):
            ref[s, b] = orc.decode(sb, int(feed[b, s]), T + s)
    torch, dev = torch_dev()
    m = q8_model(Q)
    try:
        base = qdec.qdec_state_create(m.handle, T + n)
        audio_d = torch.from_numpy(audio).to(dev)
        qdec.qdec_prefill(base, ids, T, audio_d.data_ptr(), a0, len(audio), None, None)
        rows = [qdec.qdec_clone_state(base) for _ in range(B)]
        qdec.qdec_state_destroy(base)
        logits = torch.full((n, B, shape.vocab), float("nan"), dtype=torch.float32, device=dev)
        amax = torch.full((n, B), -1, dtype=torch.int32, device=dev)
        print(f"[q8 batch] {B} rows, {n} steps", flush=True)
        for s in range(n):
            qdec.qdec_decode_batch(rows, feed[:, s], logits[s].data_ptr(), amax[s].data_ptr())
        torch.cuda.synchronize()
        for st in rows:
            qdec.qdec_state_destroy(st)
    finally:
        m.close()
    L, A = logits.cpu().numpy(), amax.cpu().numpy()
    for b in range(B):
        check_steps(L[:, b], A[:, b], ref[:, b], fp32=True, label=f"q8 batch row {b}")


def test_q8_06b_short():
    """The 0.6B shape with Q8_0 weights on the short workload's prompt (64
    tokens with an audio span), 8 teacher-forced decode steps, then a greedy
    launch of 8 steps from the same prompt: every step's full logit vector
    against the oracle, and the same tokens."""
    from qwen3_kv_cache_amd import qdec
    w = synth.WORKLOADS["short"]
    Q = synth.make_q8_weights(w.shape, w.weight_seed)
    ids, audio, a0 = synth.make_prompt(w)
    n = 8
    orc = oracle.Qwen3Oracle(oracle.OracleConfig.from_shape(w.shape), oracle_params(Q))
    toks, ref = oracle.greedy_trajectory(orc, ids, audio, a0, n)
    torch, dev = torch_dev()
    print(f"[q8 0.6B] prefill {len(ids)}, forced + greedy {n} steps", flush=True)
    m = q8_model(Q)
    try:
        gpu, amax = run_forced(m, ids, audio, a0, toks[:-1])
        T = len(ids)
        st = qdec.qdec_state_create(m.handle, T + n)
        audio_d = torch.from_numpy(np.ascontiguousarray(audio, dtype=np.float32)).to(dev)
        t0 = torch.full((1,), -1, dtype=torch.int32, device=dev)
        qdec.qdec_prefill(st, ids, T, audio_d.data_ptr(), a0, len(audio), None, t0.data_ptr())
        out = torch.full((n,), -1, dtype=torch.int32, device=dev)
        qdec.qdec_decode_greedy(st, t0.data_ptr(), T, n, None, out.data_ptr())
        torch.cuda.synchronize()
        qdec.qdec_model_status(m.handle)
        qdec.qdec_state_destroy(st)
    finally:
        m.close()
    worst = check_steps(gpu, amax, ref, fp32=True, label="q8 0.6B short")
    got = [int(t0.cpu()[0])] + [int(t) for t in out.cpu().numpy()]
    assert got == list(toks), f"greedy tokens {got} != oracle {toks}"
    record("q8 0.6B short greedy", 0, {"tokens_equal": True}, kind="tokens")
    print("q8 0.6B", worst)
