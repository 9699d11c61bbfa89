"""GPU parity at sizes the float64 oracle finishes in seconds, spanning several
tiles and ragged tails: teacher-forced prefill + decode logits and argmax."""
import numpy as np
import pytest

import oracle
import synth

from .gpu_harness import check_steps, device_model, mid_workload, oracle_forced, run_forced

pytestmark = pytest.mark.gpu

MID = {
    # D=64, GQA 2, context crosses the 256-position split and many pages;
    # T=300 leaves a ragged GEMM tile, V=5003 a ragged LM-head block
    "d64_g2": (synth.custom_shape(hidden=256, n_layer=2, n_q_head=4, n_kv_head=2, head_dim=64, ffn=768,
                                  vocab=5003, bf16=True), 300, 17, 100, 12),
    # D=128, GQA 2 (the 0.6B head geometry), 3 layers
    "d128_g2": (synth.custom_shape(hidden=512, n_layer=3, n_q_head=8, n_kv_head=4, head_dim=128, ffn=1536,
                                   vocab=4099, bf16=True), 77, 8, 20, 10),
    # GQA 4 with fp32 weights
    "d32_g4_f32": (synth.custom_shape(hidden=128, n_layer=2, n_q_head=8, n_kv_head=2, head_dim=32, ffn=384,
                                      vocab=777, bf16=False), 45, 3, 9, 6),
    # MHA (group 1), D=128, one layer, prompt of one token
    "d128_g1_T1": (synth.custom_shape(hidden=256, n_layer=1, n_q_head=4, n_kv_head=4, head_dim=128, ffn=512,
                                      vocab=1000, bf16=True), 1, 0, 0, 20),
    # MHA, D=128, a 1100-token prompt: the causal attention with two 16-query
    # blocks per wave (one query head per KV head, T >= 1024), ragged last block
    "d128_g1_T1100": (synth.custom_shape(hidden=256, n_layer=1, n_q_head=2, n_kv_head=2, head_dim=128, ffn=512,
                                         vocab=1000, bf16=True), 1100, 8, 100, 4),
    # MHA, D=128, a 200-token prompt: one 16-query block per wave with the
    # Q/K norm and RoPE applied inside the matrix-core attention launch
    "d128_g1_T200": (synth.custom_shape(hidden=256, n_layer=2, n_q_head=2, n_kv_head=2, head_dim=128, ffn=512,
                                        vocab=1000, bf16=True), 200, 8, 100, 4),
    # ffn 320: the down projection's K is five 64-wide steps, so its K
    # splits are uneven (3 + 2 steps) on the 64-row, two-sub-step GEMM tiles
    "d64_g2_ffn320_T150": (synth.custom_shape(hidden=256, n_layer=2, n_q_head=4, n_kv_head=2, head_dim=64, ffn=320,
                                              vocab=1000, bf16=True), 150, 10, 60, 4),
    # a prompt made only of audio rows (span [0, T)): no id is read
    "d64_g2_allaudio": (synth.custom_shape(hidden=256, n_layer=2, n_q_head=4, n_kv_head=2, head_dim=64, ffn=768,
                                           vocab=5003, bf16=True), 40, 0, 40, 6),
    # short prompts take the fused attention launch (QK-norm, RoPE, append and
    # attention together, T <= 64): GQA 4 with a ragged third 16-query block,
    # and D=32 at exactly 64 positions
    "d64_g4_T33": (synth.custom_shape(hidden=256, n_layer=2, n_q_head=8, n_kv_head=2, head_dim=64, ffn=768,
                                      vocab=1000, bf16=True), 33, 5, 10, 6),
    "d32_g4_T64": (synth.custom_shape(hidden=128, n_layer=2, n_q_head=8, n_kv_head=2, head_dim=32, ffn=384,
                                      vocab=777, bf16=True), 64, 20, 12, 6),
}


def test_tiny_teacher_forced():
    w = synth.WORKLOADS["tiny"]
    W = synth.make_weights(w.shape, w.weight_seed)
    ids, audio, a0 = synth.make_prompt(w)
    orc = oracle.Qwen3Oracle(oracle.OracleConfig.from_shape(w.shape), W.f32)
    toks, ref = oracle.greedy_trajectory(orc, ids, audio, a0, w.n_decode)
    m = device_model(w.shape, W)
    try:
        gpu, amax = run_forced(m, ids, audio, a0, toks[:-1])
    finally:
        m.close()
    worst = check_steps(gpu, amax, ref, fp32=True, label="tiny")
    print("tiny", worst)


@pytest.mark.parametrize("name", sorted(MID))
def test_mid_shapes(name):
    shape, T, a0, La, n = MID[name]
    W, ids, audio, a0, forced = mid_workload(shape, 7, T, a0, La, n)
    orc = oracle.Qwen3Oracle(oracle.OracleConfig.from_shape(shape), W.f32)
    ref = oracle_forced(orc, ids, audio, a0, forced)
    m = device_model(shape, W)
    try:
        gpu, amax = run_forced(m, ids, audio, a0, forced)
    finally:
        m.close()
    worst = check_steps(gpu, amax, ref, fp32=not shape.bf16, label=name)
    print(name, worst)


# Multi-step greedy decode in one launch: the device feeds each step's argmax to
# the next (NCNN page section 5 loop, section 6 greedy default). The first case
# crosses the 128-position boundary where attention switches from every rank of
# a group running it whole to a split over ranks; positions written earlier in
# the same launch are read back by later steps.
GREEDY = {
    "d128_g2_cross128": (synth.custom_shape(hidden=512, n_layer=3, n_q_head=8, n_kv_head=4, head_dim=128,
                                            ffn=1536, vocab=4099, bf16=True), 120, 8, 30, 16),
    "tiny_fp32": (synth.TINY, 32, 8, 8, 12),
}


@pytest.mark.parametrize("name", sorted(GREEDY))
def test_greedy_multi_step(name):
    from qwen3_kv_cache_amd import qdec
    from .gpu_harness import torch_dev
    shape, T, a0, La, n = GREEDY[name]
    W, ids, audio, a0, _ = mid_workload(shape, 11, T, a0, La, 1)
    orc = oracle.Qwen3Oracle(oracle.OracleConfig.from_shape(shape), W.f32)
    toks, ref = oracle.greedy_trajectory(orc, ids, audio, a0, n)
    torch, dev = torch_dev()
    m = device_model(shape, W)
    try:
        st = qdec.qdec_state_create(m.handle, T + n)
        l0 = torch.full((shape.vocab,), float("nan"), dtype=torch.float32, device=dev)
        t0 = torch.full((1,), -1, dtype=torch.int32, device=dev)
        audio_d = torch.from_numpy(audio).to(dev)
        qdec.qdec_prefill(st, ids, T, audio_d.data_ptr(), a0, len(audio), l0.data_ptr(), t0.data_ptr())
        logits = torch.full((n, shape.vocab), float("nan"), dtype=torch.float32, device=dev)
        out = torch.full((n,), -1, dtype=torch.int32, device=dev)
        print(f"[{name}] greedy {n} steps from pos {T}", flush=True)
        qdec.qdec_decode_greedy(st, t0.data_ptr(), T, n, logits.data_ptr(), out.data_ptr())
        torch.cuda.synchronize()
        assert qdec.qdec_state_pos(st) == T + n
        qdec.qdec_state_destroy(st)
    finally:
        m.close()
    got_tokens = np.concatenate([t0.cpu().numpy(), out.cpu().numpy()])
    assert list(got_tokens) == list(toks), f"{name}: tokens {got_tokens} != oracle {toks}"
    gpu = np.concatenate([l0.cpu().numpy()[None], logits.cpu().numpy()])
    # the argmax written is the token fed forward: check logits against the oracle step by step
    worst = check_steps(gpu, got_tokens, ref, fp32=not shape.bf16, label=name)
    print(name, worst)


# Batched decode (NCNN page section 5: branches decode from clones of one
# context): cloned states share the prompt's full pages, each row sits at its
# own position (branch b first takes b single steps), and the batch steps run
# through the layer-by-layer batch path. Every row must match the oracle's
# independent decode of that branch.
BATCH = {
    # D=64: rows straddle the 256-position attention split and page ends
    "d64_g2_b5": (MID["d64_g2"][0], 250, 17, 100, 5, 6),
    # GQA 4, fp32 weights (vector GEMM path)
    "d32_g4_f32_b3": (MID["d32_g4_f32"][0], 45, 3, 9, 3, 4),
    # D=128 (0.6B head geometry), the full batch of 16 rows
    "d128_g2_b16": (MID["d128_g2"][0], 77, 8, 20, 16, 3),
    # 300-token prompt: 8 clones whose first 18 pages are shared, attention
    # over three 128-position splits (the last one partial)
    "d128_g2_b8_shared": (MID["d128_g2"][0], 300, 8, 20, 8, 4),
}


@pytest.mark.parametrize("name", sorted(BATCH))
def test_decode_batch_rows(name):
    from qwen3_kv_cache_amd import qdec
    from .gpu_harness import torch_dev
    shape, T, a0, La, B, n = BATCH[name]
    W, ids, audio, a0, _ = mid_workload(shape, 13, T, a0, La, 1)
    pre = [synth.random_ids(300 + b, b, shape.vocab) for b in range(B)]      # single steps before the batch
    feed = np.stack([synth.random_ids(400 + b, n, shape.vocab) for b in range(B)])  # [B, n] batch tokens
    orc = oracle.Qwen3Oracle(oracle.OracleConfig.from_shape(shape), W.f32)
    st0 = orc.new_state()
    orc.prefill(st0, ids, audio, a0)
    ref = np.zeros((n, B, shape.vocab))
    for b in range(B):
        sb = st0.clone()
        for j, tok in enumerate(pre[b]):
            orc.decode(sb, int(tok), T + j)
        for s in range(n):
            ref[s, b] = orc.decode(sb, int(feed[b, s]), T + len(pre[b]) + s)
    torch, dev = torch_dev()
    m = device_model(shape, W)
    try:
        base = qdec.qdec_state_create(m.handle, T + B + n)
        audio_d = torch.from_numpy(audio).to(dev)
        qdec.qdec_prefill(base, ids, T, audio_d.data_ptr(), a0, len(audio), None, None)
        branches = [qdec.qdec_clone_state(base) for _ in range(B)]
        qdec.qdec_state_destroy(base)
        scratch = torch.zeros(shape.vocab, dtype=torch.float32, device=dev)
        for b in range(B):
            for j, tok in enumerate(pre[b]):
                qdec.qdec_decode_step(branches[b], int(tok), T + j, scratch.data_ptr(), None)
        logits = torch.full((n, B, shape.vocab), float("nan"), dtype=torch.float32, device=dev)
        amax = torch.full((n, B), -1, dtype=torch.int32, device=dev)
        print(f"[{name}] batch of {B} rows at positions {T}..{T + B - 1}, {n} steps", flush=True)
        for s in range(n):
            qdec.qdec_decode_batch(branches, feed[:, s], logits[s].data_ptr(), amax[s].data_ptr())
        torch.cuda.synchronize()
        for b, st in enumerate(branches):
            assert qdec.qdec_state_pos(st) == T + b + n
            qdec.qdec_state_destroy(st)
    finally:
        m.close()
    L, A = logits.cpu().numpy(), amax.cpu().numpy()
    for b in range(B):
        check_steps(L[:, b], A[:, b], ref[:, b], fp32=not shape.bf16, label=f"{name} row {b}")


def test_decode_at_the_position_limit():
    """The tiny fp32 decoder prefilled with 16381 tokens, then teacher-forced
    decode steps at positions 16381, 16382 and 16383 (the last one the decode
    kernel's in-LDS page table covers, QDEC_DECODE_MAX_POS - 1), against the
    oracle's stored logits (tests/golden/teacher_tiny_maxpos.npz, written by
    make_teacher.py; every vocabulary entry is stored): fp32 bar 1e-4 and the
    same argmax. The next position is rejected with QDEC_E_CAPACITY."""
    import os

    from qwen3_kv_cache_amd import qdec
    from .gpu_harness import torch_dev
    w = synth.WORKLOADS["tiny_maxpos"]
    z = np.load(os.path.join(os.path.dirname(__file__), "golden", "teacher_tiny_maxpos.npz"))
    assert w.prompt_len + w.n_decode == 16384  # QDEC_DECODE_MAX_POS in include/qdec.h
    V = w.shape.vocab
    assert np.array_equal(z["sample_idx"], np.arange(V))
    W = synth.make_weights(w.shape, w.weight_seed)
    ids, audio, a0 = synth.make_prompt(w)
    T = len(ids)
    torch, dev = torch_dev()
    m = device_model(w.shape, W)
    st = qdec.qdec_state_create(m.handle, w.max_ctx)
    try:
        lg = torch.full((w.n_decode + 1, V), float("nan"), dtype=torch.float32, device=dev)
        am = torch.full((w.n_decode + 1,), -1, dtype=torch.int32, device=dev)
        audio_d = torch.from_numpy(audio).to(dev)
        print(f"[maxpos] prefill {T} tokens", flush=True)
        qdec.qdec_prefill(st, ids, T, audio_d.data_ptr(), a0, len(audio), lg[0].data_ptr(), am[0].data_ptr())
        for s in range(w.n_decode):
            qdec.qdec_decode_step(st, int(z["tokens"][s]), T + s, lg[s + 1].data_ptr(), am[s + 1].data_ptr())
        with pytest.raises(qdec.QdecError) as e:
            qdec.qdec_decode_step(st, int(z["tokens"][w.n_decode]), T + w.n_decode)
        assert e.value.code == qdec.QDEC_E_CAPACITY
        torch.cuda.synchronize()
        got = lg.cpu().numpy()
        amax = am.cpu().numpy()
    finally:
        qdec.qdec_state_destroy(st)
        m.close()
    err = float(np.max(np.abs(got - z["sample_vals"])))
    print(f"[maxpos] positions {T}..{T + w.n_decode - 1}: max abs {err:.3g}", flush=True)
    assert err <= 1e-4, err
    assert list(amax) == list(z["tokens"])
