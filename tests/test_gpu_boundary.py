"""GPU tests of boundary paths (include/qdec.h) against the oracle, at a
shape the float64 oracle runs in seconds (the 0.6B head geometry: D=128,
GQA 2; hidden 512, 3 layers):

* qdec_decode_step_dev fed the previous step's device argmax (NCNN page
  section 5, greedy loop without a host round trip), and token_dev values
  outside [0, vocab) clamped on the device;
* a source state that keeps decoding beside its clone (section 5: branches
  from one context; the clone shares full pages and copies the tail page);
* the decode kernel's device-scope exchange form (QDEC_EXCHANGE_SCOPE=device)
  giving the same bits as the default form.
"""
import os

import numpy as np
import pytest

import oracle
import synth

from .gpu_harness import check_steps, device_model, mid_workload, torch_dev

pytestmark = pytest.mark.gpu

SHAPE = synth.custom_shape(hidden=512, n_layer=3, n_q_head=8, n_kv_head=4, head_dim=128, ffn=1536, vocab=4099,
                           bf16=True)


def setup(seed, T=40, a0=8, La=12):
    W, ids, audio, a0, _ = mid_workload(SHAPE, seed, T, a0, La, 1)
    orc = oracle.Qwen3Oracle(oracle.OracleConfig.from_shape(SHAPE), W.f32)
    return W, ids, audio, a0, orc


def test_decode_step_dev_feeds_argmax_and_clamps():
    from qwen3_kv_cache_amd import qdec
    torch, dev = torch_dev()
    W, ids, audio, a0, orc = setup(31)
    T, V, n = len(ids), SHAPE.vocab, 10
    toks, ref = oracle.greedy_trajectory(orc, ids, audio, a0, n)
    m = device_model(SHAPE, W)
    try:
        st = qdec.qdec_state_create(m.handle, T + n + 2)
        lg = torch.full((n + 3, V), float("nan"), dtype=torch.float32, device=dev)
        am = torch.full((n + 3,), -1, dtype=torch.int32, device=dev)
        audio_d = torch.from_numpy(audio).to(dev)
        qdec.qdec_prefill(st, ids, T, audio_d.data_ptr(), a0, len(audio), lg[0].data_ptr(), am[0].data_ptr())
        print(f"[step_dev] {n} device-fed steps from pos {T}", flush=True)
        for s in range(n):
            qdec.qdec_decode_step_dev(st, am[s].data_ptr(), T + s, lg[s + 1].data_ptr(), am[s + 1].data_ptr())
        # out-of-range device tokens: V + 5 is clamped to V - 1, -3 to 0
        bad = torch.tensor([V + 5, -3], dtype=torch.int32, device=dev)
        qdec.qdec_decode_step_dev(st, bad[0].data_ptr(), T + n, lg[n + 1].data_ptr(), am[n + 1].data_ptr())
        qdec.qdec_decode_step_dev(st, bad[1].data_ptr(), T + n + 1, lg[n + 2].data_ptr(), am[n + 2].data_ptr())
        torch.cuda.synchronize()
        qdec.qdec_model_status(m.handle)
        assert qdec.qdec_state_pos(st) == T + n + 2
        qdec.qdec_state_destroy(st)
    finally:
        m.close()
    got = am.cpu().numpy()
    assert list(got[:n + 1]) == list(toks), f"device-fed tokens {got[:n + 1]} != oracle {toks}"
    # after the chain the kernel consumed the clamped V - 1, then 0
    ost = orc.new_state()
    orc.prefill(ost, ids, audio, a0)
    for s in range(n):
        orc.decode(ost, int(toks[s]), T + s)
    ref_c = np.stack([orc.decode(ost, V - 1, T + n), orc.decode(ost, 0, T + n + 1)])
    L = lg.cpu().numpy()
    check_steps(L[:n + 1], got[:n + 1], ref, fp32=False, label="step_dev chain")
    check_steps(L[n + 1:], got[n + 1:], ref_c, fp32=False, label="step_dev clamped")


def test_clone_source_keeps_decoding():
    from qwen3_kv_cache_amd import qdec
    torch, dev = torch_dev()
    W, ids, audio, a0, orc = setup(37, T=45)  # 45 positions: a partly filled tail page at the clone
    T, V, n = len(ids), SHAPE.vocab, 6
    sa = synth.random_ids(601, n, V)
    sb = synth.random_ids(602, n, V)
    ost = orc.new_state()
    orc.prefill(ost, ids, audio, a0)
    oc = ost.clone()
    ref_a, ref_b = [], []
    for s in range(n):
        ref_a.append(orc.decode(ost, int(sa[s]), T + s))
        ref_b.append(orc.decode(oc, int(sb[s]), T + s))
    m = device_model(SHAPE, W)
    try:
        src = qdec.qdec_state_create(m.handle, T + n)
        audio_d = torch.from_numpy(audio).to(dev)
        qdec.qdec_prefill(src, ids, T, audio_d.data_ptr(), a0, len(audio), None, None)
        cl = qdec.qdec_clone_state(src)
        la = torch.full((n, V), float("nan"), dtype=torch.float32, device=dev)
        lb = torch.full((n, V), float("nan"), dtype=torch.float32, device=dev)
        aa = torch.full((n,), -1, dtype=torch.int32, device=dev)
        ab = torch.full((n,), -1, dtype=torch.int32, device=dev)
        print(f"[clone] source and clone interleaved from pos {T}", flush=True)
        for s in range(n):  # interleaved: the source writes its tail page while the clone reads its copy
            qdec.qdec_decode_step(src, int(sa[s]), T + s, la[s].data_ptr(), aa[s].data_ptr())
            qdec.qdec_decode_step(cl, int(sb[s]), T + s, lb[s].data_ptr(), ab[s].data_ptr())
        torch.cuda.synchronize()
        qdec.qdec_model_status(m.handle)
        qdec.qdec_state_destroy(src)  # either may be destroyed first
        qdec.qdec_state_destroy(cl)
    finally:
        m.close()
    check_steps(la.cpu().numpy(), aa.cpu().numpy(), np.stack(ref_a), fp32=False, label="clone source")
    check_steps(lb.cpu().numpy(), ab.cpu().numpy(), np.stack(ref_b), fp32=False, label="clone")


def test_exchange_scope_device_matches_default():
    """The decode kernel with every exchange word at device scope (the form
    used when the XCD placement check fails) gives the same bits as the
    default, group-local form, through a 70-step greedy launch that crosses
    the 64-position boundary where the attention splits over ranks."""
    from qwen3_kv_cache_amd import qdec
    torch, dev = torch_dev()
    W, ids, audio, a0, orc = setup(41)
    T, V, n = len(ids), SHAPE.vocab, 70
    outs = []
    for scope in (None, "device"):
        if scope:
            os.environ["QDEC_EXCHANGE_SCOPE"] = scope
        try:
            m = device_model(SHAPE, W)
        finally:
            os.environ.pop("QDEC_EXCHANGE_SCOPE", None)
        try:
            st = qdec.qdec_state_create(m.handle, T + n)
            lg = torch.full((n + 1, V), float("nan"), dtype=torch.float32, device=dev)
            tk = torch.full((n + 1,), -1, dtype=torch.int32, device=dev)
            audio_d = torch.from_numpy(audio).to(dev)
            qdec.qdec_prefill(st, ids, T, audio_d.data_ptr(), a0, len(audio), lg[0].data_ptr(), tk[0].data_ptr())
            print(f"[scope {scope or 'default'}] greedy {n} steps", flush=True)
            qdec.qdec_decode_greedy(st, tk[0].data_ptr(), T, n, lg[1].data_ptr(), tk[1].data_ptr())
            torch.cuda.synchronize()
            qdec.qdec_model_status(m.handle)
            qdec.qdec_state_destroy(st)
        finally:
            m.close()
        outs.append((lg.cpu().numpy(), tk.cpu().numpy()))
    (l1, t1), (l2, t2) = outs
    assert np.array_equal(t1, t2)
    assert np.array_equal(l1.view(np.uint32), l2.view(np.uint32)), "device-scope exchange changed the logits"
    toks, ref = oracle.greedy_trajectory(orc, ids, audio, a0, n)
    assert list(t1) == list(toks)
    check_steps(l1, t1, ref, fp32=False, label="exchange scope")
