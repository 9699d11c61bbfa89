"""Status codes of the C ABI on a live model (include/qdec.h): every rejected
call returns its code and leaves the state as it was, so the logits of the
calls that follow still match the oracle (tiny fp32 decoder, 1e-4)."""
import numpy as np
import pytest

import oracle
import synth

from .gpu_harness import device_model, torch_dev

pytestmark = pytest.mark.gpu


def _code(fn, *args):
    from qwen3_kv_cache_amd import qdec
    with pytest.raises(qdec.QdecError) as e:
        fn(*args)
    return e.value.code


def test_rejected_calls_leave_the_state_unchanged():
    from qwen3_kv_cache_amd import qdec
    w = synth.WORKLOADS["tiny"]
    W = synth.make_weights(w.shape, w.weight_seed)
    ids, audio, a0 = synth.make_prompt(w)
    T, V = len(ids), w.shape.vocab
    orc = oracle.Qwen3Oracle(oracle.OracleConfig.from_shape(w.shape), W.f32)
    toks, ref = oracle.greedy_trajectory(orc, ids, audio, a0, 2)
    torch, dev = torch_dev()
    m = device_model(w.shape, W)
    st = qdec.qdec_state_create(m.handle, T + 2)
    try:
        audio_d = torch.from_numpy(audio).to(dev)
        lg = torch.full((3, V), float("nan"), dtype=torch.float32, device=dev)
        am = torch.full((3,), -1, dtype=torch.int32, device=dev)
        ap = audio_d.data_ptr()
        print("[lifecycle] prefill rejections", flush=True)
        long_ids = np.concatenate([ids, ids[:3]])
        assert _code(qdec.qdec_prefill, st, long_ids, T + 3, ap, a0, len(audio)) == qdec.QDEC_E_CAPACITY
        assert _code(qdec.qdec_prefill, st, ids, 0, ap, a0, len(audio)) == qdec.QDEC_E_INVALID
        assert _code(qdec.qdec_prefill, st, ids, T, ap, T - 2, 3) == qdec.QDEC_E_INVALID  # span past the prompt
        bad = ids.copy()
        bad[0 if a0 > 0 else T - 1] = V  # a text position (audio positions are ignored)
        assert _code(qdec.qdec_prefill, st, bad, T, ap, a0, len(audio)) == qdec.QDEC_E_INVALID
        assert qdec.qdec_state_pos(st) == 0

        qdec.qdec_prefill(st, ids, T, ap, a0, len(audio), lg[0].data_ptr(), am[0].data_ptr())
        assert qdec.qdec_state_pos(st) == T
        print("[lifecycle] decode rejections", flush=True)
        assert _code(qdec.qdec_prefill, st, ids, T, ap, a0, len(audio)) == qdec.QDEC_E_STATE
        assert _code(qdec.qdec_decode_step, st, int(toks[0]), T + 1) == qdec.QDEC_E_POS
        assert _code(qdec.qdec_decode_step, st, int(toks[0]), T - 1) == qdec.QDEC_E_POS
        assert _code(qdec.qdec_decode_step, st, V, T) == qdec.QDEC_E_INVALID
        assert _code(qdec.qdec_decode_step, st, -1, T) == qdec.QDEC_E_INVALID
        assert qdec.qdec_state_pos(st) == T

        qdec.qdec_decode_step(st, int(toks[0]), T, lg[1].data_ptr(), am[1].data_ptr())
        qdec.qdec_decode_step(st, int(toks[1]), T + 1, lg[2].data_ptr(), am[2].data_ptr())
        assert qdec.qdec_state_pos(st) == T + 2
        # the state is full
        assert _code(qdec.qdec_decode_step, st, int(toks[2]), T + 2) == qdec.QDEC_E_CAPACITY
        assert qdec.qdec_state_pos(st) == T + 2
        # the model cannot go while a state lives
        assert _code(qdec.qdec_destroy, m.handle) == qdec.QDEC_E_STATE
        torch.cuda.synchronize()
        got = lg.cpu().numpy()
        err = float(np.max(np.abs(got - ref)))
        assert err <= 1e-4, f"max |gpu - oracle| = {err}"
        assert list(am.cpu().numpy()) == list(toks[:3])
    finally:
        qdec.qdec_state_destroy(st)
        m.close()
