"""GPU parity of the audio adaptor (transcribe.cpp "Forward map - funasr_nano",
section "Adaptor") against the float64 oracle, and of the adaptor feeding the
decoder's audio span.

Tolerance: the GEMMs take fp32 activations as bf16 hi + lo against exact bf16
weights, and the attention three bf16 products per fp32 product, so every
product keeps about 16 mantissa bits (relative error near 2^-16 = 1.5e-5),
summed in fp32; errors of independent terms partly cancel. Outputs are of
unit scale (LayerNorm inputs, residual rows of magnitude ~1), so the bar is
max |gpu - oracle| <= 1e-4 and a relative L2 error <= 5e-5 over the output
(measured: about 1e-5 and 5e-6)."""
import numpy as np
import pytest

import oracle
import synth
from oracle.adaptor import AdaptorConfig, adaptor

from .gpu_harness import device_model, torch_dev

pytestmark = pytest.mark.gpu

FULL = synth.AdaptorShape()
# two heads of 128, small widths: T <= 64 takes the small-M GEMM, 300 the tiled one
SMALL = synth.AdaptorShape(enc_dim=64, mid_dim=256, dim=256, ffn_dim=128, n_block=2, n_head=2)


def _cfg(s):
    return AdaptorConfig(s.enc_dim, s.mid_dim, s.dim, s.ffn_dim, s.n_block, s.n_head, 1e-12)


def _check(got, ref, label):
    err = float(np.max(np.abs(got - ref)))
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    print(f"[{label}] max abs {err:.3g} rel L2 {rel:.3g}", flush=True)
    assert np.all(np.isfinite(got)), label
    assert err <= 1e-4, (label, err)
    assert rel <= 5e-5, (label, rel)


@pytest.mark.parametrize("shape,T,seed", [(SMALL, 1, 21), (SMALL, 37, 22), (SMALL, 300, 23), (FULL, 183, 24),
                                          (FULL, 2100, 25)], ids=["small_T1", "small_T37", "small_T300",
                                                                   "full_T183", "full_T2100"])
def test_adaptor_matches_oracle(shape, T, seed):
    from qwen3_kv_cache_amd.device import Adaptor
    torch, dev = torch_dev()
    f32, bits = synth.make_adaptor_weights(shape, seed)
    frames = synth.encoder_frames(seed, T, shape.enc_dim)
    ref = adaptor(frames, f32, _cfg(shape))
    print(f"[adaptor] dims {shape} T {T}", flush=True)
    a = Adaptor(shape, bits)
    try:
        out = a.run(torch.from_numpy(frames).to(dev))
        # a second call on a shorter input reuses the scratch
        out2 = a.run(torch.from_numpy(frames[: max(1, T // 2)]).to(dev))
        torch.cuda.synchronize()
    finally:
        a.close()
    _check(out.cpu().numpy(), ref, f"adaptor T={T}")
    _check(out2.cpu().numpy(), adaptor(frames[: max(1, T // 2)], f32, _cfg(shape)), f"adaptor T={max(1, T // 2)}")


def test_adaptor_rows_drive_the_decoder():
    """183 encoder frames -> adaptor -> the first 23 rows as the audio span of
    a 48-token prompt -> prefill logits, against oracle adaptor + oracle
    decoder (the page's example: 183 frames, 23 kept)."""
    from qwen3_kv_cache_amd import qdec
    from qwen3_kv_cache_amd.device import Adaptor
    torch, dev = torch_dev()
    f32, bits = synth.make_adaptor_weights(FULL, 26)
    frames = synth.encoder_frames(26, 183, FULL.enc_dim)
    rows_ref = adaptor(frames, f32, _cfg(FULL))[:23]
    w = synth.WORKLOADS["short"]
    W = synth.make_weights(w.shape, w.weight_seed)
    ids, _, a0 = synth.make_prompt(w)
    orc = oracle.Qwen3Oracle(oracle.OracleConfig.from_shape(w.shape), W.f32)
    ref = orc.prefill(orc.new_state(), ids, rows_ref.astype(np.float64), a0)
    a = Adaptor(FULL, bits)
    m = device_model(w.shape, W)
    st = qdec.qdec_state_create(m.handle, len(ids))
    try:
        rows = a.run(torch.from_numpy(frames).to(dev))
        lg = torch.full((w.shape.vocab,), float("nan"), dtype=torch.float32, device=dev)
        am = torch.full((1,), -1, dtype=torch.int32, device=dev)
        qdec.qdec_prefill(st, ids, len(ids), rows.data_ptr(), a0, 23, lg.data_ptr(), am.data_ptr())
        torch.cuda.synchronize()
        got = lg.cpu().numpy()
        tok = int(am.cpu().numpy()[0])
    finally:
        qdec.qdec_state_destroy(st)
        m.close()
        a.close()
    err = float(np.max(np.abs(got - ref)))
    cos = float(np.dot(got, ref) / (np.linalg.norm(got) * np.linalg.norm(ref)))
    print(f"[adaptor->decoder] logits max abs {err:.3g} cos {cos:.7f}", flush=True)
    assert err <= 5e-2 and cos >= 0.9999, (err, cos)
    assert tok == oracle.pick_token(ref)


def test_adaptor_rejects_overlapping_output():
    from qwen3_kv_cache_amd import qdec
    from qwen3_kv_cache_amd.device import Adaptor
    torch, dev = torch_dev()
    _, bits = synth.make_adaptor_weights(SMALL, 27)
    a = Adaptor(SMALL, bits)
    try:
        buf = torch.zeros((8, max(SMALL.enc_dim, SMALL.dim)), dtype=torch.float32, device=dev)
        with pytest.raises(qdec.QdecError) as e:
            qdec.qdec_adaptor_run(a.handle, buf.data_ptr(), 4, buf.data_ptr() + 4 * SMALL.enc_dim)
        assert e.value.code == qdec.QDEC_E_INVALID
        with pytest.raises(qdec.QdecError) as e:
            qdec.qdec_adaptor_run(a.handle, buf.data_ptr(), 0, buf.data_ptr())
        assert e.value.code == qdec.QDEC_E_INVALID
    finally:
        a.close()
