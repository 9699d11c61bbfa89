"""qdec_sample_noalloc (include/qdec.h), the sampling entry point that
allocates nothing, against qdec_sample: two calls in a row on the fixed
scratch, the second with a smaller input, must pick the same token ids as
qdec_sample on the same logits, history, options and uniforms (and the
oracle's picks). The first call changes no device allocation."""
import numpy as np
import pytest

import synth
from oracle.sampling import SamplingParams, boundary_margin, sample

from .gpu_harness import device_model, torch_dev

pytestmark = pytest.mark.gpu


def _inputs(z, hist, n, torch, dev):
    return torch.from_numpy(z).to(dev), torch.from_numpy(hist).to(dev), torch.full((n,), -1, dtype=torch.int32,
                                                                                      device=dev)


def _pick(fn, m, bufs, n, params, nh, u, torch):
    zd, hd, out = bufs
    fn(m.handle, zd.data_ptr(), n, params.temperature, params.top_k, params.top_p, params.repetition_penalty,
       hd.data_ptr() if nh else None, nh, u, out.data_ptr())
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_sample_noalloc_matches_sample():
    from qwen3_kv_cache_amd import qdec
    torch, dev = torch_dev()
    V = 151936
    shape = synth.custom_shape(hidden=64, n_layer=1, n_q_head=2, n_kv_head=1, head_dim=32, ffn=64, vocab=V, bf16=True)
    m = device_model(shape, synth.make_weights(shape, 9))
    rng = np.random.default_rng(77)
    try:
        calls = [(16, SamplingParams(temperature=1.0, top_k=128, top_p=0.9, repetition_penalty=1.2), 40),
                 (3, SamplingParams(temperature=0.7, top_k=20, top_p=0.8, repetition_penalty=1.1), 5)]
        for i, (n, params, nh) in enumerate(calls):
            z = (3.0 * rng.standard_normal((n, V))).astype(np.float32)
            hist = rng.integers(0, V, size=(n, nh)).astype(np.int32)
            u = rng.random(n).astype(np.float32)
            print(f"[noalloc] call {i}: {n} rows, top_k {params.top_k}, history {nh}", flush=True)
            bufs = _inputs(z, hist, n, torch, dev)
            torch.cuda.synchronize()
            free0 = torch.cuda.mem_get_info(dev)[0]
            got = _pick(qdec.qdec_sample_noalloc, m, bufs, n, params, nh, u, torch)
            assert torch.cuda.mem_get_info(dev)[0] == free0, "qdec_sample_noalloc changed device allocations"
            ref = _pick(qdec.qdec_sample, m, bufs, n, params, nh, u, torch)
            assert np.array_equal(got, ref), f"call {i}: {got} != qdec_sample {ref}"
            for r in range(n):
                h = hist[r].tolist()
                want = sample(z[r], params, float(u[r]), h)
                assert got[r] == want or boundary_margin(z[r], params, float(u[r]), h) < 1e-9, (i, r, got[r], want)
        # greedy with the penalty, one row
        z = (3.0 * rng.standard_normal((1, V))).astype(np.float32)
        hist = np.array([[int(np.argmax(z[0]))]], np.int32)
        params = SamplingParams(temperature=0.0, top_k=0, top_p=1.0, repetition_penalty=1.5)
        got = _pick(qdec.qdec_sample_noalloc, m, _inputs(z, hist, 1, torch, dev), 1, params, 1,
                    np.zeros(1, np.float32), torch)
        assert got[0] == sample(z[0], params, 0.0, hist[0].tolist())
    finally:
        m.close()


def test_sample_noalloc_rejects_a_larger_vocabulary():
    from qwen3_kv_cache_amd import qdec
    torch, dev = torch_dev()
    V = qdec.QDEC_SAMPLE_NOALLOC_MAX_VOCAB + 1024
    shape = synth.custom_shape(hidden=64, n_layer=1, n_q_head=2, n_kv_head=1, head_dim=32, ffn=64, vocab=V, bf16=True)
    m = device_model(shape, synth.make_weights(shape, 10))
    try:
        z = torch.zeros((1, V), dtype=torch.float32, device=dev)
        out = torch.zeros(1, dtype=torch.int32, device=dev)
        with pytest.raises(qdec.QdecError) as e:
            qdec.qdec_sample_noalloc(m.handle, z.data_ptr(), 1, 0.0, 0, 1.0, 1.0, None, 0, np.zeros(1, np.float32),
                                     out.data_ptr())
        assert e.value.code == qdec.QDEC_E_INVALID
    finally:
        m.close()
