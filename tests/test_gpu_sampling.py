"""GPU parity of the sampling step (qdec_sample) against the oracle
(NCNN page "Qwen3ASR ncnn多平台移植", sections 1 and 6): same logits, history,
options and uniforms must give the same token ids. A pick whose uniform lies
within 1e-9 of a cumulative boundary (where float64 sums in another order
may decide differently) is reported and skipped; there are none in practice."""
import numpy as np
import pytest

import synth
from oracle.sampling import SamplingParams, boundary_margin, sample

from .gpu_harness import device_model, torch_dev

pytestmark = pytest.mark.gpu

CASES = [
    # temperature, top_k, top_p, repetition penalty, history length
    (0.0, 0, 1.0, 1.0, 0),
    (0.0, 0, 1.0, 1.3, 24),
    (1.0, 1, 1.0, 1.0, 0),
    (0.8, 50, 1.0, 1.0, 0),
    (1.0, 128, 0.9, 1.2, 40),
    (0.6, 40, 0.5, 1.1, 8),
    (1.7, 17, 0.95, 0.8, 100),
]


@pytest.mark.parametrize("vocab", [151936, 5003, 1000])
def test_sample_matches_oracle(vocab):
    from qwen3_kv_cache_amd import qdec
    torch, dev = torch_dev()
    shape = synth.custom_shape(hidden=64, n_layer=1, n_q_head=2, n_kv_head=1, head_dim=32, ffn=64, vocab=vocab,
                               bf16=True)
    W = synth.make_weights(shape, 3)
    m = device_model(shape, W)
    rng = np.random.default_rng(vocab)
    n = 16
    skipped = 0
    try:
        for ci, (T, k, p, rho, nh) in enumerate(CASES):
            params = SamplingParams(temperature=T, top_k=k, top_p=p, repetition_penalty=rho)
            for rep in range(2):
                z = (3.0 * rng.standard_normal((n, vocab))).astype(np.float32)
                # a few exact ties, to exercise the index tie-break
                z[:, 7] = z[:, 3]
                hist = rng.integers(-2, vocab + 2, size=(n, max(nh, 1))).astype(np.int32)
                hist[:, 0] = int(np.argmax(z[0]))  # the best token is often in the history
                u = rng.random(n).astype(np.float32)
                zd = torch.from_numpy(z).to(dev)
                hd = torch.from_numpy(hist).to(dev)
                out = torch.full((n,), -1, dtype=torch.int32, device=dev)
                print(f"[sample V={vocab}] case {ci} rep {rep}: T={T} k={k} p={p} rho={rho} nh={nh}", flush=True)
                qdec.qdec_sample(m.handle, zd.data_ptr(), n, T, k, p, rho, hd.data_ptr() if nh else None, nh, u,
                                 out.data_ptr())
                torch.cuda.synchronize()
                got = out.cpu().numpy()
                for r in range(n):
                    h = hist[r, :nh].tolist()
                    want = sample(z[r], params, float(u[r]), h)
                    if got[r] != want and boundary_margin(z[r], params, float(u[r]), h) < 1e-9:
                        skipped += 1
                        continue
                    assert got[r] == want, f"V={vocab} case {ci} row {r}: gpu {got[r]} != oracle {want}"
    finally:
        m.close()
    print(f"[sample V={vocab}] boundary cases skipped: {skipped}")
