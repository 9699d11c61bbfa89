"""Host-side checks of bench.py's work model (no GPU)."""
import os
import sys
from types import SimpleNamespace

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _count_prefill_flops(s, T):
    """Multiply-adds counted one by one: every weight of every projection once
    per row, every (query head, key <= query) pair twice (QK and PV) over D,
    and the LM head on the last row; 2 FLOPs each."""
    macs = 0
    per_row = 0
    for n_out, n_in in ((s.n_q_head * s.head_dim, s.hidden), (s.n_kv_head * s.head_dim, s.hidden),
                        (s.n_kv_head * s.head_dim, s.hidden), (s.hidden, s.n_q_head * s.head_dim),
                        (s.ffn, s.hidden), (s.ffn, s.hidden), (s.hidden, s.ffn)):
        per_row += n_out * n_in
    for _layer in range(s.n_layer):
        macs += per_row * T
        for t in range(T):
            for _u in range(t + 1):
                macs += s.n_q_head * 2 * s.head_dim
    macs += s.vocab * s.hidden
    return 2 * macs


def test_prefill_flops_counted():
    s = SimpleNamespace(hidden=64, n_layer=2, head_dim=16, n_q_head=4, n_kv_head=2, ffn=96, vocab=300)
    for T in (1, 7, 33):
        assert bench.prefill_flops(s, T) == _count_prefill_flops(s, T)


def test_prefill_flops_qwen3_shape():
    # the per-token projection weights of the 28 blocks: 440,401,920
    s = SimpleNamespace(hidden=1024, n_layer=28, head_dim=128, n_q_head=16, n_kv_head=8, ffn=3072, vocab=151936)
    assert bench.prefill_flops(s, 1) == 2 * 440_401_920 + 28 * 4 * 16 * 128 + 2 * 151936 * 1024
    assert abs(bench.prefill_flops(s, 8192) - 1.4913e13) / 1.4913e13 < 1e-4


def test_adaptor_flops_counted():
    a = SimpleNamespace(enc_dim=16, mid_dim=32, dim=24, ffn_dim=8, n_block=2)
    for T in (1, 5):
        macs = T * (16 * 32 + 32 * 24)
        for _b in range(2):
            macs += T * (4 * 24 * 24 + 24 * 8 + 8 * 24)
            for _t in range(T):
                for _u in range(T):
                    macs += 2 * 24  # one q.k and one p.v per (head dim) summed over heads
        assert bench.adaptor_flops(a, T) == 2 * macs


def test_batch_decode_bytes_survey_figures():
    # the step byte model quoted for 16 clones of a 512-token prefix:
    # about 1.31e9 unique bytes at the first step and 1.78e9 at step 128
    s = SimpleNamespace(hidden=1024, n_layer=28, head_dim=128, n_q_head=16, n_kv_head=8, ffn=3072, vocab=151936)
    u0, q0 = bench.batch_decode_bytes(s, 512, 16, 0)
    u128, q128 = bench.batch_decode_bytes(s, 512, 16, 128)
    assert abs(u0 / 1.31e9 - 1) < 0.01 and abs(u128 / 1.78e9 - 1) < 0.01
    # per sequence every branch re-reads the prefix: 3.07e9 .. 3.54e9 over the run
    assert abs(q0 / 3.07e9 - 1) < 0.01 and abs(q128 / 3.54e9 - 1) < 0.01
    # one branch: unique == per sequence == the single-sequence model at the same context
    u, q = bench.batch_decode_bytes(s, 512, 1, 10)
    assert u == q
    assert abs(u - bench.decode_bytes(s, [523])) < 1.0
