"""Pins of the block-int8 (Q8_0) oracle: hand-worked blocks, the bounds and
fixed points the definition implies, and exactness of the dequantized weights."""
import numpy as np
import pytest

from oracle.quant import BLOCK, dequantize, quantize


def test_hand_block():
    # amax 2.54 -> d = 0.02; w / d = 127, -63.5 (half away from zero: -64), 0.25 -> 0 ...
    w = np.zeros((1, BLOCK), np.float32)
    w[0, :4] = [2.54, -1.27, 0.005, 0.015]
    q, d = quantize(w)
    assert d.dtype == np.float16 and d.shape == (1, 1)
    assert float(d[0, 0]) == float(np.float16(np.float32(2.54) / np.float32(127)))
    assert q[0, :4].tolist() == [127, -64, 0, 1]  # 0.015 / 0.02 = 0.75 -> 1
    assert np.all(q[0, 4:] == 0)


def test_zero_block_and_sign():
    w = np.zeros((2, 2 * BLOCK), np.float32)
    w[1, BLOCK:] = -np.linspace(0.0, 1.0, BLOCK, dtype=np.float32)
    q, d = quantize(w)
    assert np.all(q[0] == 0) and float(d[0, 0]) == 0.0 and float(d[0, 1]) == 0.0
    assert q[1, -1] == -127  # the block's extreme maps to -127
    assert np.all(q[1, BLOCK:] <= 0)


def test_error_bound_and_range():
    rng = np.random.default_rng(3)
    w = (0.02 * rng.standard_normal((64, 256))).astype(np.float32)
    q, d = quantize(w)
    assert q.dtype == np.int8 and np.abs(q.astype(int)).max() <= 127
    wd = dequantize(q, d)
    # |w - q d16| <= d32 / 2 (rounding) + 127 |d32 - d16| (scale rounding to fp16)
    d32 = (np.abs(w.reshape(64, 8, BLOCK)).max(axis=2) / np.float32(127)).astype(np.float64)
    d16 = d.astype(np.float64)
    bound = d32 / 2 + 127 * np.abs(d32 - d16) + 1e-12
    err = np.abs(w.reshape(64, 8, BLOCK).astype(np.float64) - wd.reshape(64, 8, BLOCK).astype(np.float64))
    assert np.all(err <= bound[:, :, None])
    # relative to the block scale the error is about half a step
    assert float(err.max() / d32.max()) < 0.6


def test_dequantized_is_exact_product():
    rng = np.random.default_rng(4)
    q = rng.integers(-127, 128, size=(3, 64)).astype(np.int8)
    d = (np.abs(rng.standard_normal((3, 2))) * 0.01).astype(np.float16)
    wd = dequantize(q, d)
    # q * d in float64 equals the float32 product: 8 x 11 significant bits fit in 24
    ref = q.reshape(3, 2, BLOCK).astype(np.float64) * d.astype(np.float64)[:, :, None]
    np.testing.assert_array_equal(wd.reshape(3, 2, BLOCK).astype(np.float64), ref)


def test_requantizing_dequantized_weights_is_a_fixed_point():
    rng = np.random.default_rng(5)
    w = (0.02 * rng.standard_normal((8, 128))).astype(np.float32)
    q, d = quantize(w)
    q2, d2 = quantize(dequantize(q, d))
    # blocks whose extreme is +-127 keep their scale and codes exactly
    np.testing.assert_array_equal(d2, d)
    np.testing.assert_array_equal(q2, q)


def test_width_must_be_whole_blocks():
    with pytest.raises(ValueError):
        quantize(np.zeros((2, 40), np.float32))
