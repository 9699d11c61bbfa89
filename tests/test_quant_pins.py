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


def _block(amax_bits, w_bits):
    """One block whose largest magnitude and second entry are the given float32 bit patterns."""
    w = np.zeros((1, BLOCK), np.float32)
    w[0, 0] = np.uint32(amax_bits).view(np.float32)
    w[0, 1] = np.uint32(w_bits).view(np.float32)
    return w


def test_rounding_is_of_the_float32_quotient():
    # Blocks where w / d (one float32 division) and w * (1 / d) (a rounded
    # reciprocal, then a product) land on opposite sides of a half-integer, so
    # the two readings give different codes. The reading taken is w / d.
    # amax 0.0445032, w 0.0022777228: w / d = 6.4999995 -> 6 (w * (1/d) = 6.5 -> 7)
    q, _ = quantize(_block(1026967805, 991249881))
    assert q[0, 1] == 6
    # amax 0.014388194, w 0.00062311074: w / d = 5.5 -> 6 (w * (1/d) = 5.4999995 -> 5)
    q, _ = quantize(_block(1013693558, 975394881))
    assert q[0, 1] == 6
    q, _ = quantize(-_block(1013693558, 975394881))
    assert q[0, 1] == -6  # half away from zero on both sides


def test_rounding_below_one_half():
    # amax 127 gives d = 1 exactly, so q = round(w). The float32 just below 0.5
    # rounds to 0: adding 0.5 to it in float32 would round up to 1.0.
    w = np.zeros((1, BLOCK), np.float32)
    w[0, :8] = [127.0, np.nextafter(np.float32(0.5), np.float32(0)), 0.5, -0.5, 1.5, -2.5, 126.5, -126.49999]
    q, d = quantize(w)
    assert float(d[0, 0]) == 1.0
    assert q[0, :8].tolist() == [127, 0, 1, -1, 2, -3, 127, -126]


def test_width_must_be_whole_blocks():
    with pytest.raises(ValueError):
        quantize(np.zeros((2, 40), np.float32))


def test_pins_catch_planted_rounding_mistakes():
    # the two readings the pins above separate, planted in a copy of the
    # oracle's source: each must fail its pin
    import inspect

    import oracle.quant as qmod
    src = inspect.getsource(qmod)
    planted = {
        "reciprocal product": ("x = (blocks / safe[:, :, None]).astype(np.float32)",
                               "x = (blocks * (np.float32(1.0) / safe)[:, :, None]).astype(np.float32)",
                               test_rounding_is_of_the_float32_quotient),
        "float32 half add": ("q = np.sign(x) * np.floor(np.abs(x) + 0.5)",
                             "x = x.astype(np.float32); q = np.sign(x) * np.floor(np.abs(x) + np.float32(0.5))",
                             test_rounding_below_one_half),
    }
    global quantize
    original = quantize
    try:
        for name, (old, new, pin) in planted.items():
            assert old in src, name
            ns = {}
            exec(compile(src.replace(old, new), f"<planted {name}>", "exec"), ns)
            quantize = ns["quantize"]
            with pytest.raises(AssertionError):
                pin()
    finally:
        quantize = original


def test_block_bytes_hand_example():
    # one row of two blocks: d = 1.0 (fp16 0x3C00) over codes 0..31, then
    # d = -0.5 (fp16 0xB800) over codes -1, -128 + 1, 127, 0, ...; bytes are
    # the scale little-endian, then the codes as two's complement bytes
    import synth
    q = np.zeros((1, 2 * BLOCK), np.int8)
    q[0, :BLOCK] = np.arange(BLOCK)
    q[0, BLOCK:BLOCK + 3] = [-1, -127, 127]
    d = np.array([[1.0, -0.5]], np.float16)
    b = synth.pack_q8_blocks(q, d)
    assert b.dtype == np.uint8 and b.shape == (1, 2 * synth.Q8_BLOCK_BYTES)
    assert b[0, :2].tolist() == [0x00, 0x3C]
    assert b[0, 2:34].tolist() == list(range(BLOCK))
    assert b[0, 34:36].tolist() == [0x00, 0xB8]
    assert b[0, 36:39].tolist() == [0xFF, 0x81, 0x7F]
    assert np.all(b[0, 39:] == 0)


def test_blocks_parse_back_and_dequantize_to_the_product():
    # reading the bytes back (scale, then codes, per 34-byte block) recovers
    # the codes and scales, and the oracle's weights are q * d elementwise
    import synth
    Q = synth.make_q8_weights(synth.custom_shape(hidden=128, n_layer=1, n_q_head=2, n_kv_head=1, head_dim=64,
                                                 ffn=256, vocab=50), 3)
    for name in ("embed", "L0.wo", "L0.w_down"):
        q, d, b = Q.codes[name], Q.scales[name], Q.blocks[name]
        out, n = q.shape
        blk = b.reshape(out, n // BLOCK, 34)
        d_back = blk[:, :, :2].copy().view("<f2").reshape(out, n // BLOCK)
        q_back = blk[:, :, 2:].copy().view(np.int8).reshape(out, n)
        np.testing.assert_array_equal(d_back, d)
        np.testing.assert_array_equal(q_back, q)
        w = dequantize(q_back, d_back)
        for r, c in [(0, 0), (out - 1, n - 1), (out // 2, 37)]:
            assert w[r, c] == np.float32(q[r, c]) * np.float32(d[r, c // BLOCK])
    assert all(float(Q.scales[k].min()) > 0 for k in Q.scales)
