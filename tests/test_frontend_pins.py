"""Pins of the frontend oracle (oracle/frontend.py) against what the pages and
the mathematics fix: frame counts, the Hamming window's closed form,
Parseval's identity, the spectral peak of a tone, the triangle filters'
partition of unity, exact results for signals that vanish after mean removal,
and the LFR stacking worked by hand. Planted mistakes in a copy of the oracle
must each fail one of them."""
import inspect
import sys

import numpy as np
import pytest

import synth
from oracle import frontend as F

C = F.FrontendConfig()


def test_frame_and_row_counts():
    # 25 ms frames every 10 ms at 16 kHz; LFR keeps ceil(T / 6) rows
    assert [F.n_frames(n) for n in (0, 399, 400, 559, 560, 16000)] == [0, 0, 1, 1, 2, 98]
    assert F.n_lfr_rows(16000) == 17 and F.n_lfr_rows(400) == 1 and F.n_lfr_rows(399) == 0
    assert F.frontend(synth.pcm("voiced", 16000, 3)).shape == (17, 560)


def test_hamming_closed_form():
    w = F.hamming(400)
    assert w[0] == pytest.approx(0.08) and w[399] == pytest.approx(0.08)
    np.testing.assert_allclose(w, w[::-1], atol=1e-15)
    # the peak value 0.54 + 0.46 cos(pi / 399) sits at the two middle samples
    assert w[199] == pytest.approx(0.54 + 0.46 * np.cos(np.pi / 399), abs=1e-15)


def test_parseval_on_the_padded_frame():
    # sum over all 512 bins of |X_k|^2 = 512 sum x^2; with the real input's
    # symmetry the 256 kept bins and the Nyquist bin (sum x (-1)^n)^2 add up to it
    rng = np.random.default_rng(1)
    fr = rng.standard_normal((3, 400))
    p = F.power_spectrum(fr)
    assert p.shape == (3, 256)
    nyq = (fr * (-1.0) ** np.arange(400)).sum(axis=1) ** 2
    total = p[:, 0] + nyq + 2 * p[:, 1:].sum(axis=1)
    np.testing.assert_allclose(total, 512 * (fr ** 2).sum(axis=1), rtol=1e-12)


@pytest.mark.parametrize("k0", [16, 32, 100])
def test_tone_peaks_at_its_bin(k0):
    # a cosine at bin frequency 31.25 k0 Hz: after mean removal, pre-emphasis
    # and the window the power spectrum peaks at bin k0
    t = np.arange(4000) / 16000.0
    x = 5000 * np.cos(2 * np.pi * 31.25 * k0 * t)
    p = F.power_spectrum(F.frame_signal(x))
    assert np.all(np.argmax(p, axis=1) == k0)


def test_mel_scale_and_triangles():
    assert F.mel(700.0) == pytest.approx(1127.0 * np.log(2.0))
    w = F.mel_filters()
    assert w.shape == (80, 256) and w.min() >= 0 and w.max() <= 1
    edges = np.linspace(F.mel(20.0), F.mel(8000.0), 82)
    m = F.mel(np.arange(256) * 31.25)
    # overlapping triangles with shared edges: between two centres the two
    # weights sum to one, and each filter vanishes outside its two neighbours' centres
    for j in range(79):
        between = (m >= edges[j + 1]) & (m <= edges[j + 2])
        np.testing.assert_allclose(w[j, between] + w[j + 1, between], 1.0, atol=1e-12)
    for j in range(80):
        outside = (m <= edges[j]) | (m >= edges[j + 2])
        assert np.all(w[j, outside] == 0)
    # bins below 20 Hz (bin 0) and above the last centre only touch the edge filters
    assert np.all(w[:, 0] == 0)


def test_sine440_energy_peaks_in_the_nearest_filter():
    x = synth.pcm("sine440", 8000)
    fb = F.fbank(x)
    centres = np.linspace(F.mel(20.0), F.mel(8000.0), 82)[1:-1]
    want = int(np.argmin(np.abs(centres - F.mel(440.0))))
    assert np.all(np.argmax(fb, axis=1) == want)


def test_signals_that_vanish_after_mean_removal():
    # silence, and a constant offset, give zero frames: every energy sits at
    # the floor log(eps32); so do the frames of an impulse train's quiet parts
    floor = np.log(2.0 ** -23)
    for x in (synth.pcm("silence", 4000), np.full(4000, 1234.5)):
        fb = F.fbank(x)
        assert fb.shape == (23, 80)
        np.testing.assert_array_equal(fb, floor)
    fb = F.fbank(synth.pcm("impulse", 4000))
    hit = [i for i in range(fb.shape[0]) if i * 160 <= 2000 < i * 160 + 400]
    assert hit == [11, 12]  # frame 10 ends at sample 1999
    for i in range(fb.shape[0]):
        assert np.all(fb[i] > floor) if i in hit else np.all(fb[i] == floor)


def test_lfr_by_hand():
    # frames numbered 0..T-1 (every mel value equal to the frame number)
    def rows(T):
        feats = np.repeat(np.arange(T, dtype=np.float64)[:, None], 2, axis=1)
        out = F.lfr(feats)
        return out.reshape(out.shape[0], 7, 2)[:, :, 0].astype(int).tolist()
    assert rows(8) == [[0, 0, 0, 0, 1, 2, 3], [3, 4, 5, 6, 7, 7, 7]]
    assert rows(6) == [[0, 0, 0, 0, 1, 2, 3]]
    assert rows(7) == [[0, 0, 0, 0, 1, 2, 3], [3, 4, 5, 6, 6, 6, 6]]
    assert rows(1) == [[0] * 7]
    # frames keep their mel order inside a stacked row
    feats = np.arange(12, dtype=np.float64).reshape(6, 2)
    assert F.lfr(feats)[0, 8:10].tolist() == [2.0, 3.0]


def test_pins_catch_planted_mistakes():
    global F
    src = inspect.getsource(F)
    planted = {
        "log10": ("return np.log(np.maximum(e, FLOAT32_EPS))", "return np.log10(np.maximum(e, FLOAT32_EPS))",
                  test_signals_that_vanish_after_mean_removal),
        "hann window": ("return 0.54 - 0.46 * np.cos", "return 0.5 - 0.5 * np.cos", test_hamming_closed_form),
        "no left padding": ("left = (c.lfr_m - 1) // 2", "left = 0", test_lfr_by_hand),
        "mel from 0 Hz": ("edges = np.linspace(mel(c.low_freq)", "edges = np.linspace(mel(0.0)",
                          test_sine440_energy_peaks_in_the_nearest_filter),
        "no mean removal": ("fr = fr - fr.mean(axis=1, keepdims=True)", "pass",
                            test_signals_that_vanish_after_mean_removal),
        "pad to 400": ("np.fft.rfft(frames, n=c.n_fft, axis=1)", "np.fft.rfft(frames, n=c.frame_len, axis=1)",
                       test_parseval_on_the_padded_frame),
    }
    original = F
    try:
        for name, (old, new, pin) in planted.items():
            assert old in src, name
            mod = type(original)("planted_frontend")
            sys.modules[mod.__name__] = mod  # the dataclass looks its module up
            exec(compile(src.replace(old, new), f"<planted {name}>", "exec"), mod.__dict__)
            F = mod
            with pytest.raises((AssertionError, ValueError)):
                pin()
    finally:
        F = original
        sys.modules.pop("planted_frontend", None)
