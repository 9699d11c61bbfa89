"""CPU oracle of the audio frontend: Kaldi-style log-mel filterbank and LFR
frame stacking (test infrastructure: imported by tests/ and bench.py's
baseline leg only, never by the product path; numpy, float64).

Sources:
  * audio.cpp "Fun-ASR-Nano Native Runtime Implementation Plan", Task 2 Step 4:
    pre-emphasis 0.97, 25 ms Hamming frames, 10 ms shift, 80 HTK mel bins,
    natural log, centred LFR 7/6 with replicated edge frames, CMVN off;
    output time-major rows of num_mels * lfr_m = 560 values.
  * transcribe.cpp "Forward map - funasr_nano", table "Frontend": 16 kHz mono
    PCM -> Kaldi HTK fbank [T_frames, 80] -> LFR (m=7, n=6) [T_lfr, 560], no
    CMVN.

Readings where the pages are silent (each listed in the design doc):
  * PCM samples are used as given (no rescaling); 16 kHz, so a frame is 400
    samples and the shift 160;
  * framing keeps only whole frames: T_frames = 1 + (N - 400) // 160 for
    N >= 400, else none (Kaldi's default edge handling);
  * per frame, in Kaldi's order: the frame's mean is subtracted, then
    pre-emphasis y[i] = x[i] - 0.97 x[i-1] with y[0] = x[0] - 0.97 x[0], then
    the Hamming window 0.54 - 0.46 cos(2 pi n / 399); no dither;
  * the power spectrum |X_k|^2 of the frame zero-padded to 512 samples (the
    next power of two), bins k = 0 .. 255 (frequency 31.25 k Hz);
  * 80 triangular filters on the HTK mel scale mel(f) = 1127 ln(1 + f / 700),
    edges equally spaced in mel from 20 Hz to 8000 Hz (filter j rises from
    edge j to edge j+1 and falls to edge j+2, measured in mel);
  * log(max(energy, eps)) with eps the float32 machine epsilon 2^-23;
  * LFR row i stacks padded frames 6 i .. 6 i + 6 in time order, where padded
    frame p is frame clamp(p - 3, 0, T_frames - 1): three copies of the
    first frame in front, the last frame repeated past the end; there are
    ceil(T_frames / 6) rows.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

SAMPLE_RATE = 16000
FLOAT32_EPS = float(np.finfo(np.float32).eps)


@dataclass(frozen=True)
class FrontendConfig:
    frame_len: int = 400      # 25 ms at 16 kHz
    frame_shift: int = 160    # 10 ms
    n_fft: int = 512          # next power of two of the frame length
    n_mels: int = 80
    low_freq: float = 20.0
    high_freq: float = 8000.0  # Nyquist
    preemph: float = 0.97
    lfr_m: int = 7
    lfr_n: int = 6


def n_frames(n_samples: int, c: FrontendConfig = FrontendConfig()) -> int:
    """Whole frames of a signal of n_samples."""
    return 0 if n_samples < c.frame_len else 1 + (n_samples - c.frame_len) // c.frame_shift


def n_lfr_rows(n_samples: int, c: FrontendConfig = FrontendConfig()) -> int:
    """LFR rows: ceil(T_frames / n)."""
    t = n_frames(n_samples, c)
    return (t + c.lfr_n - 1) // c.lfr_n


def hamming(n: int) -> np.ndarray:
    """0.54 - 0.46 cos(2 pi i / (n - 1)), i = 0 .. n - 1."""
    i = np.arange(n, dtype=np.float64)
    return 0.54 - 0.46 * np.cos(2.0 * np.pi * i / (n - 1))


def mel(f):
    """HTK mel scale."""
    return 1127.0 * np.log(1.0 + np.asarray(f, dtype=np.float64) / 700.0)


def mel_filters(c: FrontendConfig = FrontendConfig()) -> np.ndarray:
    """[n_mels, n_fft / 2] triangle weights over the power-spectrum bins."""
    n_bins = c.n_fft // 2
    edges = np.linspace(mel(c.low_freq), mel(c.high_freq), c.n_mels + 2)
    m = mel(np.arange(n_bins) * (SAMPLE_RATE / c.n_fft))
    w = np.zeros((c.n_mels, n_bins))
    for j in range(c.n_mels):
        left, centre, right = edges[j], edges[j + 1], edges[j + 2]
        up = (m - left) / (centre - left)
        down = (right - m) / (right - centre)
        w[j] = np.where((m > left) & (m < right), np.minimum(up, down), 0.0)
    return w


def frame_signal(pcm: np.ndarray, c: FrontendConfig = FrontendConfig()) -> np.ndarray:
    """[T_frames, frame_len] frames after mean removal, pre-emphasis and window."""
    x = np.asarray(pcm, dtype=np.float64)
    t = n_frames(len(x), c)
    idx = np.arange(t)[:, None] * c.frame_shift + np.arange(c.frame_len)[None, :]
    fr = x[idx] if t else np.zeros((0, c.frame_len))
    fr = fr - fr.mean(axis=1, keepdims=True)
    prev = np.concatenate([fr[:, :1], fr[:, :-1]], axis=1)  # x[i-1], and x[0] for i = 0
    fr = fr - c.preemph * prev
    return fr * hamming(c.frame_len)[None, :]


def power_spectrum(frames: np.ndarray, c: FrontendConfig = FrontendConfig()) -> np.ndarray:
    """|X_k|^2 for k = 0 .. n_fft / 2 - 1 of each frame zero-padded to n_fft."""
    spec = np.fft.rfft(frames, n=c.n_fft, axis=1)[:, : c.n_fft // 2]
    return spec.real ** 2 + spec.imag ** 2


def fbank(pcm: np.ndarray, c: FrontendConfig = FrontendConfig()) -> np.ndarray:
    """[T_frames, n_mels] natural-log mel energies."""
    e = power_spectrum(frame_signal(pcm, c), c) @ mel_filters(c).T
    return np.log(np.maximum(e, FLOAT32_EPS))


def lfr(feats: np.ndarray, c: FrontendConfig = FrontendConfig()) -> np.ndarray:
    """[ceil(T / n), m * n_mels] stacked frames (centred, edge frames repeated)."""
    t = feats.shape[0]
    rows = (t + c.lfr_n - 1) // c.lfr_n
    left = (c.lfr_m - 1) // 2
    src = np.clip(np.arange(rows)[:, None] * c.lfr_n + np.arange(c.lfr_m)[None, :] - left, 0, max(t - 1, 0))
    return feats[src].reshape(rows, c.lfr_m * feats.shape[1])


def frontend(pcm: np.ndarray, c: FrontendConfig = FrontendConfig()) -> np.ndarray:
    """PCM -> LFR rows [T_lfr, 560] (the page's frontend gate tensor; CMVN off)."""
    return lfr(fbank(pcm, c), c)
