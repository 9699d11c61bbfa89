"""GPU parity of the audio frontend and the SAN-M encoder against the float64
oracles (oracle/frontend.py, oracle/encoder.py), at the tolerances of
audio.cpp "Fun-ASR-Nano Native Runtime Implementation Plan": frontend
atol = rtol = 2e-4 (Task 2 Step 2), encoder stages atol = rtol = 2e-3
(Task 4 Step 4). Inputs are the page's frontend fixtures (silence, an
impulse, a 440 Hz sine) and a seeded speech-like signal in place of its
sample recording; weights are seeded random bf16."""
import numpy as np
import pytest

import synth
from oracle import encoder as E
from oracle import frontend as F

from .gpu_harness import record, torch_dev

pytestmark = pytest.mark.gpu


def close(label, got, want, tol):
    err = np.abs(got.astype(np.float64) - want)
    bound = tol + tol * np.abs(want)
    worst = float((err / bound).max()) if err.size else 0.0
    record(label, 0, {"max_abs": float(err.max()) if err.size else 0.0, "worst_over_bound": worst}, kind="encoder")
    assert np.all(np.isfinite(got)), f"{label}: non-finite output"
    assert np.all(err <= bound), f"{label}: max abs {err.max():.3g}, worst/bound {worst:.3g}"
    return worst


def encoder_config(shape):
    return E.EncoderConfig(in_dim=shape.in_dim, dim=shape.dim, n_head=shape.n_head, ffn_dim=shape.ffn_dim,
                           kernel=shape.kernel, n_main=shape.n_main, n_tp=shape.n_tp)


def make_encoder(shape, seed):
    from qwen3_kv_cache_amd.device import Encoder
    w32, bits = synth.make_encoder_weights(shape, seed)
    return Encoder(shape, bits), w32


SMALL = synth.EncoderShape(n_main=2, n_tp=1)


@pytest.mark.parametrize("kind,n", [("silence", 16000), ("impulse", 8000), ("sine440", 16000), ("voiced", 48000),
                                    ("voiced", 400), ("voiced", 559), ("voiced", 4000 + 123)])
def test_frontend_matches_oracle(kind, n):
    torch, dev = torch_dev()
    enc, _ = make_encoder(synth.EncoderShape(n_main=0, n_tp=0), 1)
    try:
        x = synth.pcm(kind, n, 5)
        print(f"[frontend] {kind} {n} samples -> {enc.rows(n)} rows", flush=True)
        got = enc.frontend(torch.from_numpy(x).to(dev))
        torch.cuda.synchronize()
    finally:
        enc.close()
    want = F.frontend(x)
    assert got.shape == want.shape == (F.n_lfr_rows(n), 560)
    close(f"frontend {kind} {n}", got.cpu().numpy(), want, 2e-4)


@pytest.mark.parametrize("rows", [1, 17, 150])
def test_encoder_blocks_match_oracle(rows):
    """Stem, two main blocks, after_norm, one tp block, tp_norm at the real
    widths (560 -> 512, 4 heads, FFN 2048, 11 taps), from LFR rows."""
    torch, dev = torch_dev()
    enc, w32 = make_encoder(SMALL, 2)
    lfr = F.frontend(synth.pcm("voiced", 400 + 960 * max(rows - 1, 0), 6))[:rows]
    assert lfr.shape[0] == rows
    try:
        print(f"[encoder] 3 blocks, {rows} rows", flush=True)
        got = enc.forward(torch.from_numpy(lfr.astype(np.float32)).to(dev))
        torch.cuda.synchronize()
    finally:
        enc.close()
    want = E.encoder(lfr.astype(np.float32), w32, encoder_config(SMALL))
    close(f"encoder 3 blocks {rows} rows", got.cpu().numpy(), want, 2e-3)


def test_encoder_other_widths():
    """dim 256 (2 heads), FFN 512, 3 taps, LFR 5/4 rows of 400: the stem
    operand's pitch, the FSMN width and the LFR stacking all change."""
    torch, dev = torch_dev()
    from qwen3_kv_cache_amd.device import Encoder
    shape = synth.EncoderShape(in_dim=400, dim=256, n_head=2, ffn_dim=512, kernel=3, n_main=1, n_tp=1)
    w32, bits = synth.make_encoder_weights(shape, 3)
    enc = Encoder(shape, bits, lfr_m=5, lfr_n=4)
    c = F.FrontendConfig(lfr_m=5, lfr_n=4)
    x = synth.pcm("voiced", 16000, 7)
    try:
        print("[encoder] dim 256, LFR 5/4", flush=True)
        got = enc.run(torch.from_numpy(x).to(dev))
        torch.cuda.synchronize()
    finally:
        enc.close()
    want = E.encoder(F.frontend(x, c).astype(np.float32), w32, encoder_config(shape))
    assert got.shape == want.shape == (F.n_lfr_rows(16000, c), 256)
    close("encoder dim 256", got.cpu().numpy(), want, 2e-3)


def test_full_encoder_from_pcm():
    """The 70-block encoder (stem, 49 main, after_norm, 20 tp, tp_norm) on 2 s
    of speech-like PCM, end to end from the samples."""
    torch, dev = torch_dev()
    shape = synth.EncoderShape()
    enc, w32 = make_encoder(shape, 4)
    x = synth.pcm("voiced", 32000, 8)
    try:
        print(f"[encoder] 70 blocks, {enc.rows(len(x))} rows", flush=True)
        got = enc.run(torch.from_numpy(x).to(dev))
        torch.cuda.synchronize()
    finally:
        enc.close()
    want = E.encoder(F.frontend(x).astype(np.float32), w32, encoder_config(shape))
    assert got.shape == want.shape == (F.n_lfr_rows(32000), 512)
    print("full encoder worst/bound", close("encoder 70 blocks 2 s", got.cpu().numpy(), want, 2e-3))
