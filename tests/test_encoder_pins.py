"""Pins of the SAN-M encoder oracle (oracle/encoder.py): the sinusoid's closed
form, the FSMN memory and a whole SAN-M block against plain Python loops on
the block probe of audio.cpp "Fun-ASR-Nano Native Runtime Implementation
Plan", Task 3 Step 1 (d_in 12, d_model 8, two heads, FFN 16, kernel 3),
attention special cases, and the encoder's stage order through the
normalisations' statistics. Planted mistakes must each fail one of them."""
import inspect
import math
import sys

import numpy as np
import pytest

from oracle import encoder as E

PROBE = E.EncoderConfig(in_dim=12, dim=8, n_head=2, ffn_dim=16, kernel=3, n_main=0, n_tp=0)


def probe_params(cfg, seed, names):
    rng = np.random.default_rng(seed)
    p = {}
    for b, pre in enumerate(names):
        n_in = cfg.in_dim if b == 0 else cfg.dim
        D, F = cfg.dim, cfg.ffn_dim
        shapes = {"norm1.g": (n_in,), "norm1.b": (n_in,), "q.w": (D, n_in), "q.b": (D,), "k.w": (D, n_in),
                  "k.b": (D,), "v.w": (D, n_in), "v.b": (D,), "fsmn.w": (D, cfg.kernel), "o.w": (D, D), "o.b": (D,),
                  "norm2.g": (D,), "norm2.b": (D,), "ffn1.w": (F, D), "ffn1.b": (F,), "ffn2.w": (D, F),
                  "ffn2.b": (D,)}
        for k, s in shapes.items():
            p[pre + k] = (1.0 if k.endswith(".g") else 0.0) + 0.4 * rng.standard_normal(s)
    for k in ("after_norm", "tp_norm"):
        p[k + ".g"] = 1.0 + 0.3 * rng.standard_normal(cfg.dim)
        p[k + ".b"] = 0.3 * rng.standard_normal(cfg.dim)
    return p


# ------------------------------------------------- plain-loop reference (tiny)

def loop_ln(row, g, b, eps):
    n = len(row)
    mu = sum(row) / n
    var = sum((v - mu) ** 2 for v in row) / n
    return [(row[i] - mu) / math.sqrt(var + eps) * g[i] + b[i] for i in range(n)]


def loop_linear(row, w, b):
    return [sum(w[o][i] * row[i] for i in range(len(row))) + b[o] for o in range(len(w))]


def loop_block(x, p, pre, cfg, residual):
    T, D, H = len(x), cfg.dim, cfg.n_head
    hd = D // H
    P = {k: v.tolist() for k, v in p.items() if k.startswith(pre)}
    h = [loop_ln(r, P[pre + "norm1.g"], P[pre + "norm1.b"], cfg.ln_eps) for r in x]
    q = [loop_linear(r, P[pre + "q.w"], P[pre + "q.b"]) for r in h]
    k = [loop_linear(r, P[pre + "k.w"], P[pre + "k.b"]) for r in h]
    v = [loop_linear(r, P[pre + "v.w"], P[pre + "v.b"]) for r in h]
    att = [[0.0] * D for _ in range(T)]
    for hh in range(H):
        c0 = hh * hd
        for t in range(T):
            s = [sum(q[t][c0 + j] * k[u][c0 + j] for j in range(hd)) / math.sqrt(hd) for u in range(T)]
            m = max(s)
            e = [math.exp(z - m) for z in s]
            z = sum(e)
            for j in range(hd):
                att[t][c0 + j] = sum(e[u] / z * v[u][c0 + j] for u in range(T))
    o = [loop_linear(r, P[pre + "o.w"], P[pre + "o.b"]) for r in att]
    K = cfg.kernel
    half = (K - 1) // 2
    y = []
    for t in range(T):
        row = []
        for c in range(D):
            mem = v[t][c]
            for j in range(K):
                u = t + j - half
                if 0 <= u < T:
                    mem += P[pre + "fsmn.w"][c][j] * v[u][c]
            row.append(o[t][c] + mem)
        y.append(row)
    x1 = [[x[t][c] + y[t][c] for c in range(D)] for t in range(T)] if residual else y
    out = []
    for r in x1:
        n2 = loop_ln(r, P[pre + "norm2.g"], P[pre + "norm2.b"], cfg.ln_eps)
        f = [max(0.0, a) for a in loop_linear(n2, P[pre + "ffn1.w"], P[pre + "ffn1.b"])]
        f2 = loop_linear(f, P[pre + "ffn2.w"], P[pre + "ffn2.b"])
        out.append([r[c] + f2[c] for c in range(D)])
    return out


# ----------------------------------------------------------------------- pins

def test_positions_closed_form():
    pe = E.positions(5, 560)
    np.testing.assert_array_equal(pe[0, 0::2], 0.0)
    np.testing.assert_array_equal(pe[0, 1::2], 1.0)
    assert pe[3, 0] == pytest.approx(math.sin(3.0)) and pe[3, 1] == pytest.approx(math.cos(3.0))
    # the slowest pair: wavelength 2 pi 10000^((d-2)/d)
    w = 10000.0 ** (558.0 / 560.0)
    assert pe[4, 558] == pytest.approx(math.sin(4.0 / w)) and pe[4, 559] == pytest.approx(math.cos(4.0 / w))


def test_fsmn_special_kernels_and_loops():
    rng = np.random.default_rng(2)
    v = rng.standard_normal((9, 4))
    # centre tap 1: memory 2 v; first tap 1: v plus v delayed by one frame
    w = np.zeros((4, 3))
    w[:, 1] = 1.0
    np.testing.assert_allclose(E.fsmn(v, w), 2 * v)
    w = np.zeros((4, 3))
    w[:, 0] = 1.0
    want = v.copy()
    want[1:] += v[:-1]
    np.testing.assert_allclose(E.fsmn(v, w), want)
    # random taps, kernel 5, against loops with zero padding
    w = rng.standard_normal((4, 5))
    got = E.fsmn(v, w)
    for t in range(9):
        for c in range(4):
            ref = v[t, c] + sum(w[c, j] * v[t + j - 2, c] for j in range(5) if 0 <= t + j - 2 < 9)
            assert got[t, c] == pytest.approx(ref, abs=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((6, 8))
    v = rng.standard_normal((6, 8))
    # identical keys: every frame takes the plain average of the values
    k = np.tile(rng.standard_normal((1, 8)), (6, 1))
    np.testing.assert_allclose(E.attention(q, k, v, 2), np.tile(v.mean(axis=0), (6, 1)), atol=1e-12)
    # one frame: the value itself
    np.testing.assert_allclose(E.attention(q[:1], k[:1], v[:1], 2), v[:1], atol=1e-12)


@pytest.mark.parametrize("residual", [False, True])
def test_sanm_block_matches_loops_on_the_probe(residual):
    cfg = PROBE
    names = ["encoders0.0.", "encoders.0."]
    p = probe_params(cfg, 5 + residual, names)
    rng = np.random.default_rng(7)
    if residual:
        x = rng.standard_normal((5, cfg.dim))
        pre = "encoders.0."
    else:
        x = rng.standard_normal((5, cfg.in_dim))
        pre = "encoders0.0."
    got = E.sanm_block(x, p, pre, cfg, residual)
    want = np.array(loop_block(x.tolist(), p, pre, cfg, residual))
    assert got.shape == (5, cfg.dim)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_encoder_stage_order():
    # stem, one main block, after_norm, one tp block, tp_norm: the stage
    # tensors exist in that order, the embed is rows * sqrt(dim) + positions,
    # and the normalised stages have each row's mean and spread set by the
    # norm's bias and gain (chosen constant here)
    cfg = E.EncoderConfig(in_dim=12, dim=8, n_head=2, ffn_dim=16, kernel=3, n_main=1, n_tp=1)
    p = probe_params(cfg, 11, cfg.block_names())
    p["after_norm.g"][:] = 2.0
    p["after_norm.b"][:] = 0.5
    p["tp_norm.g"][:] = 3.0
    p["tp_norm.b"][:] = -1.0
    feats = np.random.default_rng(12).standard_normal((6, 12))
    st = {}
    out = E.encoder(feats, p, cfg, st)
    assert list(st) == ["enc.embed.out", "enc.encoders0.0.out", "enc.encoders.0.out", "enc.after_norm.out",
                        "enc.tp_encoders.0.out", "enc.tp_norm.out"]
    np.testing.assert_allclose(st["enc.embed.out"], feats * math.sqrt(8) + E.positions(6, 12))
    a = st["enc.after_norm.out"]
    np.testing.assert_allclose(a.mean(axis=1), 0.5, atol=1e-12)
    np.testing.assert_allclose(a.std(axis=1), 2.0, rtol=1e-9)
    np.testing.assert_allclose(out.mean(axis=1), -1.0, atol=1e-12)
    np.testing.assert_allclose(out.std(axis=1), 3.0, rtol=1e-9)
    # the tp block reads after_norm's output; the first main block the stem's
    np.testing.assert_allclose(st["enc.tp_encoders.0.out"], E.sanm_block(a, p, "tp_encoders.0.", cfg, True))
    np.testing.assert_allclose(st["enc.encoders.0.out"],
                               E.sanm_block(st["enc.encoders0.0.out"], p, "encoders.0.", cfg, True))


def test_pins_catch_planted_mistakes():
    global E
    src = inspect.getsource(E)
    planted = {
        "fsmn without v": ("    out = v.copy()\n", "    out = np.zeros_like(v)\n", test_fsmn_special_kernels_and_loops),
        "fsmn causal": ("half = (K - 1) // 2", "half = K - 1", test_fsmn_special_kernels_and_loops),
        "no attention residual": ("x = x + y if residual else y", "x = y",
                                  test_sanm_block_matches_loops_on_the_probe),
        "scale by in_dim": ("return x * np.sqrt(cfg.dim)", "return x * np.sqrt(cfg.in_dim)", test_encoder_stage_order),
        "positions from 1": ("pos = np.arange(t, dtype=np.float64)[:, None]",
                             "pos = np.arange(1, t + 1, dtype=np.float64)[:, None]", test_positions_closed_form),
        "unscaled scores": ("s = q[:, sl] @ k[:, sl].T / np.sqrt(hd)", "s = q[:, sl] @ k[:, sl].T",
                            test_sanm_block_matches_loops_on_the_probe),
    }
    original = E
    try:
        for name, (old, new, pin) in planted.items():
            assert old in src, name
            mod = type(original)("oracle.planted_encoder")
            mod.__package__ = "oracle"
            sys.modules[mod.__name__] = mod
            exec(compile(src.replace(old, new), f"<planted {name}>", "exec"), mod.__dict__)
            E = mod
            with pytest.raises(AssertionError):
                if pin is test_sanm_block_matches_loops_on_the_probe:
                    pin(False)
                    pin(True)
                else:
                    pin()
    finally:
        E = original
        sys.modules.pop("oracle.planted_encoder", None)
