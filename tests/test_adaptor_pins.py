"""Pins of the adaptor oracle (transcribe.cpp "Forward map - funasr_nano",
section "Adaptor"). Each check comes from outside the oracle's code: hand
arithmetic, invariances the definition implies, and torch's own modules
(nn.LayerNorm, nn.MultiheadAttention, a pre-norm nn.TransformerEncoderLayer)
loaded with the same parameters, in float64."""
import numpy as np
import pytest

import synth
from oracle.adaptor import AdaptorConfig, adaptor, block, layer_norm, mha

SMALL = synth.AdaptorShape(enc_dim=64, mid_dim=96, dim=64, ffn_dim=16, n_block=2, n_head=4)
SMALL_CFG = AdaptorConfig(enc_dim=64, mid_dim=96, dim=64, ffn_dim=16, n_block=2, n_head=4)


def test_layer_norm_hand():
    # mean 2.5, population variance 1.25: (x - 2.5) / sqrt(1.25)
    y = layer_norm(np.array([[1.0, 2.0, 3.0, 4.0]]), np.ones(4), np.zeros(4), 0.0)
    np.testing.assert_allclose(y[0], [-1.5, -0.5, 0.5, 1.5] / np.sqrt(1.25), rtol=1e-15)
    # gain and bias act after the normalisation
    y2 = layer_norm(np.array([[1.0, 2.0, 3.0, 4.0]]), np.full(4, 2.0), np.full(4, 0.5), 0.0)
    np.testing.assert_allclose(y2, 2.0 * y + 0.5, rtol=1e-15)


def test_layer_norm_invariances():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 32))
    g, b = 1 + 0.1 * rng.standard_normal(32), 0.1 * rng.standard_normal(32)
    y = layer_norm(x, g, b, 1e-12)
    # shift and positive scale of a row do not change it
    np.testing.assert_allclose(layer_norm(3.0 * x + 7.0, g, b, 1e-12), y, rtol=1e-9, atol=1e-12)
    z = layer_norm(x, np.ones(32), np.zeros(32), 1e-12)
    np.testing.assert_allclose(z.mean(axis=1), 0.0, atol=1e-12)
    np.testing.assert_allclose((z ** 2).mean(axis=1), 1.0, rtol=1e-9)


def _torch_params(f32, prefix, torch):
    return {k[len(prefix):]: torch.from_numpy(v.astype(np.float64)) for k, v in f32.items() if k.startswith(prefix)}


def test_layer_norm_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(4)
    x = rng.standard_normal((7, 48))
    g, b = 1 + 0.1 * rng.standard_normal(48), 0.1 * rng.standard_normal(48)
    ln = torch.nn.LayerNorm(48, eps=1e-12, dtype=torch.float64)
    with torch.no_grad():
        ln.weight.copy_(torch.from_numpy(g))
        ln.bias.copy_(torch.from_numpy(b))
        ref = ln(torch.from_numpy(x)).numpy()
    np.testing.assert_allclose(layer_norm(x, g, b, 1e-12), ref, rtol=1e-12, atol=1e-12)


def test_mha_matches_torch_and_is_bidirectional():
    torch = pytest.importorskip("torch")
    f32, _ = synth.make_adaptor_weights(SMALL, 9)
    p = {k: v.astype(np.float64) for k, v in f32.items()}
    x = np.random.default_rng(5).standard_normal((11, SMALL.dim))
    got = mha(x, p, "blocks.0.", SMALL.n_head)
    m = torch.nn.MultiheadAttention(SMALL.dim, SMALL.n_head, bias=True, batch_first=True, dtype=torch.float64)
    t = _torch_params(f32, "blocks.0.", torch)
    with torch.no_grad():
        m.in_proj_weight.copy_(torch.cat([t["q.w"], t["k.w"], t["v.w"]]))
        m.in_proj_bias.copy_(torch.cat([t["q.b"], t["k.b"], t["v.b"]]))
        m.out_proj.weight.copy_(t["o.w"])
        m.out_proj.bias.copy_(t["o.b"])
        xt = torch.from_numpy(x)[None]
        ref = m(xt, xt, xt, need_weights=False)[0][0].numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)
    # every frame sees every frame: permuting the frames permutes the output
    perm = np.random.default_rng(6).permutation(11)
    np.testing.assert_allclose(mha(x[perm], p, "blocks.0.", SMALL.n_head), got[perm], rtol=1e-10, atol=1e-12)


def _torch_block(f32, i, shape, torch):
    layer = torch.nn.TransformerEncoderLayer(shape.dim, shape.n_head, dim_feedforward=shape.ffn_dim, dropout=0.0,
                                             activation="relu", layer_norm_eps=1e-12, batch_first=True,
                                             norm_first=True, dtype=torch.float64)
    t = _torch_params(f32, f"blocks.{i}.", torch)
    with torch.no_grad():
        layer.self_attn.in_proj_weight.copy_(torch.cat([t["q.w"], t["k.w"], t["v.w"]]))
        layer.self_attn.in_proj_bias.copy_(torch.cat([t["q.b"], t["k.b"], t["v.b"]]))
        layer.self_attn.out_proj.weight.copy_(t["o.w"])
        layer.self_attn.out_proj.bias.copy_(t["o.b"])
        layer.norm1.weight.copy_(t["norm1.g"])
        layer.norm1.bias.copy_(t["norm1.b"])
        layer.norm2.weight.copy_(t["norm2.g"])
        layer.norm2.bias.copy_(t["norm2.b"])
        layer.linear1.weight.copy_(t["fc1.w"])
        layer.linear1.bias.copy_(t["fc1.b"])
        layer.linear2.weight.copy_(t["fc2.w"])
        layer.linear2.bias.copy_(t["fc2.b"])
    return layer.eval()


def test_block_matches_torch_encoder_layer():
    torch = pytest.importorskip("torch")
    f32, _ = synth.make_adaptor_weights(SMALL, 10)
    p = {k: v.astype(np.float64) for k, v in f32.items()}
    x = np.random.default_rng(7).standard_normal((9, SMALL.dim))
    layer = _torch_block(f32, 1, SMALL, torch)
    with torch.no_grad():
        ref = layer(torch.from_numpy(x)[None])[0].numpy()
    np.testing.assert_allclose(block(x, p, 1, SMALL_CFG), ref, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("T", [1, 5, 23])
def test_adaptor_matches_torch_stack(T):
    torch = pytest.importorskip("torch")
    f32, _ = synth.make_adaptor_weights(SMALL, 11)
    x = synth.encoder_frames(11, T, SMALL.enc_dim).astype(np.float64)
    lin1 = torch.nn.Linear(SMALL.enc_dim, SMALL.mid_dim, dtype=torch.float64)
    lin2 = torch.nn.Linear(SMALL.mid_dim, SMALL.dim, dtype=torch.float64)
    with torch.no_grad():
        lin1.weight.copy_(torch.from_numpy(f32["linear1.w"].astype(np.float64)))
        lin1.bias.copy_(torch.from_numpy(f32["linear1.b"].astype(np.float64)))
        lin2.weight.copy_(torch.from_numpy(f32["linear2.w"].astype(np.float64)))
        lin2.bias.copy_(torch.from_numpy(f32["linear2.b"].astype(np.float64)))
        net = torch.nn.Sequential(lin1, torch.nn.ReLU(), lin2,
                                  *[_torch_block(f32, i, SMALL, torch) for i in range(SMALL.n_block)])
        ref = net(torch.from_numpy(x)[None])[0].numpy()
    np.testing.assert_allclose(adaptor(x, f32, SMALL_CFG), ref, rtol=1e-10, atol=1e-12)


def test_generator_draw_order_and_rounding():
    f32, bits = synth.make_adaptor_weights(synth.AdaptorShape(), 1)
    assert list(f32)[:4] == ["linear1.w", "linear1.b", "linear2.w", "linear2.b"]
    assert f32["linear1.w"].shape == (2048, 512) and f32["blocks.1.fc2.w"].shape == (1024, 256)
    # the float32 values are exactly the bf16 bit patterns
    np.testing.assert_array_equal(f32["blocks.0.q.w"], synth.bf16_bits_to_f32(bits["blocks.0.q.w"]))
    assert abs(float(f32["blocks.0.norm1.g"].mean()) - 1.0) < 0.01
