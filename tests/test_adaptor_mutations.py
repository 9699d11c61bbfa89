"""Planted mistakes in the adaptor oracle (on the CPU) must each be caught by at
least one adaptor pin: evidence that the pins notice a mask, a dropped bias,
a wrong variance, a swapped norm position, a wrong scale or a missing ReLU."""
import numpy as np
import pytest

from oracle import adaptor as oa

from . import test_adaptor_pins as pins

PINS = [
    pins.test_layer_norm_hand,
    pins.test_layer_norm_invariances,
    pins.test_layer_norm_matches_torch,
    pins.test_mha_matches_torch_and_is_bidirectional,
    pins.test_block_matches_torch_encoder_layer,
    lambda: pins.test_adaptor_matches_torch_stack(5),
]


def caught() -> int:
    n = 0
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            n += 1
    return n


def m_ln_unbiased(x, g, b, eps):
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).sum(axis=-1, keepdims=True) / (x.shape[-1] - 1)
    return (x - mu) / np.sqrt(var + eps) * g + b


def _mha_variant(causal=False, scale_pow=0.5, drop="", swap_kq=False):
    def f(x, p, pre, n_head):
        T, D = x.shape
        hd = D // n_head
        b = {t: (np.zeros_like(p[pre + t + ".b"]) if t == drop else p[pre + t + ".b"]) for t in "qkvo"}
        q = (x @ p[pre + "q.w"].T + b["q"]).reshape(T, n_head, hd)
        k = (x @ p[pre + "k.w"].T + b["k"]).reshape(T, n_head, hd)
        v = (x @ p[pre + "v.w"].T + b["v"]).reshape(T, n_head, hd)
        if swap_kq:
            q, k = k, q
        o = np.empty((T, n_head, hd))
        for h in range(n_head):
            s = q[:, h] @ k[:, h].T / hd ** scale_pow
            if causal:
                s = np.where(np.tril(np.ones((T, T), bool)), s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            e = np.exp(s)
            o[:, h] = (e / e.sum(axis=1, keepdims=True)) @ v[:, h]
        return o.reshape(T, D) @ p[pre + "o.w"].T + b["o"]
    return f


def m_block_post_norm(x, p, i, cfg):
    pre = f"blocks.{i}."
    x = oa.layer_norm(x + oa.mha(x, p, pre, cfg.n_head), p[pre + "norm1.g"], p[pre + "norm1.b"], cfg.ln_eps)
    h = oa.relu(oa.linear(x, p[pre + "fc1.w"], p[pre + "fc1.b"]))
    return oa.layer_norm(x + oa.linear(h, p[pre + "fc2.w"], p[pre + "fc2.b"]), p[pre + "norm2.g"],
                         p[pre + "norm2.b"], cfg.ln_eps)


def m_block_no_ffn_relu(x, p, i, cfg):
    pre = f"blocks.{i}."
    x = x + oa.mha(oa.layer_norm(x, p[pre + "norm1.g"], p[pre + "norm1.b"], cfg.ln_eps), p, pre, cfg.n_head)
    h = oa.layer_norm(x, p[pre + "norm2.g"], p[pre + "norm2.b"], cfg.ln_eps)
    return x + oa.linear(oa.linear(h, p[pre + "fc1.w"], p[pre + "fc1.b"]), p[pre + "fc2.w"], p[pre + "fc2.b"])


def m_relu_leaky(x):
    return np.where(x > 0, x, 0.01 * x)


MUTATIONS = {
    "layernorm unbiased variance": ("layer_norm", m_ln_unbiased),
    "attention causal mask": ("mha", _mha_variant(causal=True)),
    "attention scale 1/head_dim": ("mha", _mha_variant(scale_pow=1.0)),
    "attention without q bias": ("mha", _mha_variant(drop="q")),
    "attention without o bias": ("mha", _mha_variant(drop="o")),
    "block post-norm": ("block", m_block_post_norm),
    "block FFN without ReLU": ("block", m_block_no_ffn_relu),
    "leaky ReLU": ("relu", m_relu_leaky),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(oa, attr, fn)
    # the pins import the functions by name from oracle.adaptor: patch there too
    monkeypatch.setattr(pins, attr, fn, raising=False)
    assert caught() >= 1, f"no pin catches: {name}"


def test_unmutated_oracle_passes_every_pin():
    assert caught() == 0
