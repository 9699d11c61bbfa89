"""Planted mistakes in the oracle (on the CPU) must each be caught by at least
one pin. This is the evidence that the pins would notice a dropped term, a
wrong sign or index, or a transposed operand in the oracle."""
import numpy as np
import pytest

import oracle
from oracle import qwen3 as oq

from . import test_oracle_pins as pins

PINS = [
    pins.test_rms_norm_closed_form,
    pins.test_rms_norm_matches_torch_and_scale_invariance,
    pins.test_rope_complex_rotation,
    pins.test_rope_invariants,
    pins.test_attention_brute_force,
    pins.test_attention_matches_torch_sdpa_gqa,
    pins.test_gqa_equals_mha_with_repeated_kv,
    pins.test_block_brute_force,
    pins.test_whole_model_matches_transformers_qwen3,
    pins.test_override_identity,
    pins.test_kv_consistency_prefill_vs_decode,
]


def caught(monkeypatch_ctx) -> list:
    failed = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failed.append(pin.__name__)
    return failed


_rms = oq.rms_norm
_rope = oq.apply_rope
_attn = oq.attention
_silu = oq.silu


def m_eps_outside(x, g, eps):
    return x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps) * g


def m_rope_sign(x, pos, theta):
    D = x.shape[-1]
    h = D // 2
    ang = oq.rope_angles(pos, D, theta)
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c + b * s, b * c - a * s], axis=-1)


def m_rope_interleaved(x, pos, theta):
    D = x.shape[-1]
    ang = oq.rope_angles(pos, D, theta)
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    a, b = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = b * c + a * s
    return out


def m_gqa_modulo(q, k, v, q_pos, n_valid, block=512):
    n_kv = k.shape[0]
    idx = np.arange(q.shape[1]) % n_kv
    return _attn(q, k[idx], v[idx], q_pos, n_valid, block)


def m_scale_d(q, k, v, q_pos, n_valid, block=512):
    return _attn(q * np.sqrt(1.0 / q.shape[-1]), k, v, q_pos, n_valid, block)


def m_mask_strict(q, k, v, q_pos, n_valid, block=512):
    T, n_q, D = q.shape
    group = n_q // k.shape[0]
    out = np.zeros_like(q)
    u = np.arange(n_valid)
    for h in range(n_q):
        for t in range(T):
            ok = u < q_pos[t]
            if not ok.any():
                continue
            s = (k[h // group, :n_valid][ok] @ q[t, h]) / np.sqrt(D)
            p = np.exp(s - s.max())
            out[t, h] = (p / p.sum()) @ v[h // group, :n_valid][ok]
    return out


def m_skip_qk_norm(x, g, eps):
    if x.ndim == 3:  # per-head norm of q / k
        return x
    return _rms(x, g, eps)


def m_silu_identity(z):
    return z


MUTATIONS = {
    "eps_outside_sqrt": ("rms_norm", m_eps_outside),
    "rope_sign": ("apply_rope", m_rope_sign),
    "rope_interleaved_pairs": ("apply_rope", m_rope_interleaved),
    "gqa_modulo_grouping": ("attention", m_gqa_modulo),
    "attention_scale_1_over_d": ("attention", m_scale_d),
    "mask_excludes_current": ("attention", m_mask_strict),
    "no_qk_norm": ("rms_norm", m_skip_qk_norm),
    "no_silu": ("silu", m_silu_identity),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_function_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(oq, attr, fn)
    monkeypatch.setattr(oracle, attr, fn)
    assert caught(monkeypatch), f"no pin caught mutation {name}"


class SwappedGateUp(oq.Qwen3Oracle):
    def __init__(self, cfg, params, dtype=np.float64):
        params = dict(params)
        for i in range(cfg.n_layer):
            params[f"L{i}.w_gate"], params[f"L{i}.w_up"] = params[f"L{i}.w_up"], params[f"L{i}.w_gate"]
        super().__init__(cfg, params, dtype)


class AddInsteadOfReplace(oq.Qwen3Oracle):
    def embed(self, ids, audio, audio_begin):
        x = self.p["embed"][np.asarray(ids) % self.cfg.vocab].copy()
        if audio is not None and len(audio):
            x[audio_begin:audio_begin + len(audio)] += audio
        return x


class NoFinalNorm(oq.Qwen3Oracle):
    def head(self, x_last):
        return x_last @ self.p["embed"].T


class RopeAtRelativeZero(oq.Qwen3Oracle):
    """Rotates every chunk as if it started at position 0."""
    def block(self, i, x, state, pos0):
        saved = oq.apply_rope
        oq.apply_rope = lambda v, pos, th: saved(v, pos - pos0, th)
        try:
            return super().block(i, x, state, pos0)
        finally:
            oq.apply_rope = saved


@pytest.mark.parametrize("cls", [SwappedGateUp, AddInsteadOfReplace, NoFinalNorm, RopeAtRelativeZero])
def test_planted_structural_mistake_is_caught(cls, monkeypatch):
    monkeypatch.setattr(oracle, "Qwen3Oracle", cls)
    monkeypatch.setattr(oq, "Qwen3Oracle", cls)
    assert caught(monkeypatch), f"no pin caught {cls.__name__}"
