"""Pins for the CPU oracle: checks against things other than the oracle itself
(the pages' printed constants, closed forms, textbook/library special cases,
brute force on tiny inputs and invariants the method must satisfy).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth
from oracle import qwen3 as oq

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny_model(dtype=np.float64, shape=None, seed=1):
    shape = shape or synth.TINY
    W = synth.make_weights(shape, seed)
    return oracle.Qwen3Oracle(oracle.OracleConfig.from_shape(shape), W.f32, dtype=dtype), W


# ------------------------------------------------------------- page constants

def test_page_constants_match_shapes():
    g = json.load(open(os.path.join(GOLDEN, "decoder_constants.json")))
    s = synth.QWEN3_0P6B
    t = g["qwen_tuple"]["value"]
    assert (s.hidden, s.ffn, s.n_layer, s.n_q_head, s.n_kv_head, s.head_dim, s.vocab) == (
        t["hidden"], t["ffn"], t["n_layer"], t["n_q_head"], t["n_kv_head"], t["head_dim"], t["vocab"])
    assert s.rope_theta == g["rope_theta"]["value"]
    assert [s.n_q_head, s.n_kv_head] == g["gqa"]["value"]
    # parameter counts implied by the tuple (tied head adds no parameters)
    shp = synth.layer_shapes(s)
    per_layer = sum(int(np.prod(v)) for k, v in shp.items() if k not in synth.NORM_TENSORS)
    assert per_layer * s.n_layer == 440_401_920  # matrices only
    gains = sum(int(np.prod(v)) for k, v in shp.items() if k in synth.NORM_TENSORS)
    assert gains == 2 * 1024 + 2 * 128
    assert s.vocab * s.hidden == 155_582_464
    # both special ids lie inside the vocabulary
    assert g["audio_token_id"]["value"] < s.vocab and g["eos_token_id"]["value"] < s.vocab


# ---------------------------------------------------------------- RMSNorm

def test_rms_norm_closed_form():
    x = np.array([3.0, 4.0])
    g = np.array([1.0, 2.0])
    # mean square 12.5; with eps=0: x / sqrt(12.5) * g
    out = oracle.rms_norm(x, g, 0.0)
    np.testing.assert_allclose(out, [3 / math.sqrt(12.5), 8 / math.sqrt(12.5)], rtol=1e-15)
    # eps sits inside the square root
    out = oracle.rms_norm(x, g, 0.5)
    np.testing.assert_allclose(out, [3 / math.sqrt(13.0), 8 / math.sqrt(13.0)], rtol=1e-15)


def test_rms_norm_matches_torch_and_scale_invariance():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 64))
    g = 1 + 0.1 * rng.standard_normal(64)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_allclose(oracle.rms_norm(x, g, 1e-6), ref, rtol=1e-13, atol=1e-14)
    for c in (1e-2, 3.0, 1e3):
        np.testing.assert_allclose(oracle.rms_norm(c * x, g, 1e-15), oracle.rms_norm(x, g, 1e-15), rtol=1e-9)


# ------------------------------------------------------------------- RoPE

def test_rope_complex_rotation():
    """NeoX RoPE is multiplication of z_j = x_j + i x_{j+D/2} by exp(i p w_j)."""
    rng = np.random.default_rng(1)
    D = 16
    x = rng.standard_normal((3, 2, D))
    pos = np.array([0, 7, 4095])
    out = oracle.apply_rope(x, pos, 1e6)
    z = x[..., : D // 2] + 1j * x[..., D // 2:]
    w = np.array([1e6 ** (-2 * j / D) for j in range(D // 2)])
    zr = z * np.exp(1j * pos[:, None, None] * w[None, None, :])
    np.testing.assert_allclose(out[..., : D // 2], zr.real, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out[..., D // 2:], zr.imag, rtol=1e-12, atol=1e-12)


def test_rope_invariants():
    rng = np.random.default_rng(2)
    D = 128
    q = rng.standard_normal((1, 1, D))
    k = rng.standard_normal((1, 1, D))
    # R_0 = identity
    np.testing.assert_array_equal(oracle.apply_rope(q, np.array([0]), 1e6), q)
    # norm preserved
    for p in (1, 100, 8255):
        np.testing.assert_allclose(np.linalg.norm(oracle.apply_rope(q, np.array([p]), 1e6)),
                                   np.linalg.norm(q), rtol=1e-13)
    # q.k depends only on the relative position
    def dot(p, s):
        return float(np.sum(oracle.apply_rope(q, np.array([p]), 1e6) * oracle.apply_rope(k, np.array([s]), 1e6)))
    d0 = dot(10, 3)
    for p, s in ((107, 100), (7, 0), (5007, 5000)):
        assert abs(dot(p, s) - d0) < 1e-9
    # lowest pair rotates by exactly p radians, highest by p * theta^(-(D-2)/D)
    ang = oracle.rope_angles(np.array([3]), D, 1e6)
    assert ang[0, 0] == 3.0
    assert math.isclose(ang[0, -1], 3.0 * 1e6 ** (-(D - 2) / D), rel_tol=1e-15)


# -------------------------------------------------------------- attention

def brute_attention(q, k, v, pos, n_valid):
    """Explicit loops in float64: q [T,nq,D], k/v [nkv, n, D]."""
    T, nq, D = q.shape
    nkv = k.shape[0]
    out = np.zeros_like(q)
    for t in range(T):
        for h in range(nq):
            g = h // (nq // nkv)
            scores = []
            for u in range(n_valid):
                if u <= pos[t]:
                    s = 0.0
                    for d in range(D):
                        s += q[t, h, d] * k[g, u, d]
                    scores.append((u, s / math.sqrt(D)))
            m = max(s for _, s in scores)
            den = sum(math.exp(s - m) for _, s in scores)
            for d in range(D):
                out[t, h, d] = sum(math.exp(s - m) / den * v[g, u, d] for u, s in scores)
    return out


def test_attention_brute_force():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((5, 4, 8))
    k = rng.standard_normal((2, 5, 8))
    v = rng.standard_normal((2, 5, 8))
    pos = np.arange(5)
    np.testing.assert_allclose(oracle.attention(q, k, v, pos, 5), brute_attention(q, k, v, pos, 5),
                               rtol=1e-12, atol=1e-13)
    # decode: one row at position 4 over the full history
    np.testing.assert_allclose(oracle.attention(q[4:], k, v, pos[4:], 5),
                               brute_attention(q[4:], k, v, pos[4:], 5), rtol=1e-12, atol=1e-13)


def test_attention_matches_torch_sdpa_gqa():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(4)
    T, nq, nkv, D = 37, 8, 2, 16
    q = rng.standard_normal((T, nq, D))
    k = rng.standard_normal((nkv, T, D))
    v = rng.standard_normal((nkv, T, D))
    ours = oracle.attention(q, k, v, np.arange(T), T, block=8)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        is_causal=True, enable_gqa=True)[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(ours, ref, rtol=1e-11, atol=1e-12)


def test_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(5)
    T, nq, nkv, D = 9, 6, 3, 8
    q = rng.standard_normal((T, nq, D))
    k = rng.standard_normal((nkv, T, D))
    v = rng.standard_normal((nkv, T, D))
    rep = nq // nkv
    a = oracle.attention(q, k, v, np.arange(T), T)
    b = oracle.attention(q, np.repeat(k, rep, axis=0), np.repeat(v, rep, axis=0), np.arange(T), T)
    np.testing.assert_allclose(a, b, rtol=1e-14, atol=0)


def test_softmax_rows_and_causality():
    rng = np.random.default_rng(6)
    s = rng.standard_normal((4, 7))
    s[:, 5:] = -np.inf
    p = oracle.softmax_rows(s)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=1e-15)
    assert np.all(p[:, 5:] == 0)
    # changing the future leaves earlier rows bit-identical (whole model)
    m, _ = tiny_model()
    ids = synth.random_ids(0, 12, m.cfg.vocab)
    ids2 = ids.copy()
    ids2[8:] = (ids2[8:] + 1) % m.cfg.vocab
    s1, s2 = m.new_state(), m.new_state()
    x1 = m.forward(s1, m.embed(ids, None, 0), 0)
    x2 = m.forward(s2, m.embed(ids2, None, 0), 0)
    np.testing.assert_array_equal(x1[:8], x2[:8])
    assert not np.array_equal(x1[8:], x2[8:])


def test_silu_closed_form():
    z = np.array([0.0, 1.0, -1.0, 50.0, -800.0])
    out = oracle.silu(z)
    assert out[0] == 0.0
    assert math.isclose(out[1], 1 / (1 + math.exp(-1)), rel_tol=1e-15)
    assert math.isclose(out[2], -1 / (1 + math.e), rel_tol=1e-15)
    assert math.isclose(out[3], 50.0, rel_tol=1e-15)
    assert out[4] == 0.0


# --------------------------------------------------------- whole-block pins

def brute_block(x, P, T, cfg, eps, theta):
    """Independent pure-Python loops for one Qwen3 block on a fresh cache."""
    H, nq, nkv, D, F = cfg["H"], cfg["nq"], cfg["nkv"], cfg["D"], cfg["F"]

    def rms(vec, g):
        ms = sum(a * a for a in vec) / len(vec)
        r = 1.0 / math.sqrt(ms + eps)
        return [a * r * b for a, b in zip(vec, g)]

    def mv(W, vec):
        return [sum(W[r][c] * vec[c] for c in range(len(vec))) for r in range(len(W))]

    def rope(vec, p):
        half = D // 2
        out = list(vec)
        for j in range(half):
            a = p * theta ** (-2.0 * j / D)
            c, s = math.cos(a), math.sin(a)
            out[j] = vec[j] * c - vec[j + half] * s
            out[j + half] = vec[j + half] * c + vec[j] * s
        return out

    Q, K, V = [], [], []
    for t in range(T):
        xn = rms(x[t], P["in_norm"])
        q = mv(P["wq"], xn)
        k = mv(P["wk"], xn)
        v = mv(P["wv"], xn)
        Q.append([rope(rms(q[h * D:(h + 1) * D], P["q_norm"]), t) for h in range(nq)])
        K.append([rope(rms(k[g * D:(g + 1) * D], P["k_norm"]), t) for g in range(nkv)])
        V.append([v[g * D:(g + 1) * D] for g in range(nkv)])
    out = []
    for t in range(T):
        o = []
        for h in range(nq):
            g = h * nkv // nq
            sc = [sum(Q[t][h][d] * K[u][g][d] for d in range(D)) / math.sqrt(D) for u in range(t + 1)]
            m = max(sc)
            e = [math.exp(a - m) for a in sc]
            den = sum(e)
            o += [sum(e[u] / den * V[u][g][d] for u in range(t + 1)) for d in range(D)]
        x1 = [a + b for a, b in zip(x[t], mv(P["wo"], o))]
        xn = rms(x1, P["post_norm"])
        gt = mv(P["w_gate"], xn)
        up = mv(P["w_up"], xn)
        z = [a / (1 + math.exp(-a)) * b for a, b in zip(gt, up)]
        out.append([a + b for a, b in zip(x1, mv(P["w_down"], z))])
    return np.array(out)


def test_block_brute_force():
    shape = synth.custom_shape(hidden=8, n_layer=1, n_q_head=2, n_kv_head=1, head_dim=4, ffn=6, vocab=16)
    m, W = tiny_model(shape=shape, seed=11)
    x = synth.random_rows(7, 4, 8).astype(np.float64)
    st = m.new_state()
    ours = m.block(0, x, st, 0)
    P = {k: W.f32[f"L0.{k}"].astype(np.float64).tolist() for k in synth.LAYER_TENSORS}
    ref = brute_block(x.tolist(), P, 4, dict(H=8, nq=2, nkv=1, D=4, F=6), 1e-6, 1e6)
    np.testing.assert_allclose(ours, ref, rtol=1e-12, atol=1e-13)


# --------------------------------------------- library whole-model special case

def transformers_logits(m: oq.Qwen3Oracle, ids, audio, a0, forced):
    """Run transformers' Qwen3ForCausalLM (float64, eager attention) with the
    oracle's own parameters; returns [1 + len(forced), V] logits."""
    torch = pytest.importorskip("torch")
    tr = pytest.importorskip("transformers")
    c = m.cfg
    conf = tr.Qwen3Config(vocab_size=c.vocab, hidden_size=c.hidden, intermediate_size=c.ffn,
                          num_hidden_layers=c.n_layer, num_attention_heads=c.n_q_head,
                          num_key_value_heads=c.n_kv_head, head_dim=c.head_dim, rms_norm_eps=c.rms_eps,
                          rope_parameters={"rope_type": "default", "rope_theta": c.rope_theta},
                          tie_word_embeddings=True, attention_bias=False, max_position_embeddings=4096)
    conf._attn_implementation = "eager"
    model = tr.Qwen3ForCausalLM(conf).to(torch.float64).eval()
    sd = {"model.embed_tokens.weight": m.p["embed"], "model.norm.weight": m.p["final_norm"],
          "lm_head.weight": m.p["embed"]}
    names = {"in_norm": "input_layernorm.weight", "wq": "self_attn.q_proj.weight",
             "wk": "self_attn.k_proj.weight", "wv": "self_attn.v_proj.weight",
             "q_norm": "self_attn.q_norm.weight", "k_norm": "self_attn.k_norm.weight",
             "wo": "self_attn.o_proj.weight", "post_norm": "post_attention_layernorm.weight",
             "w_gate": "mlp.gate_proj.weight", "w_up": "mlp.up_proj.weight", "w_down": "mlp.down_proj.weight"}
    for i in range(c.n_layer):
        for k, n in names.items():
            sd[f"model.layers.{i}.{n}"] = m.p[f"L{i}.{k}"]
    model.load_state_dict({k: torch.from_numpy(np.array(v, dtype=np.float64)) for k, v in sd.items()})
    with torch.no_grad():
        emb = torch.from_numpy(m.embed(ids, audio, a0))[None]
        out = model(inputs_embeds=emb, use_cache=True)
        res = [out.logits[0, -1].numpy()]
        pkv = out.past_key_values
        for tok in forced:
            e = torch.from_numpy(m.embed(np.array([tok]), None, 0))[None]
            out = model(inputs_embeds=e, past_key_values=pkv, use_cache=True)
            pkv = out.past_key_values
            res.append(out.logits[0, -1].numpy())
    return np.stack(res)


def oracle_forced(m, ids, audio, a0, forced):
    st = m.new_state()
    res = [m.prefill(st, ids, audio, a0)]
    for i, tok in enumerate(forced):
        res.append(m.decode(st, int(tok), len(ids) + i))
    return np.stack(res)


def test_whole_model_matches_transformers_qwen3():
    m, _ = tiny_model()
    w = synth.WORKLOADS["tiny"]
    ids, audio, a0 = synth.make_prompt(w)
    forced = synth.random_ids(3, 6, m.cfg.vocab)
    ours = oracle_forced(m, ids, audio, a0, forced)
    ref = transformers_logits(m, ids, audio, a0, forced)
    # transformers evaluates RMSNorm and RoPE frequencies in float32
    np.testing.assert_allclose(ours, ref, rtol=0, atol=2e-5)


# ------------------------------------------------------------ state invariants

def test_kv_consistency_prefill_vs_decode():
    m, _ = tiny_model()
    ids = synth.random_ids(1, 20, m.cfg.vocab)
    audio = synth.random_rows(1, 6, m.cfg.hidden)
    s_full = m.new_state()
    full = m.prefill(s_full, ids, audio, 3)
    s = m.new_state()
    m.prefill(s, ids[:-1], audio, 3)
    inc = m.decode(s, int(ids[-1]), len(ids) - 1)
    np.testing.assert_allclose(inc, full, rtol=0, atol=1e-12)
    # prefill(T) + decode(t) == prefill(T + 1)
    ext = np.concatenate([ids, [7]]).astype(np.int32)
    s2 = m.new_state()
    ref = m.prefill(s2, ext, audio, 3)
    np.testing.assert_allclose(m.decode(s_full, 7, len(ids)), ref, rtol=0, atol=1e-12)
    for layer in range(m.cfg.n_layer):
        np.testing.assert_allclose(s_full.k[layer][:, :21], s2.k[layer][:, :21], atol=1e-12)


def test_override_identity():
    m, _ = tiny_model()
    ids = synth.random_ids(2, 16, m.cfg.vocab)
    rows = m.p["embed"][ids[4:10]]
    a = m.prefill(m.new_state(), ids, rows, 4)
    b = m.prefill(m.new_state(), ids, None, 0)
    np.testing.assert_array_equal(a, b)
    # ids under the span are ignored, even out of range
    ids2 = ids.copy()
    ids2[4:10] = 10 ** 6
    np.testing.assert_array_equal(m.prefill(m.new_state(), ids2, rows, 4), b)


def test_clone_and_batch_equivalence():
    m, _ = tiny_model()
    ids = synth.random_ids(4, 10, m.cfg.vocab)
    base = m.new_state()
    m.prefill(base, ids)
    branches = [base.clone() for _ in range(3)]
    toks = [3, 99, 512]
    batched = m.decode_many(branches, toks)
    for b, t in enumerate(toks):
        s = m.new_state()
        m.prefill(s, ids)
        np.testing.assert_allclose(batched[b], m.decode(s, t, 10), rtol=0, atol=1e-13)
    assert base.n_past == 10  # source untouched


def test_fp32_rerun_bounds_oracle_error():
    m64, W = tiny_model()
    m32 = oracle.Qwen3Oracle(m64.cfg, W.f32, dtype=np.float32)
    w = synth.WORKLOADS["tiny"]
    ids, audio, a0 = synth.make_prompt(w)
    forced = synth.random_ids(5, 8, m64.cfg.vocab)
    a = oracle_forced(m64, ids, audio, a0, forced)
    b = oracle_forced(m32, ids, audio, a0, forced)
    assert np.max(np.abs(a - b)) < 1e-5


def test_pick_token_ties_and_nan():
    assert oq.pick_token(np.array([0.5, 2.0, 2.0, 1.0])) == 1
    # values that differ in float64 but round to the same float32 tie -> lowest index
    a = np.array([1.0, 1.0 + 1e-12])
    assert oq.pick_token(a) == 0
    with pytest.raises(FloatingPointError):
        oq.pick_token(np.array([0.0, np.nan]))


def test_decode_rejects_wrong_position():
    m, _ = tiny_model()
    st = m.new_state()
    m.prefill(st, synth.random_ids(0, 4, m.cfg.vocab))
    with pytest.raises(ValueError):
        m.decode(st, 1, 5)
    with pytest.raises(ValueError):
        m.prefill(st, synth.random_ids(0, 4, m.cfg.vocab))


def test_metrics_hand_example():
    t = np.array([1.0, -2.0, 0.0, 4.0])
    c = np.array([1.5, -2.0, 0.5, 3.0])
    r = oracle.step_metrics(c, t)
    assert r["max_abs"] == 1.0
    assert r["mean_abs"] == 0.5
    assert math.isclose(r["rmse"], math.sqrt((0.25 + 0 + 0.25 + 1) / 4))
    assert math.isclose(r["mean_rel"], (0.5 + 0 + 0.5 / 1e-6 + 0.25) / 4)
    assert math.isclose(r["cosine"], (1.5 + 4 + 12) / (math.sqrt(21) * math.sqrt(2.25 + 4 + 0.25 + 9)))
    assert r["argmax_equal"] and r["teacher_top2_margin"] == 3.0
