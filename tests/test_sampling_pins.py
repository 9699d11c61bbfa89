"""Pins of the sampling oracle (NCNN page "Qwen3ASR ncnn多平台移植", sections 1
and 6: greedy default, temperature, top-k, top-p, repetition penalty). Each
expected value is worked out by hand below or comes from torch's softmax /
topk / sort, not from the oracle's own code."""
import math

import numpy as np
import pytest

from oracle.sampling import SamplingParams, boundary_margin, penalize, sample

# probabilities 0.1, 0.2, 0.3, 0.4 at T = 1; candidate order 3, 2, 1, 0 with
# cumulative mass 0.4, 0.7, 0.9, 1.0
L4 = np.log(np.array([1.0, 2.0, 3.0, 4.0], dtype=np.float32)).astype(np.float32)


@pytest.mark.parametrize("u,tok", [(0.0, 3), (0.35, 3), (0.45, 2), (0.69, 2), (0.75, 1), (0.89, 1), (0.95, 0)])
def test_inverse_cdf_hand(u, tok):
    assert sample(L4, SamplingParams(temperature=1.0), u) == tok


@pytest.mark.parametrize("u,tok", [(0.5, 3), (0.56, 3), (0.6, 2), (0.99, 2)])
def test_top_p_hand(u, tok):
    # mass 0.4 < 0.6, 0.7 >= 0.6: keep {3, 2}, renormalised to 4/7, 3/7
    assert sample(L4, SamplingParams(temperature=1.0, top_p=0.6), u) == tok


@pytest.mark.parametrize("u,tok", [(0.5, 3), (0.6, 2)])
def test_top_k_hand(u, tok):
    assert sample(L4, SamplingParams(temperature=1.0, top_k=2), u) == tok
    assert sample(L4, SamplingParams(temperature=1.0, top_k=1), u) == 3


@pytest.mark.parametrize("u,tok", [(0.5, 3), (0.6, 2), (0.9, 1), (0.99, 0)])
def test_temperature_hand(u, tok):
    # T = 0.5 squares the odds: 1, 4, 9, 16 over 30; cumulative 16/30, 25/30, 29/30
    assert sample(L4, SamplingParams(temperature=0.5), u) == tok


def test_repetition_penalty_hand():
    z = np.array([2.0, -2.0, 1.0, 0.5], dtype=np.float32)
    got = penalize(z, [0, 1, 0], 2.0)
    assert got.tolist() == [1.0, -4.0, 1.0, 0.5]
    # greedy on the penalised values: 1.0 at ids 0 and 2, the lowest index wins
    assert sample(z, SamplingParams(temperature=0.0, repetition_penalty=2.0), 0.3, [0, 1, 0]) == 0
    assert sample(z, SamplingParams(temperature=0.0), 0.3) == 0
    # without penalty id 0 holds 2 / (2 + ...) of the largest mass at T = 1
    assert sample(z, SamplingParams(temperature=1.0), 0.0) == 0


def test_greedy_is_argmax():
    rng = np.random.default_rng(5)
    for _ in range(20):
        z = rng.standard_normal(300).astype(np.float32)
        assert sample(z, SamplingParams(temperature=0.0), 0.7) == int(np.argmax(z))


@pytest.mark.parametrize("T,k,p,rho", [(1.0, 0, 1.0, 1.0), (0.7, 20, 1.0, 1.0), (1.3, 0, 0.8, 1.0),
                                       (0.9, 40, 0.9, 1.3)])
def test_distribution_matches_torch(T, k, p, rho):
    """Over a grid of N uniforms each candidate is picked a number of times
    within 1 of N times its probability, the probabilities coming from torch's
    topk / sort / softmax on the penalised, tempered logits."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    V = 64
    z = (2.0 * rng.standard_normal(V)).astype(np.float32)
    hist = [3, 7, 7, 40]
    zt = torch.from_numpy(z.copy())
    if rho != 1.0:
        for t in set(hist):
            zt[t] = zt[t] / rho if zt[t] > 0 else zt[t] * rho
    zt = zt / torch.tensor(T, dtype=torch.float32)
    if k > 0:
        vals, idx = torch.topk(zt.double(), k)
    else:
        vals, idx = torch.sort(zt.double(), descending=True)
    probs = torch.softmax(vals, dim=0)
    if p < 1.0:
        cum = torch.cumsum(probs, dim=0)
        n = int(torch.searchsorted(cum, torch.tensor([p], dtype=torch.float64))[0]) + 1
        probs = probs[:n] / probs[:n].sum()
        idx = idx[:n]
    N = 4000
    counts = {}
    params = SamplingParams(temperature=T, top_k=k, top_p=p, repetition_penalty=rho)
    for j in range(N):
        t = sample(z, params, (j + 0.5) / N, hist)
        counts[t] = counts.get(t, 0) + 1
    assert set(counts) <= set(idx.tolist())
    for t, pr in zip(idx.tolist(), probs.tolist()):
        assert abs(counts.get(t, 0) - N * pr) <= 1.0 + 1e-9, (t, counts.get(t, 0), N * pr)


def test_margin_reports_near_boundary():
    # u * mass right on the boundary 0.4 between candidates 3 and 2
    assert boundary_margin(L4, SamplingParams(temperature=1.0), 0.4) < 1e-6
    assert boundary_margin(L4, SamplingParams(temperature=1.0), 0.55) == pytest.approx(0.15, abs=1e-6)
    assert math.isclose(boundary_margin(L4, SamplingParams(temperature=0.0), 0.4), 1.0)


def test_non_finite_logits_rejected():
    z = L4.copy()
    z[1] = np.nan
    with pytest.raises(FloatingPointError):
        sample(z, SamplingParams(temperature=1.0), 0.5)
