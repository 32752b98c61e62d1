"""Pins of the sampling oracle (oracle/sampling.py) to facts other than
itself: closed forms on hand-made rows, scipy's softmax, a pure-Python
sort-and-accumulate nucleus, stratified-grid counts of the inverse-CDF draw,
and the speculative-sampling identity (the emitted token follows the target
distribution exactly), checked by enumeration.  CPU only."""
import math

import numpy as np
import pytest
import scipy.special
import torch

from oracle import sampling as S
from oracle.decoder import accept_length, argmax_lowest

F64 = torch.float64


def t(x):
    return torch.tensor(x, dtype=F64)


def test_temperature_zero_is_greedy_lowest_index():
    p = S.sampling_probs(t([0.5, 2.0, -1.0, 2.0]), 0.0)
    assert p.tolist() == [0.0, 1.0, 0.0, 0.0]
    assert S.sample(t([0.5, 2.0, -1.0, 2.0]), 0.999, 0.0) == 1


def test_no_truncation_is_scipy_softmax():
    rng = np.random.default_rng(1)
    x = rng.normal(size=300) * 3
    for T in (0.3, 1.0, 1.7):
        p = S.sampling_probs(torch.from_numpy(x), T, 0, 1.0).numpy()
        assert np.abs(p - scipy.special.softmax(x / T)).max() < 1e-15
        p2 = S.sampling_probs(torch.from_numpy(x), T, 300, 1.0).numpy()  # k = V keeps everything
        assert np.abs(p2 - p).max() == 0.0


def test_top_k_hand_value_keeps_ties_at_the_cut():
    # z = [2, 1, 0, 0, -1]; the 3rd largest is 0, tied by index 3: four kept
    p = S.sampling_probs(t([2.0, 1.0, 0.0, 0.0, -1.0]), 1.0, 3, 1.0).numpy()
    den = math.e ** 2 + math.e + 2.0
    assert np.abs(p - np.array([math.e ** 2 / den, math.e / den, 1 / den, 1 / den, 0.0])).max() < 1e-15
    p1 = S.sampling_probs(t([0.1, 0.7, -0.2]), 0.5, 1, 1.0)
    assert p1.tolist() == [0.0, 1.0, 0.0]


def test_top_p_hand_values():
    logits = torch.log(t([0.15, 0.5, 0.05, 0.3]))
    # running mass by decreasing probability: 0.5, 0.8, 0.95, 1.0
    assert (S.sampling_probs(logits, 1.0, 0, 0.45).numpy() > 0).tolist() == [False, True, False, False]
    p = S.sampling_probs(logits, 1.0, 0, 0.79).numpy()
    assert np.abs(p - np.array([0.0, 0.625, 0.0, 0.375])).max() < 1e-12
    assert (S.sampling_probs(logits, 1.0, 0, 0.85).numpy() > 0).tolist() == [True, True, False, True]
    # top-k then top-p: k = 3 drops 0.05 first, renormalised mass 0.5/0.95 ...
    p = S.sampling_probs(logits, 1.0, 3, 0.55).numpy()
    assert (p > 0).tolist() == [False, True, False, True]


def _nucleus_brute(probs, top_p):
    """Plain Python: sort (prob desc, index asc), accumulate until the mass
    reaches top_p; the cut is the probability reached there; keep all >= cut."""
    order = sorted(range(len(probs)), key=lambda i: (-probs[i], i))
    run = 0.0
    cut = probs[order[-1]]
    for i in order:
        run += probs[i]
        if run >= top_p:
            cut = probs[i]
            break
    return [p >= cut for p in probs]


@pytest.mark.parametrize("seed", range(6))
def test_top_p_against_brute_force(seed):
    rng = np.random.default_rng(seed)
    x = rng.normal(size=64) * 2
    x[5] = x[9]  # a tie
    for top_p in (0.1, 0.5, 0.9, 0.99):
        base = scipy.special.softmax(x / 0.8)
        keep = _nucleus_brute(list(base), top_p)
        p = S.sampling_probs(torch.from_numpy(x), 0.8, 0, top_p).numpy()
        assert (p > 0).tolist() == keep
        ref = np.where(keep, base, 0.0)
        assert np.abs(p - ref / ref.sum()).max() < 1e-14


def test_draw_on_a_stratified_grid_matches_probabilities():
    rng = np.random.default_rng(3)
    p = scipy.special.softmax(rng.normal(size=40))
    n = 20000
    counts = np.zeros(40)
    for j in range(n):
        counts[S.draw(torch.from_numpy(p), (j + 0.5) / n)] += 1
    assert np.abs(counts - n * p).max() <= 1.0 + 1e-9


def _rand_dist(rng, V, zeros=0):
    p = rng.random(V) ** 3
    if zeros:
        p[rng.choice(V, zeros, replace=False)] = 0.0
    return p / p.sum()


@pytest.mark.parametrize("seed", range(8))
def test_speculative_identity_by_enumeration(seed):
    """P(emitted = t) = min(p, q)(t) + (1 - sum min(p, q)) residual(t) = p(t)."""
    rng = np.random.default_rng(seed)
    V = 12
    p = _rand_dist(rng, V, zeros=seed % 3)
    q = _rand_dist(rng, V, zeros=(seed + 1) % 4)
    assert np.abs(S.emitted_distribution(p, q) - p).max() < 1e-15
    # a draft equal to the target: every draft accepted, nothing from the residual
    assert np.abs(S.emitted_distribution(p, p) - p).max() < 1e-15


def test_speculative_greedy_reduces_to_the_greedy_verify_rule():
    rng = np.random.default_rng(7)
    V, K = 50, 5
    for trial in range(20):
        tl = torch.from_numpy(rng.normal(size=(K + 1, V)))
        dl = torch.from_numpy(rng.normal(size=(K, V)))
        greedy = [argmax_lowest(tl[i]) for i in range(K + 1)]
        drafts = [greedy[i] if rng.random() < 0.6 else int(rng.integers(V)) for i in range(K)]
        res = S.spec_accept(tl, dl, drafts, rng.random(K), rng.random(K + 1), 0.0)
        m = accept_length([0] + drafts, greedy)
        assert res["accepted"] == m
        assert res["token"] == greedy[m]


def test_speculative_first_token_frequencies():
    """Monte Carlo over seeded uniforms: the first emitted token of a K = 2
    round follows the target row 0's sampling distribution (chi-square)."""
    rng = np.random.default_rng(11)
    V = 6
    tl = torch.from_numpy(rng.normal(size=(3, V)))
    dl = torch.from_numpy(rng.normal(size=(2, V)))
    pq = [S.sampling_probs(dl[i], 0.9) for i in range(2)]
    n = 6000
    counts = np.zeros(V)
    for _ in range(n):
        d1 = S.draw(pq[0], rng.random())
        d2 = S.draw(pq[1], rng.random())
        res = S.spec_accept(tl, dl, [d1, d2], rng.random(2), rng.random(3), 0.9)
        counts[d1 if res["accepted"] >= 1 else res["token"]] += 1
    p0 = S.sampling_probs(tl[0], 0.9).numpy()
    chi2 = float(((counts - n * p0) ** 2 / (n * p0)).sum())
    assert chi2 < 20.5  # 5 degrees of freedom, p = 0.001
