"""Pins of the by-product oracle (CPU): row entropies and the
verification-outcome export.

Entropy is pinned by closed forms (a constant row has ln V; a row with two
logit levels has ln(V/2) plus the binary entropy of the logistic of the gap)
and by scipy's entropy of scipy's softmax.  The acceptance mass and the
residual are pinned by the exact output law of the already pinned rule
(enumeration with Fractions): the probability of accepting position 0 and the
probability of each correction token there.
"""

import numpy as np
import pytest
import scipy.special
import scipy.stats

from oracle import byproducts, rule, numerics
from tests.exact_law import law_single, random_dist


def _binary_entropy(x):
    return -x * np.log(x) - (1 - x) * np.log1p(-x)


@pytest.mark.parametrize("V", [1, 7, 1024, 128256])
@pytest.mark.parametrize("tau", [0.5, 1.0, 3.0])
def test_constant_row_has_log_v(V, tau):
    row = np.full(V, 2.5, dtype=np.float32)
    H = byproducts.entropy(numerics.row_distribution(numerics.decode(row), tau))
    assert H == pytest.approx(np.log(V), rel=1e-12, abs=1e-12)


@pytest.mark.parametrize("n,gap,tau", [(1, 1.0, 1.0), (5, 2.0, 0.7), (64, -3.0, 1.3), (500, 0.25, 2.0)])
def test_two_level_row_closed_form(n, gap, tau):
    rng = np.random.default_rng(n)
    row = np.concatenate([np.full(n, 1.0 + gap), np.full(n, 1.0)])[rng.permutation(2 * n)]
    H = byproducts.entropy(numerics.row_distribution(row, tau))
    p_hi = 1.0 / (1.0 + np.exp(-gap / tau))
    assert H == pytest.approx(np.log(n) + _binary_entropy(p_hi), rel=1e-12, abs=1e-12)


def test_matches_scipy_on_random_rows():
    rng = np.random.default_rng(3)
    for V, tau in [(10, 1.0), (1000, 0.7), (32000, 1.0), (4096, 2.5)]:
        row = (rng.standard_normal(V) * 3).astype(np.float32)
        H = byproducts.entropy(numerics.row_distribution(numerics.decode(row), tau))
        ref = scipy.stats.entropy(scipy.special.softmax(row.astype(np.float64) / tau))
        assert H == pytest.approx(ref, rel=1e-10, abs=1e-12)


def test_greedy_and_limits():
    row = np.array([0.0, 3.0, 1.0, 3.0, -2.0])
    assert byproducts.entropy(numerics.row_distribution(row, 0.0)) == 0.0
    # tau -> 0+: the two tied maxima share the mass; tau -> inf: uniform
    assert byproducts.entropy(numerics.row_distribution(row, 1e-3)) == pytest.approx(np.log(2), abs=1e-9)
    assert byproducts.entropy(numerics.row_distribution(row, 1e6)) == pytest.approx(np.log(5), abs=1e-6)


def test_row_entropies_layout_and_temperature():
    """Row (b, j) has two levels with gap (b + 1) * (j + 1) / 4; sequence b's
    temperature applies to all its rows."""
    B, n, half = 3, 4, 8
    taus = np.array([1.0, 0.5, 0.0], dtype=np.float32)
    x = np.zeros((B, n, 2 * half), dtype=np.float32)
    for b in range(B):
        for j in range(n):
            x[b, j, :half] = (b + 1) * (j + 1) / 4
    H = byproducts.row_entropies(x, taus)
    assert H.shape == (B, n)
    for b in range(B):
        for j in range(n):
            if taus[b] == 0:
                # ties among the top level: the greedy row is a one-hot
                assert H[b, j] == 0.0
                continue
            p_hi = 1.0 / (1.0 + np.exp(-((b + 1) * (j + 1) / 4) / float(taus[b])))
            assert H[b, j] == pytest.approx(np.log(half) + _binary_entropy(p_hi), rel=1e-12)
    assert np.allclose(byproducts.row_entropies(x, None)[1], [
        np.log(half) + _binary_entropy(1 / (1 + np.exp(-2 * (j + 1) / 4))) for j in range(n)])


@pytest.mark.parametrize("seed", range(6))
def test_exact_law_of_position_zero(seed):
    """beta is the exact probability that the rule accepts a draft from Q, and
    r_v the exact probability that it rejects and emits v (k = 1)."""
    rng = np.random.default_rng(seed)
    V = 5
    Q = random_dist(rng, V, zeros=seed % 2 == 1)
    P = random_dist(rng, V, zeros=seed % 3 == 1)
    bonus = random_dist(rng, V)
    law = law_single([Q], [P, bonus], rule.verify_chain)
    accepted = sum(p for e, p in law.items() if len(e) == 2)
    Pf = np.array([float(x) for x in P])
    Qf = np.array([float(x) for x in Q])
    assert byproducts.accept_mass(Pf, Qf) == pytest.approx(float(accepted), abs=1e-14)
    tok, mass = byproducts.residual_top(Pf, Qf, V)
    corr = {e[0]: p for e, p in law.items() if len(e) == 1}
    expect = sorted(corr.items(), key=lambda kv: (-kv[1], kv[0]))
    assert [int(t) for t in tok if t >= 0] == [v for v, _ in expect]
    for (v, p), m in zip(expect, mass):
        assert m == pytest.approx(float(p), abs=1e-14)
    assert np.all(mass[len(expect):] == 0) and np.all(tok[len(expect):] == -1)


def test_total_variation_identity():
    rng = np.random.default_rng(11)
    for V in (3, 100, 5000):
        P = scipy.special.softmax(rng.standard_normal(V) * 2)
        Q = scipy.special.softmax(rng.standard_normal(V) * 2)
        assert byproducts.accept_mass(P, Q) == pytest.approx(1 - 0.5 * np.abs(P - Q).sum(), abs=1e-12)
        _, mass = byproducts.residual_top(P, Q, V)
        assert mass.sum() == pytest.approx(1 - byproducts.accept_mass(P, Q), abs=1e-12)


def test_identical_and_disjoint():
    P = np.array([0.5, 0.25, 0.0, 0.25])
    tok, mass = byproducts.residual_top(P, P, 3)
    assert byproducts.accept_mass(P, P) == 1.0
    assert list(tok) == [-1, -1, -1] and list(mass) == [0, 0, 0]
    Q = np.array([0.0, 0.0, 1.0, 0.0])
    assert byproducts.accept_mass(P, Q) == 0.0
    tok, mass = byproducts.residual_top(P, Q, 4)
    assert list(tok) == [0, 1, 3, -1] and list(mass) == [0.5, 0.25, 0.25, 0.0]


def test_ties_go_to_the_lower_index():
    P = np.array([0.1, 0.2, 0.1, 0.2, 0.4])
    Q = np.array([0.0, 0.0, 0.0, 0.0, 1.0])
    tok, _ = byproducts.residual_top(P, Q, 3)
    assert list(tok) == [1, 3, 0]


def test_outcome_export_layout():
    """Greedy sequences make every entry exact: beta = [argmax Q == argmax P]
    and the residual is the one-hot of argmax P when they differ."""
    B, k, V, m = 2, 3, 6, 2
    amax = {  # exit -> [B, positions] argmax tokens
        0: np.array([[0, 1, 2], [5, 5, 5]]),
        1: np.array([[0, 2, 2, 3], [5, 4, 5, 1]]),
        2: np.array([[1, 2, 0, 3], [5, 4, 4, 1]]),
    }
    exits = []
    for e, n in [(0, k), (1, k + 1), (2, k + 1)]:
        x = np.zeros((B, n, V), dtype=np.float32)
        for b in range(B):
            for j in range(n):
                x[b, j, amax[e][b, j]] = 4.0
        exits.append(x)
    taus = np.zeros(B, dtype=np.float32)
    beta, tok, mass = byproducts.outcome_export(exits, taus, m)
    assert beta.shape == (B, 2, k + 1) and tok.shape == (B, 2, k + 1, m)
    for b in range(B):
        for s, (q, p, n) in enumerate([(0, 1, k), (1, 2, k + 1)]):
            for j in range(k + 1):
                if j >= n:
                    assert np.isnan(beta[b, s, j]) and list(tok[b, s, j]) == [-1] * m
                    continue
                same = amax[q][b, j] == amax[p][b, j]
                assert beta[b, s, j] == (1.0 if same else 0.0)
                assert list(tok[b, s, j]) == ([-1, -1] if same else [amax[p][b, j], -1])
                assert list(mass[b, s, j]) == ([0, 0] if same else [1.0, 0])
    # the single-stage export fills stage 0 only
    beta1, tok1, _ = byproducts.outcome_export(exits[:2], taus, m)
    assert np.array_equal(beta1[:, 0], beta[:, 0], equal_nan=True)
    assert np.all(np.isnan(beta1[:, 1])) and np.all(tok1[:, 1] == -1)


def test_planted_mistake_is_detected(monkeypatch):
    """A swapped min/max in the acceptance mass breaks the exact-law pin."""
    monkeypatch.setattr(byproducts, "accept_mass",
                        lambda P, Q: float(np.sum(np.maximum(P, Q))))
    with pytest.raises(AssertionError):
        test_exact_law_of_position_zero(0)
