"""Pins of the oracle's speculative-sampling rule (single stage).

Exact laws on V = 4 with rational distributions (every draft sequence
enumerated), the lossless criterion of the HiSpec summary (section 2, bullet
"Verlustfreie Garantie": output identical to the target model run alone), a
chi-square test of the emitted stream on V = 8, the acceptance-length closed
form, p == q, temperature 0 and the inverse-CDF draw against NumPy's
searchsorted.  A planted mistake shows the exact tests have power.
"""

from fractions import Fraction

import numpy as np
import pytest
from scipy import stats

import oracle.rule as rule
import oracle.verify as ov
from oracle import numerics, philox
from tests import exact_law as X


def _rows(rng, n, V, zeros=False):
    return [X.random_dist(rng, V, zeros=zeros) for _ in range(n)]


@pytest.mark.parametrize("k,seed", [(1, 0), (2, 1), (2, 2), (3, 3)])
def test_exact_law_matches_closed_form(k, seed):
    rng = np.random.default_rng(seed)
    V = 4
    Q = _rows(rng, k, V, zeros=(seed % 2 == 0))
    P = _rows(rng, k + 1, V, zeros=(seed % 2 == 1))
    law = X.law_single(Q, P, rule.verify_chain)
    assert law == X.closed_form_single(Q, P)
    assert sum(law.values()) == 1


@pytest.mark.parametrize("k,seed", [(1, 10), (2, 11), (3, 12)])
def test_lossless_completion_is_target_law(k, seed):
    rng = np.random.default_rng(seed)
    V = 4
    Q = _rows(rng, k, V)
    P = _rows(rng, k + 1, V, zeros=True)
    law = X.law_single(Q, P, rule.verify_chain)
    assert X.completed_law(law, P, k + 1) == X.product_law(P, k + 1)


def test_planted_mistake_is_detected(monkeypatch):
    """Drawing the correction from P instead of max(0, P - Q) must break both
    exact checks (the mistake is planted in the oracle, on the CPU)."""
    rng = np.random.default_rng(5)
    k, V = 2, 4
    Q = _rows(rng, k, V)
    P = _rows(rng, k + 1, V)
    monkeypatch.setattr(rule, "residual", lambda P_, Q_: P_)
    law = X.law_single(Q, P, rule.verify_chain)
    assert law != X.closed_form_single(Q, P)
    assert X.completed_law(law, P, k + 1) != X.product_law(P, k + 1)


def test_planted_accept_mistake_is_detected(monkeypatch):
    rng = np.random.default_rng(6)
    k, V = 2, 4
    Q = _rows(rng, k, V)
    P = _rows(rng, k + 1, V)
    monkeypatch.setattr(rule, "accept", lambda u, p, q: bool(u < p))
    law = X.law_single(Q, P, rule.verify_chain)
    assert X.completed_law(law, P, k + 1) != X.product_law(P, k + 1)


def _stationary_logits(rng, V, scale):
    return rng.normal(0.0, scale, size=V).astype(np.float32)


def test_chi_square_emitted_stream_is_target():
    """V = 8, k = 4, stationary rows: every emitted token (concatenated over
    calls, as a decoder appends them) is i.i.d. from P; unigram (df 7) and
    bigram (df 63) chi-square, plus
    the first emitted token alone, at alpha = 1e-3."""
    rng = np.random.default_rng(123)
    V, k, B = 8, 4, 40000
    lq = _stationary_logits(rng, V, 1.5)
    lp = (0.6 * lq + 0.8 * _stationary_logits(rng, V, 1.5)).astype(np.float32)
    Q = numerics.row_distribution(lq, 1.0)
    P = numerics.row_distribution(lp, 1.0)
    draft = np.broadcast_to(lq, (B, k, V))
    target = np.broadcast_to(lp, (B, k + 1, V))
    tokens = rng.choice(V, size=(B, k), p=Q)
    res = ov.spec_verify_single(draft, target, tokens, None, seed=7, offset=3)
    n = res["num_emitted"]
    stream = np.concatenate([res["out_tokens"][b, :n[b]] for b in range(B)])
    uni = np.bincount(stream, minlength=V)
    assert stats.chisquare(uni, uni.sum() * P).pvalue > 1e-3
    first = np.bincount(res["out_tokens"][:, 0], minlength=V)
    assert stats.chisquare(first, first.sum() * P).pvalue > 1e-3
    # bigrams over the whole stream (pairs across call boundaries included: the
    # calls concatenate into one decoded sequence); non-overlapping pairs so the
    # counts are multinomial
    m = (len(stream) // 2) * 2
    bi = np.bincount(stream[0:m:2] * V + stream[1:m:2], minlength=V * V)
    assert stats.chisquare(bi, bi.sum() * np.outer(P, P).ravel()).pvalue > 1e-3
    # acceptance length: E[a] = sum_{m=1..k} beta^m, beta = sum min(P, Q)
    beta = np.minimum(P, Q).sum()
    expect = sum(beta ** m for m in range(1, k + 1))
    a = res["accept_len"].astype(np.float64)
    assert abs(a.mean() - expect) < 4 * a.std() / np.sqrt(B)


def test_identical_rows_accept_everything():
    """p == q: p/q is exactly 1, so every draft is accepted (u < 1 always)
    and the bonus token is drawn from the last target row."""
    rng = np.random.default_rng(1)
    B, k, V = 16, 6, 300
    logits = rng.normal(0, 3, size=(B, k + 1, V)).astype(np.float32)
    tokens = rng.integers(0, V, size=(B, k))
    res = ov.spec_verify_single(logits[:, :k], logits, tokens, None, seed=3, offset=0)
    assert (res["accept_len"] == k).all()
    assert (res["num_emitted"] == k + 1).all()
    assert (res["out_tokens"][:, :k] == tokens).all()
    for b in range(B):
        _, v = philox.uniforms(np.uint64(k), b, philox.STAGE_SINGLE, 0, 3)
        P = numerics.row_distribution(logits[b, k], 1.0)
        cdf = np.cumsum(P)
        assert res["out_tokens"][b, k] == np.searchsorted(cdf, v * cdf[-1], side="right")


def test_temperature_zero_is_argmax_prefix_match():
    rng = np.random.default_rng(2)
    B, k, V = 64, 5, 50
    draft = rng.normal(0, 1, size=(B, k, V)).astype(np.float32)
    target = rng.normal(0, 1, size=(B, k + 1, V)).astype(np.float32)
    # make target argmax agree with the draft argmax for a random prefix
    tokens = draft.argmax(-1)
    for b in range(B):
        m = rng.integers(0, k + 1)
        for j in range(m):
            target[b, j, tokens[b, j]] = target[b, j].max() + 1.0
    # ties: a duplicated maximum must resolve to the lowest index
    target[0, 0, :] = 0.0
    target[0, 0, [7, 3]] = 2.0
    tokens[0, 0] = 7
    res = ov.spec_verify_single(draft, target, tokens, np.zeros(B), seed=0, offset=0)
    for b in range(B):
        amax = [int(np.argmax(target[b, j])) for j in range(k + 1)]
        a = 0
        while a < k and tokens[b, a] == amax[a]:
            a += 1
        assert res["accept_len"][b] == a
        assert list(res["out_tokens"][b, :a + 1]) == list(tokens[b, :a]) + [amax[a]]
    assert res["accept_len"][0] == 0 and res["out_tokens"][0, 0] == 3


def test_draw_matches_searchsorted():
    rng = np.random.default_rng(4)
    for _ in range(300):
        V = int(rng.integers(1, 200))
        w = rng.exponential(size=V) * (rng.random(V) < 0.7)
        if w.sum() == 0:
            continue
        v = float(rng.integers(0, 2 ** 24)) * 2.0 ** -24
        i, info = rule.draw(w, v)
        C = np.cumsum(w)
        j = int(np.searchsorted(C, v * C[-1], side="right"))
        if j >= V:            # rounding overrun: last positive weight
            j = int(np.nonzero(w)[0][-1])
        assert i == j
        assert info["c_lo"] <= info["t"] < info["c_hi"] or j == int(np.nonzero(w)[0][-1])


def test_zero_draft_probability_and_out_of_vocab():
    P = np.array([0.5, 0.5, 0.0])
    Q = np.array([1.0, 0.0, 0.0])
    assert rule.accept(0.99, rule.prob_at(P, 1), rule.prob_at(Q, 1))      # q = 0, p > 0
    assert not rule.accept(0.0, rule.prob_at(P, 2), rule.prob_at(Q, 2))   # q = 0, p = 0
    assert not rule.accept(0.0, rule.prob_at(P, 3), rule.prob_at(Q, 3))   # token >= V
    assert not rule.accept(0.0, rule.prob_at(P, -1), rule.prob_at(Q, -1))


def test_residual_zero_falls_back_to_target():
    P = [np.array([0.25, 0.75])]
    Q = [np.array([0.25, 0.75])]
    # force a rejection with u = 1 (never produced by the 24-bit generator)
    a, emitted, info = rule.verify_chain(Q, P, [1], [1.0], [0.5], bonus_row=np.array([1.0, 0]))
    assert a == 0 and info["draw"]["fallback"] and emitted == [1]


def test_fraction_and_float_paths_agree():
    rng = np.random.default_rng(8)
    k, V = 3, 5
    Qf = [rng.dirichlet(np.ones(V)) for _ in range(k)]
    Pf = [rng.dirichlet(np.ones(V)) for _ in range(k + 1)]
    Qx = X.frac_rows(Qf)
    Px = X.frac_rows(Pf)
    for _ in range(50):
        x = list(rng.integers(0, V, size=k))
        us = list(rng.random(k + 1))
        vs = list(rng.random(k + 1))
        r1 = rule.verify_chain(Qf, Pf[:k], x, us, vs, bonus_row=Pf[k])
        r2 = rule.verify_chain(Qx, Px[:k], x, [Fraction(u) for u in us],
                               [Fraction(v) for v in vs], bonus_row=Px[k])
        assert r1[0] == r2[0] and r1[1] == r2[1]


def test_no_drafts_draws_the_bonus():
    """k = 0: nothing to verify, the bonus token is drawn from P_0."""
    P0 = np.array([0.1, 0.6, 0.3])
    for v, want in ((0.05, 0), (0.1, 1), (0.69, 1), (0.7, 2), (0.999, 2)):
        a, emitted, _ = rule.verify_chain([], [], [], [0.5], [v], bonus_row=P0)
        assert a == 0 and emitted == [want]
