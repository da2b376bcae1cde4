"""Pins of the oracle's hierarchical L_d -> L_i -> L_f verification.

Losslessness (HiSpec summary section 2, bullet "Verlustfreie Garantie": the
final output equals the final exit run alone) exactly on V = 4, a chi-square of
the emitted stream against the final exit, the reductions the composition must
satisfy, and window-size invariance within a call (bullet "Dynamische
Verifizierungsrichtlinie").
"""

import numpy as np
import pytest
from scipy import stats

import oracle.rule as rule
import oracle.verify as ov
from oracle import numerics
from tests import exact_law as X


def _rows(rng, n, V, zeros=False):
    return [X.random_dist(rng, V, zeros=zeros) for _ in range(n)]


@pytest.mark.parametrize("k,seed,window", [(1, 0, 4), (2, 1, 4), (2, 2, 1), (2, 3, 2)])
def test_hier_lossless_exact(k, seed, window):
    rng = np.random.default_rng(seed)
    V = 4
    Pd = _rows(rng, k, V)
    Pi = _rows(rng, k + 1, V, zeros=(seed % 2 == 0))
    Pf = _rows(rng, k + 1, V, zeros=(seed % 2 == 1))
    law = X.law_hier(Pd, Pi, Pf, window, ov.hier_chain)
    assert sum(law.values()) == 1
    assert X.completed_law(law, Pf, k + 1) == X.product_law(Pf, k + 1)


def test_hier_planted_mistake_is_detected(monkeypatch):
    """Testing stage 2 against the draft exit instead of the intermediate exit
    breaks losslessness (mistake planted in a copy of the composition)."""
    rng = np.random.default_rng(9)
    k, V = 2, 4
    Pd = _rows(rng, k, V)
    Pi = _rows(rng, k + 1, V)
    Pf = _rows(rng, k + 1, V)

    def wrong(Pd_, Pi_, Pf_, tokens, u1, v1, u2, v2, window):
        a1, t, i1 = rule.verify_chain(Pd_, Pi_[:k], list(tokens), u1, v1, bonus_row=Pi_[k])
        q = [Pd_[j] if j < k else Pi_[j] for j in range(a1 + 1)]
        a2, e, i2 = rule.verify_chain(q, Pf_[:a1 + 1], t, u2, v2, window=window)
        return a1, a2, e, dict(stage1=i1, stage2=i2, tentative=t)

    law = X.law_hier(Pd, Pi, Pf, 4, wrong)
    assert X.completed_law(law, Pf, k + 1) != X.product_law(Pf, k + 1)


def test_hier_chi_square_stream_is_final_exit():
    rng = np.random.default_rng(77)
    V, k, B = 8, 4, 25000
    ld = rng.normal(0, 1.5, V).astype(np.float32)
    li = (0.8 * ld + 0.6 * rng.normal(0, 1.5, V)).astype(np.float32)
    lf = (0.7 * li + 0.714 * rng.normal(0, 1.5, V)).astype(np.float32)
    Pd = numerics.row_distribution(ld, 1.0)
    Pf = numerics.row_distribution(lf, 1.0)
    tokens = rng.choice(V, size=(B, k), p=Pd)
    res = ov.spec_verify_hier(np.broadcast_to(ld, (B, k, V)), np.broadcast_to(li, (B, k + 1, V)),
                              np.broadcast_to(lf, (B, k + 1, V)), tokens, None, seed=11,
                              offset=5, window=4)
    n = res["num_emitted"]
    stream = np.concatenate([res["out_tokens"][b, :n[b]] for b in range(B)])
    uni = np.bincount(stream, minlength=V)
    assert stats.chisquare(uni, uni.sum() * Pf).pvalue > 1e-3
    m = (len(stream) // 2) * 2
    bi = np.bincount(stream[0:m:2] * V + stream[1:m:2], minlength=V * V)
    assert stats.chisquare(bi, bi.sum() * np.outer(Pf, Pf).ravel()).pvalue > 1e-3
    a1, a2 = res["accept_len_inter"], res["accept_len_final"]
    assert (n == np.minimum(a1, a2) + 1).all()
    assert (res["num_drop"] == k - (n - 1)).all()


def _random_logits(rng, B, k, V):
    ld = rng.normal(0, 2, (B, k, V)).astype(np.float32)
    li = rng.normal(0, 2, (B, k + 1, V)).astype(np.float32)
    li[:, :k] = 0.9 * ld + 0.3 * li[:, :k]
    lf = (0.9 * li + 0.3 * rng.normal(0, 2, (B, k + 1, V))).astype(np.float32)
    tokens = rng.integers(0, V, (B, k))
    return ld, li.astype(np.float32), lf, tokens


def test_final_equal_intermediate_reduces_to_single_stage():
    """L_f == L_i: stage 2 accepts every tentative token, so the output is the
    single-stage verify of L_d against L_i with the same stage-0 uniforms."""
    rng = np.random.default_rng(3)
    B, k, V = 24, 5, 40
    ld, li, _, tokens = _random_logits(rng, B, k, V)
    h = ov.spec_verify_hier(ld, li, li, tokens, None, seed=5, offset=2)
    s = ov.spec_verify_single(ld, li, tokens, None, seed=5, offset=2)
    assert (h["out_tokens"] == s["out_tokens"]).all()
    assert (h["accept_len_inter"] == s["accept_len"]).all()
    assert (h["accept_len_final"] == h["accept_len_inter"] + 1).all()


def test_intermediate_equal_draft_accepts_all_drafts():
    rng = np.random.default_rng(4)
    B, k, V = 24, 4, 40
    ld, li, lf, tokens = _random_logits(rng, B, k, V)
    li[:, :k] = ld
    h = ov.spec_verify_hier(ld, li, lf, tokens, None, seed=1, offset=0)
    assert (h["accept_len_inter"] == k).all()


@pytest.mark.parametrize("tau", [1.0, 0.0])
def test_window_size_does_not_change_the_result(tau):
    rng = np.random.default_rng(12)
    B, k, V = 40, 6, 30
    ld, li, lf, tokens = _random_logits(rng, B, k, V)
    temps = np.full(B, tau)
    ref = ov.spec_verify_hier(ld, li, lf, tokens, temps, seed=2, offset=9, window=k + 1)
    for w in (1, 2, 4):
        r = ov.spec_verify_hier(ld, li, lf, tokens, temps, seed=2, offset=9, window=w)
        for key in ("out_tokens", "accept_len_inter", "accept_len_final", "num_emitted"):
            assert (r[key] == ref[key]).all()


def test_hier_temperature_zero_is_two_argmax_prefix_matches():
    rng = np.random.default_rng(13)
    B, k, V = 50, 4, 12
    ld, li, lf, _ = _random_logits(rng, B, k, V)
    tokens = ld.argmax(-1)
    h = ov.spec_verify_hier(ld, li, lf, tokens, np.zeros(B), seed=0, offset=0)
    for b in range(B):
        ai = [int(np.argmax(li[b, j])) for j in range(k + 1)]
        af = [int(np.argmax(lf[b, j])) for j in range(k + 1)]
        a1 = 0
        while a1 < k and tokens[b, a1] == ai[a1]:
            a1 += 1
        t = list(tokens[b, :a1]) + [ai[a1]]
        a2 = 0
        while a2 < len(t) and t[a2] == af[a2]:
            a2 += 1
        e = t if a2 == len(t) else t[:a2] + [af[a2]]
        assert h["accept_len_inter"][b] == a1 and h["accept_len_final"][b] == a2
        assert list(h["out_tokens"][b, :len(e)]) == e
