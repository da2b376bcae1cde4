"""Pins of the cross-call tentative buffering oracle (CPU).

* Exact law (Fractions): two rounds of the intermediate verification, then a
  flush against the final exit, with stationary distributions: the emitted
  sequence completed by independent final-exit tokens has exactly the law of
  the final exit run alone (lossless), for several vocabularies and laws.
* A round followed by a flush with the same Philox offset equals the pinned
  one-call hierarchical verification on the same rows.
* Chi-square of the emitted stream of a long buffered run against the final
  exit; L_f == L_i accepts every pending token; state bookkeeping.
"""

from collections import defaultdict
from fractions import Fraction
from itertools import product

import numpy as np
import pytest
from scipy import stats

import oracle.rule as rule
import oracle.verify as ov
from oracle import numerics, tentative as ot
from tests import exact_law as X


def _round_law(Pd, Pi):
    """Exact law of one round's appended tokens (k = 1, drafted x ~ Pd)."""
    return X.law_single([Pd], [Pi, Pi], rule.verify_chain)


def _flush_law(pend, Pi, Pf):
    """Exact law of the flush's emitted tokens for a fixed pending sequence."""
    c = len(pend)
    law = defaultdict(Fraction)
    per_pos = [X._u_regions(Pf[t], Pi[t]) for t in pend]
    for combo in product(*per_pos):
        us = [cc[0] for cc in combo]
        wu = Fraction(1)
        for cc in combo:
            wu *= cc[1]
        a2, _, _ = ot.flush_chain(pend, [Pi] * c, [Pf] * c, us, [Fraction(1, 2)] * c)
        if a2 == c:
            law[tuple(pend)] += wu
            continue
        vec = X._draw_vector(Pf, Pi)
        for vm, wv in X._v_regions(vec):
            _, emitted, _ = ot.flush_chain(pend, [Pi] * c, [Pf] * c, us, [vm] * c)
            law[tuple(emitted)] += wu * wv
    return law


@pytest.mark.parametrize("seed", range(4))
def test_two_rounds_then_flush_is_lossless_exact(seed):
    rng = np.random.default_rng(seed)
    V = 3
    Pd = X.random_dist(rng, V, zeros=seed == 1)
    Pi = X.random_dist(rng, V, zeros=seed == 2)
    Pf = X.random_dist(rng, V)
    r1 = _round_law(Pd, Pi)
    law = defaultdict(Fraction)
    for t1, p1 in r1.items():
        for t2, p2 in r1.items():
            for e, p3 in _flush_law(list(t1) + list(t2), Pi, Pf).items():
                law[e] += p1 * p2 * p3
    L = 4
    done = X.completed_law(dict(law), [Pf] * L, L)
    assert done == X.product_law([Pf] * L, L)
    assert sum(law.values()) == 1


def test_planted_mistake_breaks_the_exact_law(monkeypatch):
    """A flush that (wrongly) tests against L_d instead of L_i is not lossless."""
    rng = np.random.default_rng(0)
    V = 3
    Pd, Pi, Pf = (X.random_dist(rng, V) for _ in range(3))
    r1 = _round_law(Pd, Pi)
    law = defaultdict(Fraction)
    for t1, p1 in r1.items():
        for e, p3 in _flush_law(list(t1), Pd, Pf).items():
            law[e] += p1 * p3
    assert X.completed_law(dict(law), [Pf] * 2, 2) != X.product_law([Pf] * 2, 2)


def _random_logits(rng, B, k, V, dt=np.float32):
    ld = rng.normal(0, 2, (B, k, V))
    li = rng.normal(0, 2, (B, k + 1, V))
    li[:, :k] = 0.9 * ld + 0.3 * li[:, :k]
    lf = 0.9 * li + 0.3 * rng.normal(0, 2, (B, k + 1, V))
    return ld.astype(dt), li.astype(dt), lf.astype(dt)


@pytest.mark.parametrize("tau", [1.0, 0.0])
def test_round_then_flush_equals_one_call_hierarchy(tau):
    rng = np.random.default_rng(4)
    B, k, V = 32, 5, 30
    ld, li, lf = _random_logits(rng, B, k, V)
    temps = np.full(B, tau)
    tokens = rng.integers(0, V, (B, k))
    if tau == 0.0:
        tokens[::2] = ld[::2].argmax(-1)
    st = ot.TentativeState(B)
    a1, _ = ot.tentative_round(st, ld, li, tokens, temps, seed=9, offset=3)
    f = ot.tentative_flush(st, lf, temps, seed=9, offset=3, min_pending=1)
    h = ov.spec_verify_hier(ld, li, lf, tokens, temps, seed=9, offset=3, window=4)
    assert (a1 == h["accept_len_inter"]).all()
    assert (f["accept_len"] == h["accept_len_final"]).all()
    assert (f["num_emitted"] == h["num_emitted"]).all()
    assert (f["out_tokens"] == h["out_tokens"]).all()
    assert (st.count() == 0).all()


def test_buffered_stream_is_the_final_exit():
    """Stationary rows, rounds until N_i = 4 tokens are pending, then a flush:
    the emitted stream is i.i.d. from the final exit (unigram and bigram
    chi-square)."""
    rng = np.random.default_rng(12)
    V, k, B, N_i = 8, 3, 400, 4
    ld = rng.normal(0, 1.5, V).astype(np.float32)
    li = (0.8 * ld + 0.6 * rng.normal(0, 1.5, V)).astype(np.float32)
    lf = (0.7 * li + 0.714 * rng.normal(0, 1.5, V)).astype(np.float32)
    Pd = numerics.row_distribution(ld, 1.0)
    Pf = numerics.row_distribution(lf, 1.0)
    st = ot.TentativeState(B)
    streams = [[] for _ in range(B)]
    LD = np.broadcast_to(ld, (B, k, V))
    LI = np.broadcast_to(li, (B, k + 1, V))
    LF = np.broadcast_to(lf, (B, N_i + k + 1, V))
    offset = 0
    for it in range(40):
        active = st.count() < N_i
        tokens = rng.choice(V, size=(B, k), p=Pd)
        ot.tentative_round(st, LD, LI, tokens, None, seed=1, offset=offset, active=active)
        offset += 1
        f = ot.tentative_flush(st, LF, None, seed=1, offset=offset, min_pending=N_i)
        offset += 1
        for b in np.nonzero(f["flushed"])[0]:
            streams[b].extend(f["out_tokens"][b, :f["num_emitted"][b]].tolist())
    stream = np.concatenate([np.array(s, dtype=np.int64) for s in streams])
    assert len(stream) > 20000
    uni = np.bincount(stream, minlength=V)
    assert stats.chisquare(uni, uni.sum() * Pf).pvalue > 1e-3
    pairs = np.concatenate([np.array(s[: len(s) // 2 * 2]).reshape(-1, 2) for s in streams])
    bi = np.bincount(pairs[:, 0] * V + pairs[:, 1], minlength=V * V)
    assert stats.chisquare(bi, bi.sum() * np.outer(Pf, Pf).ravel()).pvalue > 1e-3


def test_final_equal_intermediate_accepts_all_pending():
    rng = np.random.default_rng(5)
    B, k, V = 16, 4, 25
    ld, li, _ = _random_logits(rng, B, k, V)
    st = ot.TentativeState(B)
    for off in range(3):
        ot.tentative_round(st, ld, li, rng.integers(0, V, (B, k)), None, seed=2, offset=off)
    pend = [list(t) for t in st.tokens]
    rows = [list(r) for r in st.rows]
    width = max(len(p) for p in pend) + 1
    lf = np.zeros((B, width, V), dtype=np.float32)
    for b in range(B):
        for j, r in enumerate(rows[b]):
            lf[b, j] = r
    f = ot.tentative_flush(st, lf, None, seed=2, offset=9, min_pending=1)
    for b in range(B):
        assert f["accept_len"][b] == len(pend[b])
        assert f["out_tokens"][b, :f["num_emitted"][b]].tolist() == pend[b]
        assert f["num_drop"][b] == 0


def test_state_bookkeeping():
    """Appended rows are the round's L_i rows 0..a1, inactive sequences and
    sequences below the flush threshold are left alone, a rejection discards
    the pending tokens from a2 on."""
    rng = np.random.default_rng(6)
    B, k, V = 12, 4, 20
    ld, li, lf = _random_logits(rng, B, k, V)
    active = np.arange(B) % 3 != 0
    st = ot.TentativeState(B)
    a1, _ = ot.tentative_round(st, ld, li, rng.integers(0, V, (B, k)), None, seed=0, offset=0,
                               active=active)
    for b in range(B):
        if not active[b]:
            assert a1[b] == -1 and st.tokens[b] == []
            continue
        assert len(st.tokens[b]) == a1[b] + 1
        for j in range(a1[b] + 1):
            assert np.array_equal(st.rows[b][j], li[b, j])
    counts = st.count()
    f = ot.tentative_flush(st, lf, None, seed=0, offset=1, min_pending=3)
    for b in range(B):
        if counts[b] < 3 or counts[b] == 0:
            assert not f["flushed"][b] and f["num_emitted"][b] == 0
            assert len(st.tokens[b]) == counts[b]
        else:
            a2 = f["accept_len"][b]
            assert f["flushed"][b] and len(st.tokens[b]) == 0
            assert f["num_drop"][b] == (counts[b] - a2 if a2 < counts[b] else 0)
            assert f["num_emitted"][b] == (a2 + 1 if a2 < counts[b] else counts[b])
