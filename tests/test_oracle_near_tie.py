"""Pins of the oracle's near-tie rule (the exemption every GPU parity test
applies) and of the alternative outcome it names.

A near tie is a decision that a float32 implementation may take differently
from the float64 oracle: an accept test u < p/q with u within RATIO_EPS of
p/q, or an inverse-CDF draw whose threshold v*R lies within CDF_DELTA of a
boundary of the chosen token (or whose residual mass is below CDF_DELTA, or
that took the R = 0 fallback).  Each bound is pinned from both sides on
constructed infos, so a wrong sign, a wrong stage, a wrong position or a band
that is too wide fails here; the alternative outcome (the same decision taken
the other way) is pinned against the rule run with the uniform moved across
the boundary.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle.rule as rule
import oracle.verify as ov

EPS = 1e-5
DELTA = 1e-6


def chain(tests, draw=None):
    return dict(tests=list(tests), draw=draw)


def draw_info(R, t, c_lo, c_hi, fallback=False):
    d = dict(R=R, t=t, c_lo=c_lo, c_hi=c_hi)
    if fallback:
        d["fallback"] = True
    return d


def ev(info):
    return ov.near_tie_event(info, EPS, DELTA)


# --- accept tests -------------------------------------------------------------

@pytest.mark.parametrize("du,tie", [(-0.99e-5, True), (0.99e-5, True), (-1.01e-5, False),
                                    (1.01e-5, False), (0.0, True)])
def test_ratio_band_both_sides(du, tie):
    p, q = 0.25, 0.5                      # rho = 0.5 exactly
    e = ev(chain([(0.5 + du, p, q)]))
    assert (e is not None) == tie
    if tie:
        assert e["kind"] == "test" and e["flip"] == ("test", 0) and e["stage"] == 1


def test_ratio_uses_p_over_q_not_q_over_p():
    # rho = p/q = 0.2; q/p = 5 would never be near a uniform
    assert ev(chain([(0.2 + 0.3e-5, 0.1, 0.5)])) is not None
    # u near q/p - 4 = 1.0 (a shifted ratio) is far from rho
    assert ev(chain([(0.99999, 0.1, 0.5)])) is None


def test_position_of_the_first_tie():
    tests = [(0.9, 0.1, 0.2), (0.1, 0.7, 0.2), (0.3 + 0.5e-5, 0.3, 1.0), (0.5, 0.25, 0.5)]
    e = ev(chain(tests))
    assert e["flip"] == ("test", 2)


def test_decisions_that_do_not_depend_on_u():
    # p = 0 rejects for every u, q = 0 < p accepts for every u, p = q accepts
    # every u < 1: none of them is a tie, whatever u is
    for u in (0.0, 1e-7, 0.5, 1.0 - 2.0 ** -24):
        assert ev(chain([(u, 0.0, 0.3)])) is None
        assert ev(chain([(u, 0.0, 0.0)])) is None
        assert ev(chain([(u, 0.4, 0.0)])) is None
        assert ev(chain([(u, 0.3, 0.3)])) is None
    # and such a test really does not turn with u
    for u in (0.0, 0.999):
        assert not rule.accept(u, 0.0, 0.3)
        assert rule.accept(u, 0.4, 0.0)


def test_tiny_ratio_is_a_tie_only_for_tiny_u():
    # p/q = 1e-9: the test accepts only u = 0 (float64) -- a float32 p may
    # underflow to 0 and reject it
    assert ev(chain([(0.0, 1e-10, 0.1)])) is not None
    assert ev(chain([(2.0 ** -24 * 200, 1e-10, 0.1)])) is None


# --- draws ----------------------------------------------------------------------

@pytest.mark.parametrize("lo,hi,want", [
    (0.5e-6, 0.2, -1),     # threshold just above C(y-1): the token before may win
    (0.2, 0.5e-6, 1),      # threshold just below C(y): the token after may win
    (1.5e-6, 0.2, None),   # outside the band on the low side
    (0.2, 1.5e-6, None),   # outside the band on the high side
])
def test_cdf_boundary_band(lo, hi, want):
    t = 0.5
    e = ev(chain([(0.9, 0.1, 0.2)], draw_info(1.0, t, t - lo, t + hi)))
    if want is None:
        assert e is None
    else:
        assert e["kind"] == "boundary" and e["flip"] == ("draw", want)


def test_residual_mass_band():
    assert ev(chain([], draw_info(0.9e-6, 0.45e-6, 0.0, 0.9e-6)))["flip"] == ("draw", "p")
    # a mass of 5 delta with the threshold far from both boundaries: no tie
    assert ev(chain([], draw_info(5e-6, 2.5e-6, 0.0, 5e-6))) is None


def test_fallback_draw_is_unresolved():
    e = ev(chain([(0.9, 0.1, 0.2)], draw_info(0.3, 0.1, 0.0, 0.2, fallback=True)))
    assert e["kind"] == "fallback" and e["flip"] is None


def test_tests_come_before_the_draw():
    info = chain([(0.5 + 0.5e-5, 0.25, 0.5)], draw_info(1.0, 0.5, 0.5 - 1e-7, 0.6))
    assert ev(info)["kind"] == "test"


# --- the hierarchy ----------------------------------------------------------------

def test_stage_of_the_event():
    clean = chain([(0.9, 0.1, 0.2)], draw_info(1.0, 0.5, 0.1, 0.7))
    tied = chain([(0.5 + 0.5e-5, 0.25, 0.5)])
    assert ev(dict(stage1=clean, stage2=tied))["stage"] == 2
    assert ev(dict(stage1=tied, stage2=tied))["stage"] == 1
    assert ev(dict(stage1=clean, stage2=clean)) is None


def test_each_stage_uses_its_own_uniforms_and_ratios():
    # stage 1: u1 = 0.3 with rho1 = 0.8; stage 2: u2 = 0.8 with rho2 = 0.3.
    # Pairing u1 with rho2 (or u2 with rho1) would report a tie.
    s1 = chain([(0.3, 0.4, 0.5)])
    s2 = chain([(0.8, 0.15, 0.5)])
    assert ev(dict(stage1=s1, stage2=s2)) is None
    assert ev(chain([(0.3, 0.15, 0.5)])) is not None
    assert ev(chain([(0.8, 0.4, 0.5)])) is not None


# --- the alternative outcome ----------------------------------------------------------

def _dist(ws):
    a = np.array(ws, dtype=np.float64)
    return a / a.sum()


def test_flipped_test_equals_the_uniform_moved_across():
    """Flipping the accept test at j equals running the rule with u_j moved to
    the other side of p/q (accept -> reject and reject -> accept)."""
    rng = np.random.default_rng(3)
    V, k = 6, 3
    for trial in range(40):
        Q = [_dist(rng.random(V) + 0.05) for _ in range(k)]
        P = [_dist(rng.random(V) + 0.05) for _ in range(k + 1)]
        toks = [int(x) for x in rng.integers(0, V, k)]
        vs = rng.random(k + 1)
        j = int(rng.integers(0, k))
        us = rng.random(k + 1) * 0.2           # positions before j accept often
        rho = P[j][toks[j]] / Q[j][toks[j]]
        if rho >= 1.0:
            continue
        for side in (-1, 1):
            us[j] = rho + side * 1e-9          # near the boundary on one side
            base = rule.verify_chain(Q, P[:k], toks, us, vs, bonus_row=P[k])
            if base[0] < j:                    # stopped before j: nothing to flip there
                continue
            flipped = rule.verify_chain(Q, P[:k], toks, us, vs, bonus_row=P[k],
                                        flip=("test", j))
            us2 = us.copy()
            us2[j] = rho - side * 1e-9         # the other side
            moved = rule.verify_chain(Q, P[:k], toks, us2, vs, bonus_row=P[k])
            assert flipped[0] == moved[0] and flipped[1] == moved[1]
            assert flipped[1] != base[1] or flipped[0] != base[0]


def test_flipped_draw_equals_the_threshold_moved_across():
    """("draw", -1) equals the draw with v*R moved just below C(y-1), ("draw",
    +1) with v*R moved up to C(y); zero weights in between are skipped."""
    w = np.array([0.1, 0.0, 0.3, 0.0, 0.0, 0.2, 0.4])
    C = np.cumsum(w)
    R = C[-1]
    for y in (2, 5, 6):
        prev = max(i for i in range(y) if w[i] > 0)
        v = (C[y - 1] + 1e-12) / R             # just above C(y-1): picks y
        i0, _ = rule.draw(w, v)
        assert i0 == y
        i_lo, _ = rule.draw(w, v, shift=-1)
        j_lo, _ = rule.draw(w, (C[y - 1] - 1e-12) / R)
        assert i_lo == j_lo == prev
    for y in (0, 2, 5):
        nxt = min(i for i in range(y + 1, len(w)) if w[i] > 0)
        v = (C[y] - 1e-12) / R                 # just below C(y): picks y
        assert rule.draw(w, v)[0] == y
        i_hi, _ = rule.draw(w, v, shift=1)
        j_hi, _ = rule.draw(w, C[y] / R)       # at C(y): the next positive weight
        assert i_hi == j_hi == nxt
    # no neighbour: the pick stays
    assert rule.draw(w, 0.0, shift=-1)[0] == 0
    assert rule.draw(w, 0.999, shift=1)[0] == 6


def test_mass_flip_draws_from_p():
    P = _dist([1, 2, 3, 4])
    Q = P.copy()
    Q[1] -= 1e-7
    Q[2] += 1e-7                                # residual mass 1e-7
    a, e, info = rule.verify_chain([Q], [P], [2], [1.0 - 2.0 ** -24], [0.7], bonus_row=None)
    assert a == 0 and info["draw"]["R"] < DELTA
    a2, e2, _ = rule.verify_chain([Q], [P], [2], [1.0 - 2.0 ** -24], [0.7], bonus_row=None,
                                  flip=("draw", "p"))
    assert e2[-1] == rule.draw(P, 0.7)[0] and e2[-1] != e[-1]


def test_event_and_alternative_through_the_hierarchy():
    """A uniform planted next to stage 2's ratio at position 0: the event names
    stage 2, test 0, and the alternative is the run with that uniform moved
    across the ratio."""
    V, k = 5, 3
    rng = np.random.default_rng(11)
    Pd = [_dist(rng.random(V) + 0.1) for _ in range(k)]
    Pi = [_dist(rng.random(V) + 0.1) for _ in range(k + 1)]
    Pf = [_dist(rng.random(V) + 0.1) for _ in range(k + 1)]
    toks = [0, 1, 2]
    u1 = np.zeros(k + 1)                         # stage 1 accepts every draft it can
    v1 = np.full(k + 1, 0.37)
    v2 = np.full(k + 1, 0.61)
    found = 0
    for x in range(V):
        toks[0] = x
        rho2 = Pf[0][x] / Pi[0][x]
        if not (rho2 < 1.0) or Pd[0][x] > Pi[0][x] * 1e9:
            continue
        u2 = np.full(k + 1, 0.99)
        u2[0] = rho2 - 2e-6                      # accepts, by 2e-6
        a1, a2, em, info = ov.hier_chain(Pd, Pi, Pf, toks, u1, v1, u2, v2, 4)
        e = ov.near_tie_event(info, EPS, DELTA)
        assert e is not None and e["stage"] == 2 and e["flip"] == ("test", 0)
        alt = ov.hier_chain(Pd, Pi, Pf, toks, u1, v1, u2, v2, 4, flip=e)
        u2m = u2.copy()
        u2m[0] = rho2 + 2e-6                     # rejects
        moved = ov.hier_chain(Pd, Pi, Pf, toks, u1, v1, u2m, v2, 4)
        assert alt[:3] == moved[:3]
        assert alt[1] == 0 and a2 != 0
        found += 1
    assert found >= 2


def test_batch_functions_take_flips():
    """spec_verify_single with flips on one sequence changes that sequence only,
    and matches the per-sequence flipped run."""
    rng = np.random.default_rng(5)
    B, k, V = 3, 2, 7
    dl = rng.normal(0, 1, (B, k, V)).astype(np.float32)
    tl = rng.normal(0, 1, (B, k + 1, V)).astype(np.float32)
    tok = rng.integers(0, V, (B, k))
    base = ov.spec_verify_single(dl, tl, tok, None, 1, 2)
    flips = {1: dict(stage=1, kind="test", flip=("test", 0))}
    alt = ov.spec_verify_single(dl, tl, tok, None, 1, 2, flips=flips)
    for b in (0, 2):
        assert np.array_equal(alt["out_tokens"][b], base["out_tokens"][b])
    one = ov.verify_single_sequence(dl[1], tl[1], tok[1], 1.0, 1, 1, 2, flip=flips[1])
    assert alt["accept_len"][1] == one[0]
    assert base["accept_len"][1] != alt["accept_len"][1] or \
        not np.array_equal(base["out_tokens"][1], alt["out_tokens"][1])


def test_fraction_rows_still_work():
    """The exact-law tests drive the rule with Fraction rows: the flip
    argument leaves that path intact."""
    P = [np.array([Fraction(1, 2), Fraction(1, 2)], dtype=object)] * 2
    Q = [np.array([Fraction(1, 4), Fraction(3, 4)], dtype=object)]
    a, e, _ = rule.verify_chain(Q, P[:1], [1], [Fraction(9, 10)], [Fraction(1, 3)] * 2,
                                bonus_row=P[1])
    assert a == 0 and e == [0]
