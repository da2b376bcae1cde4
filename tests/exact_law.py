"""Exact output laws of the oracle's verification on tiny vocabularies.

Helper for the oracle pins.  The oracle is a sampling procedure driven by
uniforms; its exact output law is obtained by splitting each uniform's range
into the intervals on which the procedure's result is constant, calling the
oracle once at an interior point of every combination, and weighting by the
interval lengths (all in exact ``Fraction`` arithmetic).  The split points are
the ones the standard rule implies (p/q for an accept uniform, the normalised
CDF of the distribution being drawn for a draw uniform); an oracle whose result
is not constant on those intervals simply produces a wrong law, which the
closed-form comparisons then catch.
"""

from collections import defaultdict
from fractions import Fraction
from itertools import product

import numpy as np


def frac_rows(rows):
    return [np.array([Fraction(x) for x in r], dtype=object) for r in rows]


def random_dist(rng, V, denom=12, zeros=False):
    """A random rational distribution over V tokens (optionally with zeros)."""
    while True:
        w = rng.integers(0 if zeros else 1, denom, size=V)
        if w.sum() > 0:
            return np.array([Fraction(int(x), int(w.sum())) for x in w], dtype=object)


def _u_regions(p, q):
    """Intervals of the accept uniform: [0, min(1, p/q)) and the rest."""
    rho = Fraction(1) if q == 0 else min(Fraction(1), p / q)
    out = []
    if rho > 0:
        out.append((rho / 2, rho))
    if rho < 1:
        out.append(((rho + 1) / 2, 1 - rho))
    return out


def _v_regions(weights):
    """Intervals of the draw uniform between consecutive normalised CDF points."""
    C = np.cumsum(weights)
    R = C[-1]
    pts = sorted({Fraction(0), Fraction(1)} | {c / R for c in C if 0 < c / R < 1})
    return [((lo + hi) / 2, hi - lo) for lo, hi in zip(pts[:-1], pts[1:]) if hi > lo]


def _draw_vector(P, Q):
    r = np.maximum(P - Q, 0 * P[0])
    return r if sum(r) > 0 else P


def law_single(Q, P, chain):
    """Exact law of ``chain(Q, P[:k], x, us, vs, bonus_row=P[k])`` with x ~ prod Q_j.
    Returns {emitted tuple: probability}."""
    k, V = len(Q), len(P[0])
    law = defaultdict(Fraction)
    for x in product(range(V), repeat=k):
        px = Fraction(1)
        for j in range(k):
            px *= Q[j][x[j]]
        if px == 0:
            continue
        per_pos = [_u_regions(P[j][x[j]], Q[j][x[j]]) for j in range(k)]
        for combo in product(*per_pos):
            us = [c[0] for c in combo]
            wu = Fraction(1)
            for c in combo:
                wu *= c[1]
            a, _, _ = chain(Q, P[:k], list(x), us, [Fraction(1, 2)] * (k + 1), bonus_row=P[k])
            vec = _draw_vector(P[a], Q[a]) if a < k else P[k]
            for vm, wv in _v_regions(vec):
                vs = [vm] * (k + 1)
                _, emitted, _ = chain(Q, P[:k], list(x), us, vs, bonus_row=P[k])
                law[tuple(emitted)] += px * wu * wv
    return {e: p for e, p in law.items() if p != 0}


def closed_form_single(Q, P):
    """Law of the emitted sequence under the standard rule, written directly:
    m accepted drafts then a residual token (m < k), or k drafts and a bonus."""
    k, V = len(Q), len(P[0])
    law = {}
    for m in range(k + 1):
        for e in product(range(V), repeat=m + 1):
            pr = Fraction(1)
            for j in range(m):
                pr *= min(P[j][e[j]], Q[j][e[j]])
            pr *= max(Fraction(0), P[m][e[m]] - Q[m][e[m]]) if m < k else P[k][e[k]]
            if pr != 0:
                law[e] = pr
    return law


def completed_law(law, P, length):
    """Extend every emitted sequence with independent tokens e_m ~ P_m up to
    ``length`` tokens (the 'run the target alone afterwards' completion)."""
    out = defaultdict(Fraction)
    V = len(P[0])
    for e, pr in law.items():
        n = len(e)
        for tail in product(range(V), repeat=length - n):
            p = pr
            for i, tok in enumerate(tail):
                p *= P[n + i][tok]
            if p != 0:
                out[e + tail] += p
    return dict(out)


def product_law(P, length):
    """Law of ``length`` independent tokens e_m ~ P_m (autoregressive target
    alone, with position-indexed rows)."""
    V = len(P[0])
    out = {}
    for e in product(range(V), repeat=length):
        p = Fraction(1)
        for m, tok in enumerate(e):
            p *= P[m][tok]
        if p != 0:
            out[e] = p
    return out


def law_hier(Pd, Pi, Pf, window, hier):
    """Exact law of ``hier(Pd, Pi, Pf, x, u1, v1, u2, v2, window)`` with
    x ~ prod Pd_j."""
    k, V = len(Pd), len(Pi[0])
    law = defaultdict(Fraction)
    half = [Fraction(1, 2)] * (k + 1)
    zero = [Fraction(0)] * (k + 1)
    for x in product(range(V), repeat=k):
        px = Fraction(1)
        for j in range(k):
            px *= Pd[j][x[j]]
        if px == 0:
            continue
        per_pos = [_u_regions(Pi[j][x[j]], Pd[j][x[j]]) for j in range(k)]
        for combo in product(*per_pos):
            u1 = [c[0] for c in combo] + [Fraction(1, 2)]
            wu1 = Fraction(1)
            for c in combo:
                wu1 *= c[1]
            a1, _, _, _ = hier(Pd, Pi, Pf, list(x), u1, half, zero, zero, window)
            vec1 = _draw_vector(Pi[a1], Pd[a1]) if a1 < k else Pi[k]
            for v1m, wv1 in _v_regions(vec1):
                v1 = [v1m] * (k + 1)
                _, _, _, info = hier(Pd, Pi, Pf, list(x), u1, v1, zero, zero, window)
                t = info["tentative"]
                per2 = [_u_regions(Pf[j][t[j]], Pi[j][t[j]]) for j in range(len(t))]
                for combo2 in product(*per2):
                    u2 = [c[0] for c in combo2] + [Fraction(1, 2)] * (k + 1 - len(t))
                    wu2 = Fraction(1)
                    for c in combo2:
                        wu2 *= c[1]
                    _, a2, _, _ = hier(Pd, Pi, Pf, list(x), u1, v1, u2, half, window)
                    if a2 < len(t):
                        regions2 = _v_regions(_draw_vector(Pf[a2], Pi[a2]))
                    else:
                        regions2 = [(Fraction(1, 2), Fraction(1))]
                    for v2m, wv2 in regions2:
                        v2 = [v2m] * (k + 1)
                        _, _, e, _ = hier(Pd, Pi, Pf, list(x), u1, v1, u2, v2, window)
                        law[tuple(e)] += px * wu1 * wv1 * wu2 * wv2
    return {e: p for e, p in law.items() if p != 0}
