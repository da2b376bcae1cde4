"""The speculative-sampling rule on one chain of drafted tokens.

Test infrastructure only (see ``oracle/__init__``).

Works on plain float64 NumPy rows and equally on object arrays of
``fractions.Fraction`` (the exact-law tests drive it that way), so nothing here
uses a float-only NumPy routine.

Rule (standard speculative sampling, whose losslessness the HiSpec summary
section 2 bullet "Verlustfreie Garantie" relies on in each of its two stages):

* position j with drafted token x, draft distribution Q_j, target P_j, uniform
  u: accept iff u * Q_j(x) < P_j(x), i.e. u < P/Q (probability min(1, P/Q));
  with Q_j(x) = 0 this accepts iff P_j(x) > 0.  A token outside the vocabulary
  has P = Q = 0 and is rejected;
* at the first rejected position a: resample from r = max(0, P_a - Q_a)
  (the residual "proportional to the difference of target and draft
  probabilities", SSD summary section 3.B); if r sums to zero draw from P_a;
* if every position is accepted and a bonus row is given: draw the bonus token
  from it (the "Bonus-Token", SSD summary section 2 item 1).
"""

import numpy as np


def prob_at(row, x):
    """Row probability at token x; 0 for tokens outside the vocabulary."""
    x = int(x)
    if 0 <= x < len(row):
        return row[x]
    return 0 * row[0]


def accept(u, p_x, q_x):
    """Accept iff u * q(x) < p(x)."""
    return bool(u * q_x < p_x)


def _neighbour(weights, i, step):
    """The nearest index before (step -1) or after (step +1) i with a positive
    weight; i itself when there is none."""
    j = i + step
    while 0 <= j < len(weights):
        if weights[j] > 0:
            return j
        j += step
    return i


def draw(weights, v, shift=0):
    """Inverse-CDF draw from a non-negative weight vector with uniform v in [0,1).

    C(i) = sum of weights[0..i] (sequential, index order), R = C(V-1).
    Returns (index, info) with index = the smallest i such that C(i) > v * R.
    If rounding leaves no such i, the largest i with a positive weight is
    taken.  Returns (None, info) when R == 0.
    info = dict(R, t=v*R, c_lo=C(i-1), c_hi=C(i)) for the parity exemptions.

    ``shift`` = -1 / +1 takes, instead, the nearest index before / after that
    one with a positive weight (the other side of a CDF boundary the threshold
    lies next to); info still describes the inverse-CDF pick.
    """
    C = np.cumsum(weights)
    R = C[-1]
    if not R > 0:
        return None, dict(R=R, t=0 * R, c_lo=0 * R, c_hi=0 * R)
    t = v * R
    above = np.nonzero(C > t)[0]
    if above.size:
        i = int(above[0])
    else:
        i = int(np.nonzero(weights > 0)[0][-1])
    c_lo = C[i - 1] if i > 0 else 0 * R
    info = dict(R=R, t=t, c_lo=c_lo, c_hi=C[i])
    if shift:
        i = _neighbour(weights, i, shift)
    return i, info


def residual(P, Q):
    """r = max(0, P - Q), element-wise."""
    return np.maximum(P - Q, 0 * P[0])


def verify_chain(Q_rows, P_rows, tokens, us, vs, bonus_row=None, window=None, flip=None):
    """Verify drafted ``tokens`` (length n) against (Q_j, P_j), j < n.

    Positions are visited in windows of ``window`` consecutive positions (all of
    them at once when None); within the call the result does not depend on the
    window size -- a window only groups tests.

    ``flip`` takes one decision the other way, which gives the outcome an
    implementation that rounds differently reaches at a near tie:
    ("test", j) inverts the accept test at position j; ("draw", -1) or
    ("draw", +1) takes the nearest token before or after the inverse-CDF pick
    that has a positive weight; ("draw", "p") draws from P_a as the R = 0
    fallback does.  None: the rule as stated.

    Returns (a, emitted, info):
      a       number of accepted leading tokens (first rejection, else n);
      emitted tokens[:a] + [correction] on a rejection, tokens + [bonus] when
              all were accepted and ``bonus_row`` is given, else tokens;
      info    per tested position (u, p, q) and the draw info (or None).
    """
    n = len(tokens)
    if window is not None and int(window) < 1:
        raise ValueError("window must be >= 1")
    w = max(n, 1) if window is None else int(window)
    flip_test = flip[1] if flip is not None and flip[0] == "test" else None
    flip_draw = flip[1] if flip is not None and flip[0] == "draw" else None
    tests = []
    a = n
    start = 0
    while start < n and a == n:
        for j in range(start, min(start + w, n)):
            p_x = prob_at(P_rows[j], tokens[j])
            q_x = prob_at(Q_rows[j], tokens[j])
            tests.append((us[j], p_x, q_x))
            ok = accept(us[j], p_x, q_x)
            if j == flip_test:
                ok = not ok
            if not ok:
                a = j
                break
        start += w
    emitted = [int(t) for t in tokens[:a]]
    draw_info = None
    shift = flip_draw if flip_draw in (-1, 1) else 0
    if a < n:
        if flip_draw == "p":
            y, draw_info = draw(P_rows[a], vs[a])
            draw_info["fallback"] = True
        else:
            y, draw_info = draw(residual(P_rows[a], Q_rows[a]), vs[a], shift)
            if y is None:
                y, draw_info = draw(P_rows[a], vs[a], shift)
                draw_info["fallback"] = True
        emitted.append(y)
    elif bonus_row is not None:
        y, draw_info = draw(bonus_row, vs[n], shift)
        emitted.append(y)
    return a, emitted, dict(tests=tests, draw=draw_info)
