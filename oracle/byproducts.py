"""By-products of the verification stream: row entropies and the
verification-outcome export (float64).

Test infrastructure only (see ``oracle/__init__``).

Row entropy.  The Shannon entropy, in nats, of each streamed row's token
distribution (the softmax at the sequence's temperature, ``numerics``):
H = -sum_v P_v ln P_v with 0 ln 0 = 0; a greedy row (temperature 0, a one-hot)
has H = 0.  It is the signal an entropy-driven adaptive draft length keys on
("Optimierung der Inferenzgeschwindigkeit von Sprachmodellen durch spekulative
Dekodierung", mind-verse.de, the paragraphs on SVIP: the entropy of the draft's
token distribution measures the draft model's uncertainty and sets the draft
length).

Verification outcome.  For a tested position with draft distribution Q and
target distribution P (the rule in ``rule``):
  * beta = sum_v min(P_v, Q_v), the probability that the standard rule accepts
    a token drafted from Q there;
  * r = max(0, P - Q), the residual whose normalisation the correction token is
    drawn from (SSD summary section 3.B); r_v is the probability of rejecting
    at that position and correcting to v, and sum_v r_v = 1 - beta.
The export lists the m tokens with the largest r_v (ties: lower index first;
only r_v > 0), padded with token -1 and mass 0.  Together with beta (the
accepted length falls off geometrically with it) these are the likely
verification outcomes -- how many tokens are accepted and which token follows
-- that a speculation cache prepares for (SSD summary, section 2 items 1-2 and
section 3.A "Geometrischer Fan-out"; the residual, section 3.B).
"""

import numpy as np

from . import numerics


def entropy(P):
    """Shannon entropy (nats) of a distribution given as float64 probabilities."""
    P = np.asarray(P, dtype=np.float64)
    nz = P[P > 0]
    return float(-np.sum(nz * np.log(nz)))


def row_entropies(exit_logits, temperature):
    """Entropy of every row of one exit's raw logits [B, n, V]; temperature [B]
    (None = all 1).  Returns float64 [B, n]."""
    x = np.asarray(exit_logits)
    B, n = x.shape[0], x.shape[1]
    out = np.zeros((B, n))
    for b in range(B):
        tau = 1.0 if temperature is None else float(temperature[b])
        for j in range(n):
            out[b, j] = entropy(numerics.row_distribution(numerics.decode(x[b, j]), tau))
    return out


def accept_mass(P, Q):
    """beta = sum_v min(P_v, Q_v)."""
    return float(np.sum(np.minimum(np.asarray(P, np.float64), np.asarray(Q, np.float64))))


def residual_top(P, Q, m):
    """The m largest entries of r = max(0, P - Q): (tokens int64 [m], mass float64 [m]),
    largest first, ties to the lower index, padded with (-1, 0)."""
    r = np.maximum(np.asarray(P, np.float64) - np.asarray(Q, np.float64), 0.0)
    order = np.lexsort((np.arange(r.size), -r))   # primary: -r ascending, then index
    tok = np.full(m, -1, dtype=np.int64)
    mass = np.zeros(m)
    n = 0
    for v in order[:m]:
        if not r[v] > 0:
            break
        tok[n] = v
        mass[n] = r[v]
        n += 1
    return tok, mass


def outcome_export(exits, temperature, m):
    """Outcome export of a call.  ``exits`` = [draft, target] (single stage) or
    [L_d, L_i, L_f] (hierarchy) raw logits, draft [B, k, V], others [B, k+1, V].

    Returns (beta [B, 2, k+1], tokens [B, 2, k+1, m], mass [B, 2, k+1, m]).
    Stage 0 pairs (Q, P) = (draft or L_d row j, target or L_i row j) for j < k;
    stage 1 (hierarchy only) pairs (L_i row j, L_f row j) for j <= k.  Entries
    without a pair hold beta = NaN and the padding."""
    B, k = np.asarray(exits[0]).shape[0], np.asarray(exits[0]).shape[1]
    beta = np.full((B, 2, k + 1), np.nan)
    tok = np.full((B, 2, k + 1, m), -1, dtype=np.int64)
    mass = np.zeros((B, 2, k + 1, m))
    stages = [(0, 1, k)] + ([(1, 2, k + 1)] if len(exits) == 3 else [])
    for b in range(B):
        tau = 1.0 if temperature is None else float(temperature[b])
        for s, (eq, ep, n) in enumerate(stages):
            for j in range(n):
                Q = numerics.row_distribution(numerics.decode(np.asarray(exits[eq])[b, j]), tau)
                P = numerics.row_distribution(numerics.decode(np.asarray(exits[ep])[b, j]), tau)
                beta[b, s, j] = accept_mass(P, Q)
                tok[b, s, j], mass[b, s, j] = residual_top(P, Q, m)
    return beta, tok, mass
