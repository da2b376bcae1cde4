"""Batched single-stage and hierarchical (L_d -> L_i -> L_f) verification.

Test infrastructure only (see ``oracle/__init__``).

Sequences are independent (per-sequence acceptance without padding, HiSpec
summary section 2 bullet "Unterstuetzung fuer Batch-Inferenz"), so every batch
function is a plain loop over sequences calling ``rule.verify_chain``.

Single stage (drafts x_0..x_{k-1}, draft rows Q_0..Q_{k-1}, target rows
P_0..P_k): the standard rule with the bonus row P_k; uniforms from Philox
stage 0.

Hierarchical (HiSpec summary section 2 "Kernmechanismus" and bullets
"Verlustfreie Garantie", "Dynamische Verifizierungsrichtlinie"), the reading
taken where the summary is silent:

1. stage 1 is the standard rule with draft L_d and target L_i (rows
   Pd_0..Pd_{k-1}, Pi_0..Pi_k, Philox stage 0): a1 accepted drafts, then the
   L_i correction (a1 < k) or the L_i bonus (a1 = k); the tentative sequence is
   t = (x_0..x_{a1-1}, y), |t| = a1 + 1, distributed exactly as L_i would
   have produced it;
2. stage 2 is the standard rule again, with t as the draft, q = Pi_j and the
   final exit as target p = Pf_j, j = 0..a1, visited in windows of N_i
   positions (Philox stage 1); a2 = first rejection, else a1 + 1; on a
   rejection the L_f correction is drawn from max(0, Pf_a2 - Pi_a2); no L_f
   bonus is drawn (the final exit's distribution after t is not an input);
3. n = min(a1, a2) + 1 tokens are emitted; kept = n - 1 drafted KV slots stay
   valid and num_drop = k - kept are rolled back.

Temperature applies to every exit of a sequence; 0 means greedy.
"""

import numpy as np

from . import numerics, philox, rule


def _rows(raw_rows, tau):
    return [numerics.row_distribution(numerics.decode(r), tau) for r in raw_rows]


def _uniform_vectors(n, b, stage, offset, seed):
    j = np.arange(n, dtype=np.uint64)
    return philox.uniforms(j, b, stage, offset, seed)


def verify_single_sequence(draft_raw, target_raw, tokens, tau, b, seed, offset, flip=None):
    """One sequence of the single-stage verify.  draft_raw [k, V], target_raw
    [k+1, V] raw logits; returns (a, emitted, info).  ``flip``: a near-tie
    event (``near_tie_event``) whose decision is taken the other way."""
    k = len(tokens)
    Q = _rows(draft_raw, tau)
    P = _rows(target_raw, tau)
    us, vs = _uniform_vectors(k + 1, b, philox.STAGE_SINGLE, offset, seed)
    return rule.verify_chain(Q, P[:k], list(tokens), us, vs, bonus_row=P[k],
                             flip=flip["flip"] if flip else None)


def verify_hier_sequence(ld_raw, li_raw, lf_raw, tokens, tau, b, seed, offset, window,
                         flip=None):
    """One sequence of the hierarchical verify.  Returns (a1, a2, emitted, info).
    ``flip``: a near-tie event (``near_tie_event``) taken the other way."""
    k = len(tokens)
    Pd = _rows(ld_raw, tau)
    Pi = _rows(li_raw, tau)
    Pf = _rows(lf_raw, tau)
    u1, v1 = _uniform_vectors(k + 1, b, philox.STAGE_SINGLE, offset, seed)
    u2, v2 = _uniform_vectors(k + 1, b, philox.STAGE_FINAL, offset, seed)
    return hier_chain(Pd, Pi, Pf, tokens, u1, v1, u2, v2, window, flip)


def hier_chain(Pd, Pi, Pf, tokens, u1, v1, u2, v2, window, flip=None):
    """The two stages on distributions (float64 or Fraction rows) and explicit
    uniforms (u1, v1 for stage 1 and u2, v2 for stage 2, indexed by position).
    ``flip``: a near-tie event of stage 1 or 2 taken the other way.
    Returns (a1, a2, emitted, info)."""
    k = len(tokens)
    f1 = flip["flip"] if flip and flip["stage"] == 1 else None
    f2 = flip["flip"] if flip and flip["stage"] == 2 else None
    a1, t, info1 = rule.verify_chain(Pd, Pi[:k], list(tokens), u1, v1, bonus_row=Pi[k], flip=f1)
    a2, emitted, info2 = rule.verify_chain(Pi[:a1 + 1], Pf[:a1 + 1], t, u2, v2,
                                           bonus_row=None, window=window, flip=f2)
    return a1, a2, emitted, dict(stage1=info1, stage2=info2, tentative=t)


def _pad(emitted, width):
    out = np.full(width, -1, dtype=np.int32)
    out[:len(emitted)] = emitted
    return out


def spec_verify_single(draft_logits, target_logits, draft_tokens, temperature,
                       seed, offset, sequences=None, flips=None):
    """Batched single-stage verify.

    draft_logits [B, k, V], target_logits [B, k+1, V] raw (uint16 bf16 bits or
    float32); draft_tokens [B, k] int; temperature [B] float or None (all 1).
    ``sequences`` restricts the work to a subset of b (outputs of the others
    are left at -1); ``flips`` maps a sequence to a near-tie event taken the
    other way there.  Returns a dict of arrays plus per-sequence infos.
    """
    B, k, _ = draft_logits.shape
    temps = np.ones(B) if temperature is None else np.asarray(temperature, dtype=np.float64)
    seqs = range(B) if sequences is None else sequences
    accept_len = np.full(B, -1, dtype=np.int32)
    num_emitted = np.full(B, -1, dtype=np.int32)
    out_tokens = np.full((B, k + 1), -1, dtype=np.int32)
    infos = {}
    for b in seqs:
        a, emitted, info = verify_single_sequence(draft_logits[b], target_logits[b],
                                                  draft_tokens[b], temps[b], b, seed, offset,
                                                  (flips or {}).get(b))
        accept_len[b] = a
        num_emitted[b] = len(emitted)
        out_tokens[b] = _pad(emitted, k + 1)
        infos[b] = info
    return dict(accept_len=accept_len, num_emitted=num_emitted, out_tokens=out_tokens,
                num_drop=np.where(num_emitted >= 0, k - (num_emitted - 1), -1).astype(np.int32),
                infos=infos)


def spec_verify_hier(ld_logits, li_logits, lf_logits, draft_tokens, temperature,
                     seed, offset, window=4, sequences=None, flips=None):
    """Batched hierarchical verify.  ld [B, k, V], li/lf [B, k+1, V];
    ``sequences`` and ``flips`` as in ``spec_verify_single``."""
    B, k, _ = ld_logits.shape
    temps = np.ones(B) if temperature is None else np.asarray(temperature, dtype=np.float64)
    seqs = range(B) if sequences is None else sequences
    a1s = np.full(B, -1, dtype=np.int32)
    a2s = np.full(B, -1, dtype=np.int32)
    num_emitted = np.full(B, -1, dtype=np.int32)
    out_tokens = np.full((B, k + 1), -1, dtype=np.int32)
    infos = {}
    for b in seqs:
        a1, a2, emitted, info = verify_hier_sequence(ld_logits[b], li_logits[b], lf_logits[b],
                                                     draft_tokens[b], temps[b], b, seed,
                                                     offset, window, (flips or {}).get(b))
        a1s[b], a2s[b] = a1, a2
        num_emitted[b] = len(emitted)
        out_tokens[b] = _pad(emitted, k + 1)
        infos[b] = info
    return dict(accept_len_inter=a1s, accept_len_final=a2s, num_emitted=num_emitted,
                out_tokens=out_tokens,
                num_drop=np.where(num_emitted >= 0, k - (num_emitted - 1), -1).astype(np.int32),
                infos=infos)


def _chain_event(info, ratio_eps, cdf_delta):
    """First near tie of one chain, in the order the rule takes its decisions:
    the accept tests by position, then the draw."""
    for j, (u, p, q) in enumerate(info["tests"]):
        # p = 0 rejects and q = 0 < p accepts whatever u is; p = q accepts
        # every u < 1; otherwise the test turns at u = p / q
        if p > 0 and q > 0 and p != q and abs(u - p / q) < ratio_eps:
            return dict(kind="test", flip=("test", j))
    d = info["draw"]
    if d is None:
        return None
    if d.get("fallback"):
        # R = 0 here; a float32 R may come out positive, and its draw from the
        # rounding residue is not predictable
        return dict(kind="fallback", flip=None)
    if d["R"] < cdf_delta:
        # a float32 R may round to 0 and take the fallback draw from p
        return dict(kind="mass", flip=("draw", "p"))
    lo, hi = d["t"] - d["c_lo"], d["c_hi"] - d["t"]
    if lo < cdf_delta or hi < cdf_delta:
        return dict(kind="boundary", flip=("draw", -1 if lo <= hi else 1))
    return None


def near_tie_event(info, ratio_eps=1e-5, cdf_delta=1e-6):
    """The first decision of a sequence at which a float32 implementation and
    this float64 one may legitimately part: an accept test with
    |u - p/q| < ratio_eps (p, q > 0, p != q), or a draw whose threshold v*R lies
    within cdf_delta (probability units) of either CDF boundary of the chosen
    token, whose residual mass is below cdf_delta, or that took the R = 0
    fallback.  Returns None, or dict(stage (1 or 2; 1 for a single chain),
    kind, flip): ``flip`` is the decision taken the other way (see
    ``rule.verify_chain``), None where the other outcome is not one token.
    Accepts the info of one chain or of a hierarchy."""
    if "stage1" in info:
        for stage, key in ((1, "stage1"), (2, "stage2")):
            ev = _chain_event(info[key], ratio_eps, cdf_delta)
            if ev is not None:
                ev["stage"] = stage
                return ev
        return None
    ev = _chain_event(info, ratio_eps, cdf_delta)
    if ev is not None:
        ev["stage"] = 1
    return ev


def near_tie(info, ratio_eps=1e-5, cdf_delta=1e-6):
    """True when a sequence has a near tie (``near_tie_event``)."""
    return near_tie_event(info, ratio_eps, cdf_delta) is not None
