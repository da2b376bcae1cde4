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


def verify_single_sequence(draft_raw, target_raw, tokens, tau, b, seed, offset):
    """One sequence of the single-stage verify.  draft_raw [k, V], target_raw
    [k+1, V] raw logits; returns (a, emitted, info)."""
    k = len(tokens)
    Q = _rows(draft_raw, tau)
    P = _rows(target_raw, tau)
    us, vs = _uniform_vectors(k + 1, b, philox.STAGE_SINGLE, offset, seed)
    return rule.verify_chain(Q, P[:k], list(tokens), us, vs, bonus_row=P[k])


def verify_hier_sequence(ld_raw, li_raw, lf_raw, tokens, tau, b, seed, offset, window):
    """One sequence of the hierarchical verify.  Returns (a1, a2, emitted, info)."""
    k = len(tokens)
    Pd = _rows(ld_raw, tau)
    Pi = _rows(li_raw, tau)
    Pf = _rows(lf_raw, tau)
    u1, v1 = _uniform_vectors(k + 1, b, philox.STAGE_SINGLE, offset, seed)
    u2, v2 = _uniform_vectors(k + 1, b, philox.STAGE_FINAL, offset, seed)
    return hier_chain(Pd, Pi, Pf, tokens, u1, v1, u2, v2, window)


def hier_chain(Pd, Pi, Pf, tokens, u1, v1, u2, v2, window):
    """The two stages on distributions (float64 or Fraction rows) and explicit
    uniforms (u1, v1 for stage 1 and u2, v2 for stage 2, indexed by position).
    Returns (a1, a2, emitted, info)."""
    k = len(tokens)
    a1, t, info1 = rule.verify_chain(Pd, Pi[:k], list(tokens), u1, v1, bonus_row=Pi[k])
    a2, emitted, info2 = rule.verify_chain(Pi[:a1 + 1], Pf[:a1 + 1], t, u2, v2,
                                           bonus_row=None, window=window)
    return a1, a2, emitted, dict(stage1=info1, stage2=info2, tentative=t)


def _pad(emitted, width):
    out = np.full(width, -1, dtype=np.int32)
    out[:len(emitted)] = emitted
    return out


def spec_verify_single(draft_logits, target_logits, draft_tokens, temperature,
                       seed, offset, sequences=None):
    """Batched single-stage verify.

    draft_logits [B, k, V], target_logits [B, k+1, V] raw (uint16 bf16 bits or
    float32); draft_tokens [B, k] int; temperature [B] float or None (all 1).
    ``sequences`` restricts the work to a subset of b (outputs of the others
    are left at -1).  Returns a dict of arrays plus per-sequence infos.
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
                                                  draft_tokens[b], temps[b], b, seed, offset)
        accept_len[b] = a
        num_emitted[b] = len(emitted)
        out_tokens[b] = _pad(emitted, k + 1)
        infos[b] = info
    return dict(accept_len=accept_len, num_emitted=num_emitted, out_tokens=out_tokens,
                num_drop=np.where(num_emitted >= 0, k - (num_emitted - 1), -1).astype(np.int32),
                infos=infos)


def spec_verify_hier(ld_logits, li_logits, lf_logits, draft_tokens, temperature,
                     seed, offset, window=4, sequences=None):
    """Batched hierarchical verify.  ld [B, k, V], li/lf [B, k+1, V]."""
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
                                                     offset, window)
        a1s[b], a2s[b] = a1, a2
        num_emitted[b] = len(emitted)
        out_tokens[b] = _pad(emitted, k + 1)
        infos[b] = info
    return dict(accept_len_inter=a1s, accept_len_final=a2s, num_emitted=num_emitted,
                out_tokens=out_tokens,
                num_drop=np.where(num_emitted >= 0, k - (num_emitted - 1), -1).astype(np.int32),
                infos=infos)


def near_tie(info, ratio_eps=1e-5, cdf_delta=1e-6):
    """True when a sequence's result may legitimately differ between a float32
    implementation and this float64 one: an accept test with |u - p/q| <
    ratio_eps, or a draw whose threshold v*R lies within cdf_delta (probability
    units) of either CDF boundary of the chosen token, or whose residual mass
    is below cdf_delta.  Accepts the info of one chain or of a hierarchy."""
    if "stage1" in info:
        return near_tie(info["stage1"], ratio_eps, cdf_delta) or \
            near_tie(info["stage2"], ratio_eps, cdf_delta)
    for u, p, q in info["tests"]:
        if q > 0:
            rho = p / q
        else:
            rho = np.inf if p > 0 else 0.0
        if abs(u - rho) < ratio_eps:
            return True
    d = info["draw"]
    if d is not None:
        if d.get("fallback"):
            return True
        if d["R"] < cdf_delta:
            return True
        if d["t"] - d["c_lo"] < cdf_delta or d["c_hi"] - d["t"] < cdf_delta:
            return True
    return False
