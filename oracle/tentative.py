"""Cross-call tentative buffering: the dynamic verification policy of the
hierarchy, spread over calls.

Test infrastructure only (see ``oracle/__init__``).

HiSpec accumulates a window of tentatively accepted tokens (default N_i = 4)
before it runs the expensive full-model verification, so that the final exit
is called less often while chains of unverified tokens stay short (HiSpec
summary, section 2, bullet "Dynamische Verifizierungsrichtlinie"); entries of
discarded tokens are removed before the next phase (bullet "Wiederverwendung
von KV-Cache ...").  Reading taken here (the pages give no procedure):

* state per sequence: the pending tentative tokens t_0..t_{c-1} and, for each,
  the L_i row it was accepted or drawn under (stage 1's q for stage 2);
* a round (one intermediate verification): stage 1 -- the standard rule with
  q = L_d rows 0..k-1, p = L_i rows 0..k, Philox stage 0 -- gives a1 accepted
  drafts and the L_i correction or bonus y; (x_0..x_{a1-1}, y) and the L_i
  rows 0..a1 are appended to the pending state; the drafts after a1 are
  discarded (k - a1 of them);
* a flush (the full verification, for a sequence with at least N_i pending
  tokens, or forced): stage 2 -- the standard rule with q = the pending L_i
  rows, p = the final exit's rows at the pending positions, Philox stage 1 --
  over t_0..t_{c-1}: a2 = first rejection, else c; on a rejection the L_f
  correction z is drawn from norm(max(0, p - q)) at a2 and t_0..t_{a2-1}, z
  are emitted, otherwise all c pending tokens; no L_f bonus (as in the
  one-call hierarchy); the pending state empties; c - a2 pending tokens are
  discarded on a rejection, none otherwise.

A round followed by a flush with the same Philox offset is exactly the
one-call hierarchical verification (``verify.hier_chain``).
"""

import numpy as np

from . import numerics, philox, rule


def round_chain(Pd, Pi, tokens, u, v):
    """Stage 1 on distributions (float64 or Fraction rows): returns
    (a1, appended tokens, appended L_i rows, info)."""
    k = len(tokens)
    a1, t, info = rule.verify_chain(Pd, Pi[:k], list(tokens), u, v, bonus_row=Pi[k])
    return a1, t, [Pi[j] for j in range(a1 + 1)], info


def flush_chain(pend_tokens, pend_rows, Pf, u, v):
    """Stage 2 over the pending tokens: q = their L_i rows, p = Pf rows (at
    least len(pend_tokens) of them).  Returns (a2, emitted, info)."""
    c = len(pend_tokens)
    return rule.verify_chain(list(pend_rows), list(Pf[:c]), list(pend_tokens), u, v,
                             bonus_row=None)


class TentativeState:
    """Pending tokens and the raw L_i logit rows they were tested under, per
    sequence (raw rows keep the oracle's float64 decode exact)."""

    def __init__(self, batch):
        self.tokens = [[] for _ in range(batch)]
        self.rows = [[] for _ in range(batch)]

    def count(self):
        return np.array([len(t) for t in self.tokens], dtype=np.int32)


def tentative_round(state, ld_logits, li_logits, draft_tokens, temperature, seed, offset,
                    active=None):
    """One round for every active sequence.  ld [B, k, V], li [B, k+1, V] raw
    logits.  Returns a1 [B] (-1 for inactive sequences) and the per-sequence
    infos; appends to ``state``."""
    B, k = np.asarray(ld_logits).shape[:2]
    temps = np.ones(B) if temperature is None else np.asarray(temperature, dtype=np.float64)
    a1s = np.full(B, -1, dtype=np.int32)
    infos = {}
    for b in range(B):
        if active is not None and not active[b]:
            continue
        tau = temps[b]
        Pd = [numerics.row_distribution(numerics.decode(r), tau) for r in ld_logits[b]]
        Pi = [numerics.row_distribution(numerics.decode(r), tau) for r in li_logits[b]]
        u, v = philox.uniforms(np.arange(k + 1, dtype=np.uint64), b, philox.STAGE_SINGLE,
                               offset, seed)
        a1, t, _, info = round_chain(Pd, Pi, draft_tokens[b], u, v)
        a1s[b] = a1
        state.tokens[b].extend(int(x) for x in t)
        state.rows[b].extend(np.array(li_logits[b][j]) for j in range(a1 + 1))
        infos[b] = info
    return a1s, infos


def tentative_flush(state, lf_logits, temperature, seed, offset, min_pending):
    """Flush every sequence with at least ``min_pending`` pending tokens (and at
    least one).  lf [B, cap+1, V] raw: row j is the final exit's row at pending
    position j.  Returns a dict: accept_len (a2, -1 when not flushed),
    num_emitted (0 when not flushed), out_tokens [B, cap+1] (-1 padded),
    num_drop (pending tokens discarded), flushed [B] bool, infos."""
    lf = np.asarray(lf_logits)
    B, width = lf.shape[:2]
    temps = np.ones(B) if temperature is None else np.asarray(temperature, dtype=np.float64)
    a2s = np.full(B, -1, dtype=np.int32)
    n_emit = np.zeros(B, dtype=np.int32)
    out = np.full((B, width), -1, dtype=np.int32)
    drop = np.zeros(B, dtype=np.int32)
    flushed = np.zeros(B, dtype=bool)
    infos = {}
    for b in range(B):
        c = len(state.tokens[b])
        if c == 0 or c < min_pending:
            continue
        tau = temps[b]
        Pi = [numerics.row_distribution(numerics.decode(r), tau) for r in state.rows[b]]
        Pf = [numerics.row_distribution(numerics.decode(lf[b, j]), tau) for j in range(c)]
        u, v = philox.uniforms(np.arange(c, dtype=np.uint64), b, philox.STAGE_FINAL, offset, seed)
        a2, emitted, info = flush_chain(state.tokens[b], Pi, Pf, u, v)
        a2s[b] = a2
        n_emit[b] = len(emitted)
        out[b, :len(emitted)] = emitted
        drop[b] = c - a2
        flushed[b] = True
        infos[b] = info
        state.tokens[b] = []
        state.rows[b] = []
    return dict(accept_len=a2s, num_emitted=n_emit, out_tokens=out, num_drop=drop,
                flushed=flushed, infos=infos)
