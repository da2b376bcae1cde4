"""Verification of drafts whose logits come from a linear LM head.

Test infrastructure only (see ``oracle/__init__``).

In an early-exit model every exit turns its hidden state into a token
distribution (HiSpec summary, section 2 "Kernmechanismus": the draft exit L_d
and the final exit L_f each yield distributions at the drafted positions).
With a shared linear LM head W (one d-vector per vocabulary entry, stored
[V, d]) the logits of a hidden state h are l[v] = sum_i h[i] * W[v, i].  Here
they are formed in float64 from the bf16 inputs (every product of two bf16
values is exact in float64) and then go through the single-stage rule of
``verify.spec_verify_single`` unchanged: q from the draft exit at the k
drafted positions, p from the final exit at k + 1 positions.
"""

import numpy as np

from . import numerics, verify


def lmhead_logits(h_raw, w_raw, chunk=4096):
    """Logits [R, V] (float64) of hidden states h_raw [R, d] under the head
    w_raw [V, d] (both uint16 bf16 bits), vocabulary chunk by chunk."""
    H = numerics.decode_bf16(np.asarray(h_raw).reshape(-1, np.asarray(h_raw).shape[-1]))
    V, d = w_raw.shape
    if H.shape[1] != d:
        raise ValueError("hidden size of h and W differ")
    out = np.empty((H.shape[0], V), dtype=np.float64)
    for v0 in range(0, V, chunk):
        Wc = numerics.decode_bf16(w_raw[v0:v0 + chunk])
        out[:, v0:v0 + chunk] = H @ Wc.T
    return out


def spec_verify_lmhead_single(h_draft, h_target, w, draft_tokens, temperature, seed, offset,
                              sequences=None, flips=None):
    """Batched single-stage verify through an LM head.

    h_draft [B, k, d] and h_target [B, k+1, d] hidden states, w [V, d] head,
    all uint16 bf16 bits; draft_tokens [B, k]; temperature [B] or None.
    Returns what ``verify.spec_verify_single`` returns on the head's logits
    (sequences outside ``sequences`` are left at -1; ``flips`` as there).
    """
    B, k, d = h_draft.shape
    if h_target.shape != (B, k + 1, d):
        raise ValueError("h_target must be [B, k+1, d]")
    V = w.shape[0]
    seqs = list(range(B)) if sequences is None else list(sequences)
    ld = np.zeros((B, k, V), dtype=np.float64)
    lt = np.zeros((B, k + 1, V), dtype=np.float64)
    if seqs:
        rows = np.concatenate([h_draft[seqs].reshape(-1, d), h_target[seqs].reshape(-1, d)])
        L = lmhead_logits(rows, w)
        nd = len(seqs) * k
        ld[seqs] = L[:nd].reshape(len(seqs), k, V)
        lt[seqs] = L[nd:].reshape(len(seqs), k + 1, V)
    return verify.spec_verify_single(ld, lt, draft_tokens, temperature, seed, offset,
                                     sequences=seqs, flips=flips)
