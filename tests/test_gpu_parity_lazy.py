"""GPU parity of the lazy final exit: spec_verify_hier_rollback_lazy reads only
the L_f rows stage 2 can reach and must give bit-identical results to the
dense call (and match the oracle, whose hierarchy never looks at L_f past a1)."""

import numpy as np
import pytest
import torch

import workloads
from tests import parity as P

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
KEYS = ("accept_len_inter", "accept_len_final", "out_tokens", "num_emitted", "num_drop",
        "freed_blocks", "num_freed")


@pytest.fixture(scope="module")
def sv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lossless_token_verification_amd as m
    m.library()
    return m


def _both(sv, w, seed, offset, window, ws=None):
    g = P.to_device(w, DEV)
    outs = []
    for fn in (sv.spec_verify_hier_rollback, sv.spec_verify_hier_rollback_lazy):
        table, lens = g["block_table"].clone(), g["seq_lens"].clone()
        o = fn(g["ld_logits"], g["li_logits"], g["lf_logits"], g["draft_tokens"],
               g["temperature"], table, lens, block_size=w["block_size"], max_freed=2,
               window=window, seed=seed, offset=offset, diag=True, workspace=ws)
        o["table"], o["lens"] = table, lens
        outs.append(o)
    torch.cuda.synchronize()
    return outs


CASES = [
    # (B, k, V, dtype, temps, window)
    (12, 8, 50021, "bf16", (1.0,), 4),
    (8, 6, 20011, "f32", (0.0, 0.7, 1.0), 4),
    (6, 5, 3001, "bf16", (1.0,), 1),           # misaligned rows
    (4, 3, 9000, "f32", (0.9,), 2),
    (3, 0, 5000, "bf16", (1.0,), 4),           # k = 0
    (5, 8, 4096, "bf16", (1.0,), 4),
    (6, 4, 7000, "f32", (1.0,), 4),            # window == k: stage 1 decided in one pass
    (5, 2, 6000, "bf16", (1.0, 0.0), 7),       # window > k
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}k{c[1]}V{c[2]}{c[3]}w{c[5]}")
def test_lazy_equals_dense_and_oracle(sv, case):
    B, k, V, dt, temps, window = case
    report = {}
    for trial in range(3):
        w = workloads.make_hier(B, k, V, dtype=dt, temps=temps, window=window,
                                seed=(81, B, k, V, trial), ctx=(16, 64))
        dense, lazy = _both(sv, w, trial + 2, trial, window)
        for key in KEYS + ("table", "lens"):
            assert torch.equal(dense[key], lazy[key]), key
        ref = P.oracle_hier(w, trial + 2, trial, window)
        P.compare(lazy, ref, KEYS[:5], range(B), dt == "bf16", report,
                  alt=P.alt_hier(w, trial + 2, trial, window))
    print(f"lazy {case}: {report}")
    P.check_floor(report, 0.9)


@pytest.mark.parametrize("dt,window", [("bf16", 4), ("f32", 3)])
def test_lazy_open_sequences(sv, dt, window):
    """Sequences that accept every draft of the stage-1 window: L_i rows equal
    to the L_d rows make p / q exactly 1 there.  Half the sequences match over
    the window only (the rest of their L_d / L_i rows and every L_f row are
    listed, then stage 1 continues past the window), a quarter over every
    position (all k drafts accepted, the bonus drawn); the others are left
    random."""
    B, k, V = 8, 8, 20011
    for trial in range(2):
        w = workloads.make_hier(B, k, V, dtype=dt, temps=(1.0,), window=window,
                                seed=(84, trial, window), ctx=(16, 64))
        for b in range(0, B, 2):
            n = k if b % 4 == 0 else window
            w["li_logits"][b, :n] = w["ld_logits"][b, :n]
        dense, lazy = _both(sv, w, 7, trial, window)
        for key in KEYS + ("table", "lens"):
            assert torch.equal(dense[key], lazy[key]), key
        a1 = lazy["accept_len_inter"].cpu().numpy()
        assert (a1[0::4] == k).all() and (a1[2::4] >= window).all(), a1
        ref = P.oracle_hier(w, 7, trial, window)
        P.compare(lazy, ref, KEYS[:5], range(B), dt == "bf16", alt=P.alt_hier(w, 7, trial, window))


def test_lazy_and_dense_alternate_on_one_workspace(sv):
    """Stale statistics of rows the lazy call skips never leak into a result."""
    w1 = workloads.make_hier(16, 8, 30000, dtype="bf16", seed=(82, 0), ctx=(16, 64))
    w2 = workloads.make_hier(16, 8, 30000, dtype="bf16", seed=(82, 1), ctx=(16, 64))
    ws = sv.alloc_workspace(sv.workspace_bytes(16, 8, 30000, torch.bfloat16, 3), DEV)
    for w in (w1, w2, w1):
        dense, lazy = _both(sv, w, 5, 1, 4, ws=ws)
        for key in KEYS + ("table", "lens"):
            assert torch.equal(dense[key], lazy[key]), key


@pytest.mark.parametrize("trial,seed,offset", [(0, 0, 3), (2, 17, 2 ** 20 + 1)])
def test_full_size_lazy_equals_dense(sv, trial, seed, offset):
    """The headline workload through the lazy call: bit-identical to the dense
    call, and every sequence compared with the oracle directly."""
    w = workloads.make("hier", trial, device=DEV)
    dense, lazy = _both(sv, w, seed, offset, w["window"])
    for key in KEYS + ("table", "lens"):
        assert torch.equal(dense[key], lazy[key]), key
    a1 = lazy["accept_len_inter"].cpu().numpy()
    print("full size lazy: mean a1", a1.mean(), "L_f rows read per sequence", (a1 + 1).mean())
    wc = P._host(w)
    ref = P.oracle_hier(wc, seed, offset, w["window"])
    report = {}
    P.compare(lazy, ref, KEYS[:5], range(w["B"]), True, report,
              alt=P.alt_hier(wc, seed, offset, w["window"]))
    print("full size lazy vs oracle:", report)
    P.check_floor(report, 0.9)
