"""GPU parity of the cross-call tentative buffering (intermediate rounds append
to a pending state, a flush verifies it against the final exit), through the
C ABI, against the oracle (``oracle.tentative``).

Bars: pending counts, tokens and rows, a1, a2, emitted tokens and discard
counts bit for bit, except for sequences the oracle marks as a near tie (the
verification's exemption rule, tests/parity.py); such a sequence is dropped
from the comparison from that call on, since its state may then differ.
"""

import numpy as np
import pytest
import torch

import workloads
from oracle import tentative as ot
from oracle import verify as ov
from tests import parity as P

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def sv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lossless_token_verification_amd as m
    m.library()
    return m


def _near(info):
    return ov.near_tie(info, P.RATIO_EPS, P.CDF_DELTA)


def _pad_rows(x, width):
    """[B, n, V] -> [B, width, V] with zero rows appended."""
    B, n, V = x.shape
    out = torch.zeros((B, width, V), dtype=x.dtype, device=x.device)
    out[:, :n] = x
    return out


def _compare_state(sv_state, st, live):
    count = sv_state["count"].cpu().numpy()
    toks = sv_state["tokens"].cpu().numpy()
    rows = P.raw(sv_state["rows"].cpu())
    for b in live:
        c = len(st.tokens[b])
        assert count[b] == c, (b, count[b], c)
        assert toks[b, :c].tolist() == st.tokens[b], b
        for j in range(c):
            assert np.array_equal(rows[b, j], st.rows[b][j]), (b, j)


@pytest.mark.parametrize("dt,temps", [("bf16", (1.0,)), ("f32", (0.0, 0.7, 1.0))])
def test_round_then_flush_is_the_one_call_hierarchy(sv, dt, temps):
    B, k, V = 12, 6, 30011
    w = workloads.make_hier(B, k, V, dtype=dt, temps=temps, window=4, seed=(71, B, k, V),
                            ctx=(16, 64))
    g = P.to_device(w, DEV)
    cap = k + 1
    pend = sv.make_pending(B, cap, V, g["ld_logits"].dtype, DEV)
    r = sv.spec_verify_tentative_round(g["ld_logits"], g["li_logits"], g["draft_tokens"],
                                       g["temperature"], pend, seed=5, offset=7)
    f = sv.spec_verify_tentative_flush(_pad_rows(g["lf_logits"], cap + 1), g["temperature"],
                                       pend, min_pending=1, seed=5, offset=7)
    torch.cuda.synchronize()
    ref = P.oracle_hier(w, 5, 7, 4)
    live = [b for b in range(B) if not _near(ref["infos"][b])]
    assert len(live) >= B - 2
    a1 = r["accept_len"].cpu().numpy()
    a2 = f["accept_len"].cpu().numpy()
    n = f["num_emitted"].cpu().numpy()
    toks = f["out_tokens"].cpu().numpy()
    for b in live:
        assert a1[b] == ref["accept_len_inter"][b], b
        assert a2[b] == ref["accept_len_final"][b], b
        assert n[b] == ref["num_emitted"][b], b
        assert toks[b, :n[b]].tolist() == ref["out_tokens"][b, :n[b]].tolist(), b
        assert r["num_drop"][b].item() == k - a1[b]
    assert (pend["count"].cpu().numpy() == 0).all()


CASES = [
    # (B, k, V, dtype, temps, cap, N_i)
    (8, 4, 20011, "bf16", (1.0,), 12, 4),
    (6, 3, 9001, "f32", (0.0, 0.7, 1.0), 8, 4),
    (5, 5, 3001, "bf16", (1.0, 0.5), 10, 3),      # misaligned rows
    (4, 2, 70001, "f32", (1.0,), 6, 4),           # several 64 KiB chunks per row
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}k{c[1]}V{c[2]}{c[3]}cap{c[5]}")
def test_buffered_rounds_and_flushes(sv, case):
    """Rounds for the sequences below N_i pending tokens, then a flush of those
    at or above it, repeated; state and outputs against the oracle after every
    call."""
    B, k, V, dt, temps, cap, N_i = case
    st = ot.TentativeState(B)
    pend = None
    live = set(range(B))
    flushed_total = 0
    offset = 0
    for it in range(5):
        w = workloads.make_hier(B, k, V, dtype=dt, temps=temps, window=4,
                                seed=(72, B, k, V, it), ctx=(16, 64))
        g = P.to_device(w, DEV)
        if pend is None:
            pend = sv.make_pending(B, cap, V, g["ld_logits"].dtype, DEV)
        active_np = (st.count() < N_i) & (st.count() + k + 1 <= cap)
        active = torch.from_numpy(active_np.astype(np.int32)).to(DEV)
        r = sv.spec_verify_tentative_round(g["ld_logits"], g["li_logits"], g["draft_tokens"],
                                           g["temperature"], pend, active=active, seed=3,
                                           offset=offset)
        torch.cuda.synchronize()
        a1_ref, infos = ot.tentative_round(st, P.raw(w["ld_logits"]), P.raw(w["li_logits"]),
                                           w["draft_tokens"].numpy(), P.raw(w["temperature"])
                                           if w["temperature"] is not None else None,
                                           seed=3, offset=offset, active=active_np)
        offset += 1
        live -= {b for b, info in infos.items() if _near(info)}
        a1 = r["accept_len"].cpu().numpy()
        for b in live:
            if active_np[b]:
                assert a1[b] == a1_ref[b], (it, b)
        _compare_state(pend, st, live)
        # the final exit's rows at the pending positions (fresh random rows)
        lf = workloads.make_hier(B, cap, V, dtype=dt, temps=temps, window=4,
                                 seed=(73, B, k, V, it), ctx=(16, 64))["lf_logits"]
        f = sv.spec_verify_tentative_flush(lf.to(DEV), g["temperature"], pend, min_pending=N_i,
                                           seed=3, offset=offset)
        torch.cuda.synchronize()
        fr = ot.tentative_flush(st, P.raw(lf), P.raw(w["temperature"])
                                if w["temperature"] is not None else None,
                                seed=3, offset=offset, min_pending=N_i)
        offset += 1
        live -= {b for b, info in fr["infos"].items() if _near(info)}
        got = {kk: f[kk].cpu().numpy() for kk in ("accept_len", "num_emitted", "num_drop",
                                                  "out_tokens")}
        for b in live:
            assert got["accept_len"][b] == fr["accept_len"][b], (it, b)
            assert got["num_emitted"][b] == fr["num_emitted"][b], (it, b)
            assert got["num_drop"][b] == fr["num_drop"][b], (it, b)
            assert np.array_equal(got["out_tokens"][b], fr["out_tokens"][b]), (it, b)
        flushed_total += int(fr["flushed"].sum())
        _compare_state(pend, st, live)
    assert flushed_total >= B and len(live) >= B - 2, (flushed_total, len(live))
    assert sv.device_status(r["workspace"]) & sv.SV_FLAG_PENDING_FULL == 0


def test_overflow_is_flagged_and_truncated(sv):
    B, k, V, cap = 4, 6, 5000, 4
    w = workloads.make_hier(B, k, V, dtype="f32", temps=(1.0,), window=4, seed=(74,),
                            ctx=(16, 64))
    g = P.to_device(w, DEV)
    # L_i == L_d: every draft is accepted, k + 1 = 7 tokens do not fit 4
    pend = sv.make_pending(B, cap, V, torch.float32, DEV)
    li = g["li_logits"].clone()
    li[:, :k] = g["ld_logits"]
    r = sv.spec_verify_tentative_round(g["ld_logits"], li, g["draft_tokens"], None, pend)
    torch.cuda.synchronize()
    assert (r["accept_len"].cpu() == k).all()
    assert (pend["count"].cpu() == cap).all()
    assert sv.device_status(r["workspace"]) & sv.SV_FLAG_PENDING_FULL
    assert torch.equal(pend["tokens"].cpu(), w["draft_tokens"][:, :cap])
    assert torch.equal(pend["rows"].cpu(), w["ld_logits"][:, :cap])


@pytest.mark.parametrize("trial,seed,offset", [(0, 0, 0), (1, 5, 4242)])
def test_full_size_round_and_flush(sv, trial, seed, offset):
    """B=256 k=8 V=128256 bf16: a round and a flush (min_pending 1) agree with
    the one-call hierarchy's oracle on every sequence (near ties: the oracle's
    outcome or the one with that decision flipped)."""
    w = workloads.make("hier", trial, device=DEV)
    B, k, V = w["B"], w["k"], w["V"]
    cap = k + 1
    pend = sv.make_pending(B, cap, V, torch.bfloat16, DEV)
    r = sv.spec_verify_tentative_round(w["ld_logits"], w["li_logits"], w["draft_tokens"],
                                       w["temperature"], pend, seed=seed, offset=offset)
    f = sv.spec_verify_tentative_flush(_pad_rows(w["lf_logits"], cap + 1), w["temperature"],
                                       pend, min_pending=1, seed=seed, offset=offset)
    torch.cuda.synchronize()
    wc = P._host(w)
    ref = P.oracle_hier(wc, seed, offset, w["window"])
    got = dict(accept_len_inter=r["accept_len"], accept_len_final=f["accept_len"],
               out_tokens=f["out_tokens"][:, :k + 1], num_emitted=f["num_emitted"])
    report = {}
    P.compare(got, ref, ("accept_len_inter", "accept_len_final", "out_tokens", "num_emitted"),
              range(B), True, report, alt=P.alt_hier(wc, seed, offset, w["window"]))
    print(f"full size round + flush, trial {trial}:", report)
    P.check_floor(report, 0.9)
    assert (pend["count"].cpu() == 0).all()
