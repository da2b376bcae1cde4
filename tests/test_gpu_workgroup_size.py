"""The kernels at another workgroup size: libspecverify_t128.so is the same
sources built with 128-thread workgroups (32 KiB stream chunks, two wavefronts
per verification workgroup, twice the chunk partials to merge).  A race on
LDS or between wavefronts that the 256-thread layout happens to hide would show
as a difference here.  Both builds, through the C ABI on the same inputs, must
agree with the oracle (the parity bars of tests/parity.py) and with each other
on every sequence that is not a near tie."""

import os

import numpy as np
import pytest
import torch

import workloads
from tests import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
HIER_KEYS = ("accept_len_inter", "accept_len_final", "out_tokens", "num_emitted", "num_drop")
SINGLE_KEYS = ("accept_len", "out_tokens", "num_emitted", "num_drop")


@pytest.fixture(scope="module")
def both():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lossless_token_verification_amd as sv
    lib256 = sv.library()
    path = os.path.join(os.path.dirname(sv.LIB_PATH), "libspecverify_t128.so")
    assert os.path.exists(path), "the 128-thread build is missing: run build()"
    return sv, lib256, sv.load_library(path)


def _on(sv, lib, fn):
    keep = sv._lib
    sv._lib = lib
    try:
        out = fn()
        torch.cuda.synchronize()
        return out
    finally:
        sv._lib = keep


HIER = [(12, 8, 50021, "bf16", (1.0,), 4), (8, 6, 20011, "f32", (0.0, 0.7, 1.0), 4),
        (6, 5, 3001, "bf16", (1.0,), 1), (3, 63, 70001, "bf16", (1.0,), 4)]
SINGLE = [(16, 4, 70001, "bf16", (1.0,)), (10, 3, 1001, "bf16", (1.0, 0.5)),
          (12, 5, 40003, "f32", (0.0, 0.7, 1.0)), (5, 0, 4096, "f32", (1.0,))]


@pytest.mark.parametrize("case", HIER, ids=lambda c: f"B{c[0]}k{c[1]}V{c[2]}{c[3]}w{c[5]}")
def test_hier_at_128_threads(both, case):
    sv, lib256, lib128 = both
    B, k, V, dt, temps, window = case
    w = workloads.make_hier(B, k, V, dtype=dt, temps=temps, window=window,
                            seed=(141, B, k, V), ctx=(16, 64))
    g = P.to_device(w, DEV)

    def run():
        return sv.spec_verify_hier(g["ld_logits"], g["li_logits"], g["lf_logits"],
                                   g["draft_tokens"], g["temperature"], window=window, seed=2,
                                   offset=3, diag=True)
    a, b = _on(sv, lib256, run), _on(sv, lib128, run)
    ref = P.oracle_hier(w, 2, 3, window)
    for out in (a, b):
        report = {}
        P.compare(out, ref, HIER_KEYS, range(B), dt == "bf16", report,
                  alt=P.alt_hier(w, 2, 3, window))
        P.check_floor(report, 0.9)
    _agree(a, b, ref, HIER_KEYS, B)


@pytest.mark.parametrize("case", SINGLE, ids=lambda c: f"B{c[0]}k{c[1]}V{c[2]}{c[3]}")
def test_single_at_128_threads(both, case):
    sv, lib256, lib128 = both
    B, k, V, dt, temps = case
    w = workloads.make_single(B, k, V, dtype=dt, temps=temps, seed=(142, B, k, V))
    g = P.to_device(w, DEV)

    def run():
        return sv.spec_verify_single(g["draft_logits"], g["target_logits"], g["draft_tokens"],
                                     g["temperature"], seed=4, offset=5, diag=True)
    a, b = _on(sv, lib256, run), _on(sv, lib128, run)
    ref = P.oracle_single(w, 4, 5)
    for out in (a, b):
        report = {}
        P.compare(out, ref, SINGLE_KEYS, range(B), dt == "bf16", report,
                  alt=P.alt_single(w, 4, 5))
        P.check_floor(report, 0.9)
    _agree(a, b, ref, SINGLE_KEYS, B)


def test_rollback_call_at_128_threads(both):
    """The benchmarked call (verification + KV rollback) on a batch of 64."""
    sv, lib256, lib128 = both
    w = workloads.make_hier(64, 8, 30011, dtype="bf16", temps=(1.0, 0.0), seed=(143, 0),
                            ctx=(20, 200))
    g = P.to_device(w, DEV)
    outs = []
    for lib in (lib256, lib128):
        t, l = g["block_table"].clone(), g["seq_lens"].clone()

        def run():
            return sv.spec_verify_hier_rollback(g["ld_logits"], g["li_logits"], g["lf_logits"],
                                                g["draft_tokens"], g["temperature"], t, l,
                                                block_size=16, max_freed=1, window=4, seed=6,
                                                offset=7)
        outs.append((_on(sv, lib, run), t.cpu(), l.cpu()))
    ref = P.oracle_hier(w, 6, 7, 4)
    (a, ta, la), (b, tb, lb) = outs
    _agree(a, b, ref, HIER_KEYS + ("freed_blocks", "num_freed"), 64)
    same = [bb for bb in range(64) if torch.equal(a["num_drop"][bb].cpu(), b["num_drop"][bb].cpu())]
    assert torch.equal(ta[same], tb[same]) and torch.equal(la[same], lb[same])


BYP = [("hier", 6, 8, 70001, "bf16", (1.0,), 8), ("hier", 5, 4, 20011, "f32", (0.0, 0.7, 1.0), 3),
       ("single", 6, 4, 3001, "bf16", (1.0, 0.5), 8)]


@pytest.mark.parametrize("case", BYP, ids=lambda c: f"{c[0]}B{c[1]}k{c[2]}V{c[3]}{c[4]}m{c[6]}")
def test_byproducts_at_128_threads(both, case):
    """Row entropies and the outcome export (the lane sets, candidate buffers
    and per-stage thread halves of the outcome pass scale with the workgroup)
    on both builds, each against the oracle."""
    from tests import test_gpu_parity_byproducts as tb
    sv, lib256, lib128 = both
    kind, B, k, V, dt, temps, top_m = case
    if kind == "hier":
        w = workloads.make_hier(B, k, V, dtype=dt, temps=temps, window=4, seed=(144, B, V),
                                ctx=(16, 64))
    else:
        w = workloads.make_single(B, k, V, dtype=dt, temps=temps, seed=(145, B, V))
    outs = [_on(sv, lib, lambda: tb._run(sv, w, 3, 4, entropy=True, outcome=True, top_m=top_m))
            for lib in (lib256, lib128)]
    for out in outs:
        tb.check_entropy(out["entropy"].cpu().numpy(), w)
        assert tb.check_outcome(out, w, top_m) > 0
    a, b = (o["accept_mass"].cpu().numpy() for o in outs)
    assert np.array_equal(np.isnan(a), np.isnan(b))
    assert np.nanmax(np.abs(a - b)) <= 1e-6


def _agree(a, b, ref, keys, B):
    """The two builds give the same outputs on every sequence without a near
    tie (at a near tie either may take the other outcome)."""
    from oracle import verify as ov
    for bb in range(B):
        if ov.near_tie(ref["infos"][bb], P.RATIO_EPS, P.CDF_DELTA):
            continue
        for key in keys:
            assert np.array_equal(a[key][bb].cpu().numpy(), b[key][bb].cpu().numpy()), (key, bb)
