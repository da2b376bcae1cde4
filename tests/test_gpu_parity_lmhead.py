"""GPU parity of the LM-head path (MFMA GEMM with reduced epilogue, decisions,
recomputed rows, draws) against the CPU oracle, which forms the head's logits
in float64.  Bars as in tests/parity.py, with bf16 inputs (probabilities within
2e-3 relative)."""

import numpy as np
import pytest
import torch

import workloads
from tests import parity as P

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
KEYS = ("accept_len", "out_tokens", "num_emitted", "num_drop")


@pytest.fixture(scope="module")
def sv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lossless_token_verification_amd as m
    m.library()
    return m


def _run(sv, w, seed, offset, **kw):
    g = P.to_device(w, DEV)
    return sv.spec_verify_lmhead_single(g["h_draft"], g["h_target"], g["w_vocab"],
                                        g["draft_tokens"], g["temperature"], seed=seed,
                                        offset=offset, diag=True, **kw)


SMALL = [
    # (B, k, d, V, w_std, temps)
    (6, 4, 256, 5003, 0.2, (1.0,)),            # ragged last vocabulary tile
    (4, 3, 128, 1000, 0.3, (0.0, 0.7, 1.0)),  # greedy and sampled rows, V % 4 == 0
    (5, 2, 192, 129, 0.3, (1.0,)),            # one row tile, V just past a tile
    (3, 0, 64, 777, 0.3, (1.0,)),             # k = 0: bonus only
    (2, 63, 64, 300, 0.1, (1.0,)),            # k = 63
    (1, 1, 65536, 300, 0.004, (1.0,)),        # d = SV_MAX_HIDDEN: 1024 K steps
    (9, 5, 512, 20011, 0.05, (1.3,)),         # several M tiles, flat rows
    # 2B = 280 recomputed rows: a second, partial recompute tile; 420 GEMM rows
    (140, 1, 128, 3000, 0.2, (1.0, 0.0)),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"B{c[0]}k{c[1]}d{c[2]}V{c[3]}")
def test_lmhead_small_parity(sv, case):
    B, k, d, V, w_std, temps = case
    report = {}
    for trial in range(2):
        w = workloads.make_lmhead(B, k, V, d, w_std=w_std, temps=temps,
                                  seed=(71, B, k, d, V, trial))
        out = _run(sv, w, seed=trial + 1, offset=trial * 5)
        torch.cuda.synchronize()
        ref = P.oracle_lmhead(w, trial + 1, trial * 5)
        P.compare(out, ref, KEYS, range(B), True, report, alt=P.alt_lmhead(w, trial + 1, trial * 5))
    print(f"lmhead {case}: {report}")
    P.check_floor(report, 0.75)


def test_lmhead_identical_exits_accept_all(sv):
    """Draft and final hidden states equal: both logit rows come out of the same
    GEMM bit for bit, every draft is accepted, and the bonus is drawn."""
    B, k, d, V = 16, 5, 256, 9000
    w = workloads.make_lmhead(B, k, V, d, w_std=0.2, seed=(72, 0))
    w["h_draft"] = w["h_target"][:, :k].contiguous()
    out = _run(sv, w, 4, 1)
    ref = P.oracle_lmhead(w, 4, 1)
    assert (out["accept_len"].cpu() == k).all()
    P.compare(out, ref, KEYS, range(B), True)


def test_lmhead_greedy_is_exact(sv):
    w = workloads.make_lmhead(24, 4, 6000, 256, w_std=0.2, temps=(0.0,), seed=(73, 0))
    out = _run(sv, w, 0, 0)
    ref = P.oracle_lmhead(w, 0, 0)
    for key in KEYS:
        assert np.array_equal(out[key].cpu().numpy(), ref[key])


def test_lmhead_padded_head_stride_and_packed(sv):
    B, k, d, V = 5, 3, 128, 3001
    w = workloads.make_lmhead(B, k, V, d, w_std=0.2, seed=(74, 0))
    a = _run(sv, w, 2, 2, packed=True)
    wide = torch.zeros((V, d + 64), dtype=torch.bfloat16)
    wide[:, :d] = w["w_vocab"]
    g = P.to_device(w, DEV)
    b = sv.spec_verify_lmhead_single(g["h_draft"], g["h_target"], wide.to(DEV)[:, :d],
                                     g["draft_tokens"], g["temperature"], seed=2, offset=2)
    torch.cuda.synchronize()
    for key in KEYS:
        assert torch.equal(a[key], b[key])
    ne = a["num_emitted"].cpu().tolist()
    cu = a["cu_offsets"].cpu().tolist()
    assert cu == [0] + list(np.cumsum(ne))
    packed = a["packed_tokens"].cpu().tolist()
    toks = a["out_tokens"].cpu().tolist()
    for i in range(B):
        assert packed[cu[i]:cu[i + 1]] == toks[i][:ne[i]]


def test_lmhead_host_validation(sv):
    w = workloads.make_lmhead(2, 2, 500, 96 + 32, seed=(75, 0))     # d = 128 is fine
    g = P.to_device(w, DEV)
    with pytest.raises(sv.SpecVerifyError):
        sv.spec_verify_lmhead_single(g["h_draft"][:, :, :96].contiguous(),
                                     g["h_target"][:, :, :96].contiguous(),
                                     g["w_vocab"][:, :96].contiguous(), g["draft_tokens"],
                                     g["temperature"])
    empty = workloads.make_lmhead(1, 2, 500, 64, seed=(75, 1))
    e = P.to_device(empty, DEV)
    out = sv.spec_verify_lmhead_single(e["h_draft"][:0], e["h_target"][:0], e["w_vocab"],
                                       e["draft_tokens"][:0], e["temperature"][:0])
    assert out["accept_len"].numel() == 0


@pytest.mark.parametrize("trial,seed,offset", [(0, 0, 0), (1, 99, 12345)])
def test_full_size_lmhead(sv, trial, seed, offset):
    """B=128, k=4, d=4096, V=128256 (the fused LM-head workload), in the
    benchmark's launch configuration: every sequence's outputs are
    well-formed and every sequence is compared with the oracle."""
    w = workloads.make("lmhead", trial, device=DEV)
    out = _run(sv, w, seed, offset)
    torch.cuda.synchronize()
    B, k, V = w["B"], w["k"], w["V"]
    a = out["accept_len"].cpu().numpy()
    ne = out["num_emitted"].cpu().numpy()
    toks = out["out_tokens"].cpu().numpy()
    assert ((a >= 0) & (a <= k)).all() and (ne == a + 1).all()
    assert ((toks >= 0) | (np.arange(k + 1)[None] >= ne[:, None])).all() and toks.max() < V
    wc = P._host(w)
    ref = P.oracle_lmhead(wc, seed, offset)
    report = {}
    P.compare(out, ref, KEYS, range(B), True, report, alt=P.alt_lmhead(wc, seed, offset))
    print(f"lmhead full size, trial {trial}:", report)
    P.check_floor(report, 0.75)
