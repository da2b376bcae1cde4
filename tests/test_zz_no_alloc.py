"""spec_verify_hier_rollback_noalloc (the entry point that allocates nothing;
its workspace is the library's static per-GPU scratch) against
spec_verify_hier_rollback with a caller workspace, through the C ABI: two calls
in a row on one GPU, the second with a smaller input, bit for bit on every
output and on the rolled-back KV state."""

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


def _pair(sv, w, seed, offset):
    g = P.to_device(w, DEV)
    kw = dict(block_size=w["block_size"], max_freed=2, window=w["window"], seed=seed,
              offset=offset)
    t1, l1 = g["block_table"].clone(), g["seq_lens"].clone()
    ref = sv.spec_verify_hier_rollback(g["ld_logits"], g["li_logits"], g["lf_logits"],
                                       g["draft_tokens"], g["temperature"], t1, l1, **kw)
    t2, l2 = g["block_table"].clone(), g["seq_lens"].clone()
    got = sv.spec_verify_hier_rollback_noalloc(g["ld_logits"], g["li_logits"], g["lf_logits"],
                                               g["draft_tokens"], g["temperature"], t2, l2, **kw)
    torch.cuda.synchronize()
    assert got["workspace"] is None
    for key in KEYS:
        assert torch.equal(ref[key], got[key]), key
    assert torch.equal(t1, t2) and torch.equal(l1, l2)
    return got


def test_noalloc_equals_workspace_call_twice_second_smaller(sv):
    big = workloads.make_hier(96, 8, 70001, dtype="bf16", temps=(1.0, 0.0, 0.7), window=4,
                              seed=(131, 0), ctx=(20, 200))
    small = workloads.make_hier(7, 3, 20011, dtype="f32", temps=(1.0,), window=2,
                                seed=(131, 1), ctx=(20, 200))
    a = _pair(sv, big, 3, 5)
    b = _pair(sv, small, 4, 6)
    # the second call's outputs are its own (nothing of the first call's left)
    assert a["out_tokens"].shape[0] == 96 and b["out_tokens"].shape[0] == 7


def test_noalloc_oversized_call_is_refused(sv):
    B, k, V = 256, 63, 1 << 20
    assert sv.workspace_bytes(B, k, V, torch.bfloat16, 3) > sv.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((1, 1, 8), dtype=torch.bfloat16, device=DEV)
    d = sv.make_desc(B, k, V, sv.SV_DTYPE_BF16)
    lib = sv.library()
    st = lib.spec_verify_hier_rollback_noalloc(
        __import__('ctypes').byref(d), 4, x.data_ptr(), x.data_ptr(), x.data_ptr(), x.data_ptr(), None, x.data_ptr(),
        x.data_ptr(), x.data_ptr(), x.data_ptr(), None, 8, 16, x.data_ptr(), x.data_ptr(),
        x.data_ptr(), 1, x.data_ptr(), None, None)
    assert st == sv.SV_ERR_WORKSPACE
