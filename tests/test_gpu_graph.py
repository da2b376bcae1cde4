"""The verification call under HIP graph capture: it enqueues kernels only (no
memset, no allocation, no synchronisation), so a captured step replays with the
eager result.  Several replays, with eager work and synchronisations between
them, each checked against the eager call."""

import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def sv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lossless_token_verification_amd as m
    m.library()
    return m


def test_captured_step_replays_the_eager_result(sv):
    w = workloads.make_hier(64, 8, 32000, dtype="bf16", temps=(1.0, 0.0), window=4,
                            seed=(81,), ctx=(64, 512), device=DEV)
    B, k, V = w["B"], w["k"], w["V"]
    ws = sv.alloc_workspace(sv.workspace_bytes(B, k, V, torch.bfloat16, 3), DEV)
    t0, l0 = w["block_table"].clone(), w["seq_lens"].clone()
    table, lens = t0.clone(), l0.clone()
    kw = dict(block_size=w["block_size"], max_freed=1, window=4, seed=3, offset=11, workspace=ws)
    args = (w["ld_logits"], w["li_logits"], w["lf_logits"], w["draft_tokens"], w["temperature"])
    out = sv.spec_verify_hier_rollback(*args, table, lens, **kw)
    torch.cuda.synchronize()
    ref = {n: v.clone() for n, v in out.items() if n != "workspace"}
    ref_t, ref_l = table.clone(), lens.clone()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            sv.spec_verify_hier_rollback(*args, table, lens, out=out, **kw)
    torch.cuda.synchronize()
    for rep in range(4):
        # eager work in between: another call with another offset on the same buffers
        table.copy_(t0)
        lens.copy_(l0)
        sv.spec_verify_hier_rollback(*args, table, lens, out=out,
                                     **{**kw, "offset": 100 + rep})
        torch.cuda.synchronize()
        table.copy_(t0)
        lens.copy_(l0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n, v in ref.items():
            assert torch.equal(out[n], v), (rep, n)
        assert torch.equal(table, ref_t) and torch.equal(lens, ref_l), rep
