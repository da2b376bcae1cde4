"""The timing events of the diagnostics (stats_begin / stats_end) take the
start and end of the statistics kernels through extended launches: results
with and without them are identical, and the interval they give is positive
and no longer than the whole call."""

import ctypes

import numpy as np
import pytest
import torch

import workloads
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


class _Events:
    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
            self.ev.append(e)

    def record(self, i):
        stream = ctypes.c_void_p(torch.cuda.current_stream(torch.device(DEV)).cuda_stream)
        assert self.hip.hipEventRecord(self.ev[i], stream) == 0

    def ms(self, a, b):
        out = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(out), self.ev[a], self.ev[b]) == 0
        return out.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)


def _same(a, b, keys):
    for key in keys:
        assert torch.equal(a[key].cpu(), b[key].cpu()), key


@pytest.mark.parametrize("lazy", [False, True])
def test_hier_rollback_events(sv, lazy):
    w = workloads.make_hier(24, 6, 40000, dtype="bf16", temps=(1.0, 0.0), window=4,
                            seed=(81, int(lazy)), ctx=(16, 64))
    g = P.to_device(w, DEV)
    fn = sv.spec_verify_hier_rollback_lazy if lazy else sv.spec_verify_hier_rollback
    ev = _Events(4)
    outs = []
    for events in (None, (ev.ev[1].value, ev.ev[2].value)):
        table, lens = g["block_table"].clone(), g["seq_lens"].clone()
        ev.record(0)
        o = fn(g["ld_logits"], g["li_logits"], g["lf_logits"], g["draft_tokens"],
               g["temperature"], table, lens, block_size=w["block_size"], max_freed=2,
               window=4, seed=3, offset=1, events=events)
        ev.record(3)
        torch.cuda.synchronize()
        o["table"], o["lens"] = table, lens
        outs.append(o)
    _same(outs[0], outs[1], ("accept_len_inter", "accept_len_final", "out_tokens",
                             "num_emitted", "num_drop", "freed_blocks", "num_freed", "table",
                             "lens"))
    stats_ms, call_ms = ev.ms(1, 2), ev.ms(0, 3)
    ev.close()
    assert 0.0 < stats_ms <= call_ms, (stats_ms, call_ms)


def test_lmhead_events(sv):
    w = workloads.make_lmhead(6, 3, 5003, 256, w_std=0.2, temps=(1.0,), seed=(82, 0))
    g = P.to_device(w, DEV)
    ev = _Events(4)
    outs = []
    for events in (None, (ev.ev[1].value, ev.ev[2].value)):
        ev.record(0)
        o = sv.spec_verify_lmhead_single(g["h_draft"], g["h_target"], g["w_vocab"],
                                         g["draft_tokens"], g["temperature"], seed=2, offset=0,
                                         events=events)
        ev.record(3)
        torch.cuda.synchronize()
        outs.append({k: (v.clone() if torch.is_tensor(v) else v) for k, v in o.items()})
    _same(outs[0], outs[1], ("accept_len", "out_tokens", "num_emitted", "num_drop"))
    stats_ms, call_ms = ev.ms(1, 2), ev.ms(0, 3)
    ev.close()
    assert 0.0 < stats_ms <= call_ms, (stats_ms, call_ms)
    assert np.isfinite(stats_ms)
