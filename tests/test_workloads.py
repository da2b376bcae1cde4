"""The seeded input generators: shapes, dtypes, determinism and the laws they
are meant to follow (small sizes on the CPU)."""

import numpy as np
import torch

import workloads


def test_single_shapes_and_determinism():
    a = workloads.make_single(5, 3, 1001, dtype="bf16", seed=(4, 2))
    b = workloads.make_single(5, 3, 1001, dtype="bf16", seed=(4, 2))
    assert a["draft_logits"].shape == (5, 3, 1001) and a["draft_logits"].dtype == torch.bfloat16
    assert a["target_logits"].shape == (5, 4, 1001)
    assert a["draft_tokens"].dtype == torch.int32 and a["draft_tokens"].shape == (5, 3)
    assert torch.equal(a["target_logits"], b["target_logits"])
    assert torch.equal(a["draft_tokens"], b["draft_tokens"])
    assert int(a["draft_tokens"].min()) >= 0 and int(a["draft_tokens"].max()) < 1001


def test_hier_correlations_and_block_tables():
    w = workloads.make_hier(16, 8, 4096, seed=(3, 0))
    d = w["ld_logits"].float()
    i = w["li_logits"].float()[:, :8]
    f = w["lf_logits"].float()
    c_di = np.corrcoef(d.flatten().numpy(), i.flatten().numpy())[0, 1]
    c_if = np.corrcoef(w["li_logits"].float().flatten().numpy(), f.flatten().numpy())[0, 1]
    assert abs(c_di - 0.85) < 0.01 and abs(c_if - 0.8) < 0.01
    assert abs(float(d.std()) - 3.0) < 0.05
    lens, table = w["seq_lens"], w["block_table"]
    assert ((lens >= 512 + 8) & (lens <= 4096 + 8)).all()
    used = table[table >= 0]
    assert len(torch.unique(used)) == len(used)
    for b in range(16):
        n = (int(lens[b]) + 15) // 16
        assert (table[b, :n] >= 0).all() and (table[b, n:] == -1).all()


def test_greedy_drafts_are_argmax_and_temperatures():
    w = workloads.make_single(64, 5, 300, dtype="f32", law="t3", scale=4.0, alpha=(0.3, 0.99),
                              temps=(0.0, 0.7, 1.0), seed=(4, 0))
    t = w["temperature"]
    assert set(t.tolist()) <= {0.0, float(np.float32(0.7)), 1.0}
    assert (t == 0).any() and (t > 0).any()
    g = t == 0
    assert torch.equal(w["draft_tokens"][g], w["draft_logits"][g].argmax(-1).to(torch.int32))


def test_raw_view_round_trips():
    x = torch.randn(3, 7).to(torch.bfloat16)
    raw = workloads.to_numpy_raw(x)
    assert raw.dtype == np.uint16
    back = torch.from_numpy(raw.view(np.int16).copy()).view(torch.bfloat16)
    assert torch.equal(back, x)


def test_lmhead_shapes_laws_and_drafts():
    w = workloads.make_lmhead(6, 3, 700, 64, seed=(5, 1))
    assert w["h_draft"].shape == (6, 3, 64) and w["h_target"].shape == (6, 4, 64)
    assert w["w_vocab"].shape == (700, 64) and w["w_vocab"].dtype == torch.bfloat16
    assert abs(float(w["w_vocab"].float().std()) - 0.02) < 0.002
    assert abs(float(w["h_target"].float().std()) - 1.0) < 0.05
    assert w["draft_tokens"].dtype == torch.int32
    assert int(w["draft_tokens"].min()) >= 0 and int(w["draft_tokens"].max()) < 700
    w2 = workloads.make_lmhead(6, 3, 700, 64, seed=(5, 1))
    assert torch.equal(w["draft_tokens"], w2["draft_tokens"])
    g = workloads.make_lmhead(4, 2, 300, 32, temps=(0.0,), seed=(5, 2))
    logits = g["h_draft"].float() @ g["w_vocab"].float().T
    assert torch.equal(g["draft_tokens"].long(), logits.argmax(-1))
