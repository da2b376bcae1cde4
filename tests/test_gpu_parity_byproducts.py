"""GPU parity of the by-products: row entropies and the verification-outcome
export (acceptance mass beta and the largest residual tokens per tested
position), through the C ABI, against the oracle.

Bars:
* entropy (nats) within ENT_TOL * (1 + H): each probability carries a relative
  error of a few fp32 ulps (exp2 of an fp32 exponent, fp32 scaling), so
  |dH| <= sum P |ln P + 1| eps ~ eps (H + 1) with eps ~ 1e-6; greedy rows are 0
  exactly;
* beta within PROB_ABS (the probability tolerance of the verification);
* the residual list: the sorted values of the top_m largest residuals are
  unique, so the exported masses match the oracle's sorted masses within
  PROB_ABS position by position; each exported token is distinct and its
  oracle residual matches its exported mass within PROB_ABS (so tokens whose
  residuals tie within the tolerance may come in either order); padding
  (-1, 0) only where the oracle's residual is within PROB_ABS of 0;
* greedy sequences (one-hot distributions) are exact;
* requesting by-products leaves the verification outputs unchanged.
"""

import numpy as np
import pytest
import torch

import workloads
from oracle import byproducts as ob
from oracle import numerics, rule
from tests import parity as P

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
ENT_TOL = 2e-5
PROB_ABS = 1e-5


@pytest.fixture(scope="module")
def sv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lossless_token_verification_amd as m
    m.library()
    return m


def _exits(w):
    if "ld_logits" in w:
        return [w["ld_logits"], w["li_logits"], w["lf_logits"]]
    return [w["draft_logits"], w["target_logits"]]


def _run(sv, w, seed=0, offset=0, **kw):
    g = P.to_device(w, DEV)
    if "ld_logits" in w:
        return sv.spec_verify_hier(g["ld_logits"], g["li_logits"], g["lf_logits"],
                                   g["draft_tokens"], g["temperature"], window=w.get("window", 4),
                                   seed=seed, offset=offset, **kw)
    return sv.spec_verify_single(g["draft_logits"], g["target_logits"], g["draft_tokens"],
                                 g["temperature"], seed=seed, offset=offset, **kw)


def _temps(w):
    t = w.get("temperature")
    return None if t is None else t.cpu().numpy()


def _split_entropy(flat, B, k, n_exits):
    sizes = [B * k] + [B * (k + 1)] * (n_exits - 1)
    out, o = [], 0
    for e, n in enumerate(sizes):
        out.append(flat[o:o + n].reshape(B, k if e == 0 else k + 1))
        o += n
    return out


def check_entropy(gpu_flat, w, sequences=None):
    exits = _exits(w)
    B, k = exits[0].shape[0], exits[0].shape[1]
    temps = _temps(w)
    got = _split_entropy(gpu_flat, B, k, len(exits))
    seqs = range(B) if sequences is None else sequences
    worst = 0.0
    for e, x in enumerate(exits):
        xr = P.raw(x)
        for b in seqs:
            tau = 1.0 if temps is None else float(temps[b])
            for j in range(xr.shape[1]):
                H = ob.entropy(numerics.row_distribution(numerics.decode(xr[b, j]), tau))
                g = float(got[e][b, j])
                if tau <= 0:
                    assert g == 0.0, (e, b, j, g)
                    continue
                err = abs(g - H)
                assert err <= ENT_TOL * (1 + H), (e, b, j, g, H)
                worst = max(worst, err / (1 + H))
    return worst


def _pair_rows(w, b, s, j, tau):
    exits = _exits(w)
    q = numerics.row_distribution(numerics.decode(P.raw(exits[s][b:b + 1, j])[0]), tau)
    p = numerics.row_distribution(numerics.decode(P.raw(exits[s + 1][b:b + 1, j])[0]), tau)
    return p, q


def check_outcome(out, w, top_m, sequences=None):
    exits = _exits(w)
    B, k = exits[0].shape[0], exits[0].shape[1]
    hier = len(exits) == 3
    temps = _temps(w)
    beta = out["accept_mass"].cpu().numpy()
    tok = out["residual_tokens"].cpu().numpy() if top_m else None
    mass = out["residual_mass"].cpu().numpy() if top_m else None
    seqs = range(B) if sequences is None else sequences
    checked = 0
    for b in seqs:
        tau = 1.0 if temps is None else float(temps[b])
        for s in range(2):
            for j in range(k + 1):
                valid = j < k if s == 0 else (hier and j <= k)
                if not valid:
                    assert np.isnan(beta[b, s, j])
                    if top_m:
                        assert (tok[b, s, j] == -1).all() and (mass[b, s, j] == 0).all()
                    continue
                p, q = _pair_rows(w, b, s, j, tau)
                ref_beta = ob.accept_mass(p, q)
                ref_tok, ref_mass = ob.residual_top(p, q, top_m) if top_m else (None, None)
                if tau <= 0:   # one-hots: exact
                    assert beta[b, s, j] == ref_beta, (b, s, j)
                    if top_m:
                        assert np.array_equal(tok[b, s, j], ref_tok), (b, s, j)
                        assert np.array_equal(mass[b, s, j], ref_mass.astype(np.float32))
                    checked += 1
                    continue
                assert abs(beta[b, s, j] - ref_beta) <= PROB_ABS, (b, s, j, beta[b, s, j], ref_beta)
                if top_m:
                    r = rule.residual(p, q)
                    gt, gm = tok[b, s, j], mass[b, s, j]
                    assert np.all(np.diff(gm) <= 0), gm
                    assert np.all(np.abs(gm - ref_mass) <= PROB_ABS), (b, s, j, gm, ref_mass)
                    real = gt[gt >= 0]
                    assert len(set(real.tolist())) == len(real)
                    assert np.all(real < r.size)
                    n = len(real)
                    assert np.all(gt[n:] == -1) and np.all(gm[n:] == 0)
                    assert np.all(np.abs(r[real] - gm[:n]) <= PROB_ABS), (b, s, j)
                    assert np.all(ref_mass[n:] <= PROB_ABS)
                checked += 1
    return checked


SINGLE = [
    # (B, k, V, dtype, temps, law)
    (6, 4, 70001, "bf16", (1.0,), "normal"),
    (5, 3, 40003, "f32", (0.0, 0.7, 1.0), "t3"),
    (4, 3, 1001, "bf16", (1.0, 0.5), "normal"),     # misaligned rows
    (3, 5, 515, "f32", (1.3,), "normal"),           # misaligned, tiny V
    (3, 0, 4096, "f32", (1.0,), "normal"),          # k = 0: nothing tested
    (2, 2, 1, "f32", (1.0,), "normal"),             # V = 1
    (2, 63, 2048, "bf16", (1.0,), "normal"),        # k = 63
]


@pytest.mark.parametrize("case", SINGLE, ids=lambda c: f"B{c[0]}k{c[1]}V{c[2]}{c[3]}")
@pytest.mark.parametrize("top_m", [8, 3])
def test_single_byproducts(sv, case, top_m):
    B, k, V, dt, temps, law = case
    w = workloads.make_single(B, k, V, dtype=dt, law=law, scale=3.0, alpha=(0.5, 0.95),
                              temps=temps, seed=(61, B, k, V))
    out = _run(sv, w, 1, 2, entropy=True, outcome=True, top_m=top_m, diag=True)
    torch.cuda.synchronize()
    worst = check_entropy(out["entropy"].cpu().numpy(), w)
    n = check_outcome(out, w, top_m)
    print(f"single {case[:4]} top_m={top_m}: entropy worst rel {worst:.2e}, {n} positions")
    # the verification itself is unchanged by the by-products
    base = _run(sv, w, 1, 2)
    torch.cuda.synchronize()
    for key in ("accept_len", "out_tokens", "num_emitted", "num_drop"):
        assert torch.equal(out[key], base[key])


HIER = [
    (6, 8, 50021, "bf16", (1.0,)),
    (5, 6, 20011, "f32", (0.0, 0.7, 1.0)),
    (4, 5, 3001, "bf16", (1.0,)),        # misaligned rows
    (3, 0, 5000, "bf16", (1.0,)),        # k = 0: stage 2 only, position 0
]


@pytest.mark.parametrize("case", HIER, ids=lambda c: f"B{c[0]}k{c[1]}V{c[2]}{c[3]}")
def test_hier_byproducts(sv, case):
    B, k, V, dt, temps = case
    w = workloads.make_hier(B, k, V, dtype=dt, temps=temps, window=4, seed=(62, B, k, V),
                            ctx=(16, 64))
    out = _run(sv, w, 3, 4, entropy=True, outcome=True, top_m=4)
    torch.cuda.synchronize()
    worst = check_entropy(out["entropy"].cpu().numpy(), w)
    n = check_outcome(out, w, 4)
    print(f"hier {case[:4]}: entropy worst rel {worst:.2e}, {n} positions")
    base = _run(sv, w, 3, 4)
    torch.cuda.synchronize()
    for key in ("accept_len_inter", "accept_len_final", "out_tokens", "num_emitted", "num_drop"):
        assert torch.equal(out[key], base[key])


def test_outcome_without_residuals_and_entropy_alone(sv):
    w = workloads.make_single(4, 3, 9000, dtype="bf16", temps=(1.0,), seed=(63,))
    out = _run(sv, w, outcome=True, top_m=0)
    torch.cuda.synchronize()
    assert "residual_tokens" not in out
    check_outcome(out, w, 0)
    out = _run(sv, w, entropy=True)
    torch.cuda.synchronize()
    check_entropy(out["entropy"].cpu().numpy(), w)


def test_identical_rows_accept_everything(sv):
    """q = p: beta = 1 (up to fp32 rounding) and no residual anywhere."""
    w = workloads.make_single(3, 4, 20000, dtype="bf16", temps=(1.0,), seed=(64,))
    w["target_logits"][:, :4] = w["draft_logits"]
    out = _run(sv, w, outcome=True, top_m=8)
    torch.cuda.synchronize()
    beta = out["accept_mass"].cpu().numpy()[:, 0, :4]
    assert np.all(np.abs(beta - 1.0) <= PROB_ABS)
    assert (out["residual_tokens"].cpu().numpy()[:, 0, :4] == -1).all()


@pytest.fixture(scope="module")
def full_size(sv):
    """The benchmarked call (hierarchy + KV rollback) at B=256 k=8 V=128256 bf16
    with every by-product, and the same call without them."""
    w = workloads.make("hier", 0, device=DEV)
    kw = dict(block_size=w["block_size"], max_freed=1, window=w["window"])
    t1, l1 = w["block_table"].clone(), w["seq_lens"].clone()
    out = sv.spec_verify_hier_rollback(w["ld_logits"], w["li_logits"], w["lf_logits"],
                                       w["draft_tokens"], w["temperature"], t1, l1,
                                       entropy=True, outcome=True, top_m=8, **kw)
    t2, l2 = w["block_table"].clone(), w["seq_lens"].clone()
    base = sv.spec_verify_hier_rollback(w["ld_logits"], w["li_logits"], w["lf_logits"],
                                        w["draft_tokens"], w["temperature"], t2, l2, **kw)
    torch.cuda.synchronize()
    host = {kk: (v.cpu() if torch.is_tensor(v) else v) for kk, v in out.items()}
    return dict(w=P._host(w), out=host, base=base, kv=(t1, l1, t2, l2), raw_out=out)


def test_full_size_byproducts_leave_outputs_unchanged(full_size):
    """Requesting the by-products changes no verification output or KV state."""
    out, base = full_size["raw_out"], full_size["base"]
    for key in ("accept_len_inter", "accept_len_final", "out_tokens", "num_emitted", "num_drop",
                "freed_blocks", "num_freed"):
        assert torch.equal(out[key], base[key]), key
    t1, l1, t2, l2 = full_size["kv"]
    assert torch.equal(t1, t2) and torch.equal(l1, l2)


def test_full_size_entropies(full_size):
    """Every row entropy of every sequence against the oracle."""
    w, out = full_size["w"], full_size["out"]
    worst = check_entropy(out["entropy"].numpy(), w)
    ent = out["entropy"].numpy()
    assert np.isfinite(ent).all() and (ent >= 0).all() and (ent <= np.log(w["V"]) + 1e-3).all()
    print(f"full size: entropy worst rel {worst:.2e}")


@pytest.mark.parametrize("half", [0, 1])
def test_full_size_outcome_export(full_size, half):
    """The outcome export (beta, top 8 residual tokens) of every tested
    position of every sequence against the oracle, in two halves of the batch."""
    w, out = full_size["w"], full_size["out"]
    B = w["B"]
    seqs = list(range(half * B // 2, (half + 1) * B // 2))
    n = check_outcome(out, w, 8, sequences=seqs)
    print(f"full size: outcome export of {n} positions (sequences {seqs[0]}..{seqs[-1]})")


def test_tied_and_clustered_residuals(sv):
    """Residuals that tie, or whose largest entries sit in one 16-byte vector
    (one thread of the kernel), take the exact path: ties come out in token
    order, as the oracle lists them."""
    B, k, V = 3, 2, 5000
    d = np.zeros((B, k, V), dtype=np.float32)
    t = np.zeros((B, k + 1, V), dtype=np.float32)
    d[0, 0, 0] = 8.0           # q ~ one-hot at 0; p puts equal mass on 8..15
    t[0, 0, 8:16] = 5.0
    d[1, 0, 3] = 30.0          # q one-hot at 3; p uniform: every other token ties
    d[2, 1, 100] = 30.0        # p's mass on 4 consecutive tokens of one vector
    t[2, 1, 4000:4004] = [6.0, 6.5, 6.25, 6.5]
    w = {"draft_logits": torch.from_numpy(d), "target_logits": torch.from_numpy(t),
         "draft_tokens": torch.zeros((B, k), dtype=torch.int32), "temperature": None}
    out = _run(sv, w, outcome=True, top_m=8)
    torch.cuda.synchronize()
    check_outcome(out, w, 8)
    tok = out["residual_tokens"].cpu().numpy()
    assert list(tok[0, 0, 0]) == list(range(8, 16))
    assert list(tok[1, 0, 0]) == [0, 1, 2, 4, 5, 6, 7, 8]
    assert list(tok[2, 0, 1][:4]) == [4001, 4003, 4002, 4000]


def _exact_lists(out, w, top_m, positions):
    """The exported lists at (b, s, j) equal the oracle's exactly: tokens in
    order (ties in token order) and masses within PROB_ABS."""
    tok = out["residual_tokens"].cpu().numpy()
    mass = out["residual_mass"].cpu().numpy()
    for b, s, j in positions:
        p, q = _pair_rows(w, b, s, j, 1.0)
        ref_tok, ref_mass = ob.residual_top(p, q, top_m)
        assert list(tok[b, s, j]) == list(ref_tok), (b, s, j, tok[b, s, j], ref_tok)
        assert np.all(np.abs(mass[b, s, j] - ref_mass) <= PROB_ABS), (b, s, j)


def test_outcome_large_residuals_in_one_thread(sv):
    """The largest residuals of a chunk all in groups of one thread (tokens
    2048 apart: one lane of the kernel for 256 or 128 threads), more than its
    list keeps: the chunk is scanned again exactly.  A second row has them in
    two threads, a third in consecutive vectors of one thread."""
    B, k, V = 3, 1, 70001
    g = torch.Generator().manual_seed(93)
    d = (torch.randn((B, k, V), generator=g) * 0.5).to(torch.bfloat16)
    t = d[:, :1].float().repeat(1, k + 1, 1).to(torch.bfloat16)
    for i in range(12):                       # 12 spikes, lane 5, distinct values
        t[0, 0, 5 * 8 + i * 2048 + (i % 8)] = 6.0 + 0.25 * i
    for i in range(12):                       # lanes 7 and 9 of chunk 1
        t[1, 0, 32768 + (7 if i % 2 else 9) * 8 + (i // 2) * 2048 + 3] = 7.0 - 0.125 * i
    for i in range(10):                       # vectors 16 apart (pairs of vectors)
        t[2, 0, 12 * 8 + i * 256 * 8 * 2 + 1] = 5.0 + 0.0625 * i
    w = {"draft_logits": d, "target_logits": t,
         "draft_tokens": torch.zeros((B, k), dtype=torch.int32), "temperature": None}
    out = _run(sv, w, outcome=True, top_m=8)
    torch.cuda.synchronize()
    check_outcome(out, w, 8)
    _exact_lists(out, w, 8, [(0, 0, 0), (1, 0, 0), (2, 0, 0)])


def test_outcome_ties_at_the_floor(sv):
    """Equal residuals (equal bf16 logit pairs) around the 8th place of a
    chunk: the tied groups are read again, and the list comes out in token
    order.  Row 0: 30 tied tokens over the 4 chunks; row 1: 40 tied tokens in
    one chunk, more groups than are read again (the exact rescan)."""
    B, k, V = 2, 1, 128256
    g = torch.Generator().manual_seed(94)
    d = (torch.randn((B, k, V), generator=g) * 0.5).to(torch.bfloat16)
    t = d[:, :1].float().repeat(1, k + 1, 1).to(torch.bfloat16)
    d2 = d.clone()
    tied0 = torch.randperm(V, generator=g)[:30]
    tied1 = torch.randperm(32768, generator=g)[:40] + 65536
    for b, tied in ((0, tied0), (1, tied1)):
        t[b, 0, tied] = 4.0
        d2[b, 0, tied] = -3.0
    w = {"draft_logits": d2, "target_logits": t,
         "draft_tokens": torch.zeros((B, k), dtype=torch.int32), "temperature": None}
    out = _run(sv, w, outcome=True, top_m=8)
    torch.cuda.synchronize()
    check_outcome(out, w, 8)
    _exact_lists(out, w, 8, [(0, 0, 0), (1, 0, 0)])
    tok = out["residual_tokens"].cpu().numpy()
    assert list(tok[0, 0, 0]) == sorted(tied0.tolist())[:8]
    assert list(tok[1, 0, 0]) == sorted(tied1.tolist())[:8]


def _mask(x, gen, frac, narrow_rows):
    """Masked vocabulary: a fraction `frac` of every row's logits set to -inf,
    and in `narrow_rows` (row indices of the flattened [B * n] rows) all but
    three entries.  In place; x is a CPU tensor [B, n, V]."""
    B, n, V = x.shape
    m = torch.rand((B, n, V), generator=gen) < frac
    flat = m.view(B * n, V)
    for r in narrow_rows:
        keep = torch.randperm(V, generator=gen)[:3]
        flat[r] = True
        flat[r, keep] = False
    x[m] = float("-inf")


@pytest.mark.parametrize("kind,dt", [("single", "bf16"), ("hier", "f32"), ("hier", "bf16")])
def test_masked_vocabulary(sv, kind, dt):
    """-inf logits (a masked vocabulary): the row statistics, the decisions,
    the draws, the entropies (the stream's unclamped T sums turn NaN on such
    chunks and are taken again with the clamp) and the outcome export all
    against the oracle.  Drafted tokens are drawn where q > 0 by the workload
    before masking, so some fall on masked entries (q(x) = 0 or p(x) = 0)."""
    B, k, V = 6, 4, 9001
    gen = torch.Generator().manual_seed(91)
    if kind == "single":
        w = workloads.make_single(B, k, V, dtype=dt, temps=(1.0, 0.7), seed=(66, V))
        _mask(w["draft_logits"], gen, 0.3, [1, 7])
        _mask(w["target_logits"], gen, 0.3, [2, 8])
        keys = ("accept_len", "out_tokens", "num_emitted", "num_drop")
        ref = P.oracle_single(w, 5, 6)
    else:
        w = workloads.make_hier(B, k, V, dtype=dt, temps=(1.0, 0.7), window=4, seed=(67, V),
                                ctx=(16, 64))
        _mask(w["ld_logits"], gen, 0.3, [1])
        _mask(w["li_logits"], gen, 0.3, [3, 9])
        _mask(w["lf_logits"], gen, 0.3, [4])
        keys = ("accept_len_inter", "accept_len_final", "out_tokens", "num_emitted", "num_drop")
        ref = P.oracle_hier(w, 5, 6, 4)
    out = _run(sv, w, 5, 6, entropy=True, outcome=True, top_m=4, diag=True)
    torch.cuda.synchronize()
    report = {}
    alt = P.alt_single(w, 5, 6) if kind == "single" else P.alt_hier(w, 5, 6, 4)
    P.compare(out, ref, keys, range(B), dt == "bf16", report, alt=alt)
    worst = check_entropy(out["entropy"].cpu().numpy(), w)
    n = check_outcome(out, w, 4)
    print(f"masked {kind} {dt}: {report}, entropy worst rel {worst:.2e}, {n} positions")
    assert report["compared"] >= B - 1
