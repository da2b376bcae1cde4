"""Helpers of the GPU parity tests: run the HIP path through the binding and
compare it with the CPU oracle on the same inputs.

Bars (as the tests state them):
* accepted lengths, emitted tokens, emitted counts and block tables are
  compared bit for bit, except for sequences the oracle marks as a near tie:
  an accept test with |u - p/q| < RATIO_EPS, or a draw whose threshold v*R lies
  within CDF_DELTA (probability units) of a CDF boundary of the chosen token;
* p(x), q(x) of every tested position agree within PROB_ABS (fp32 logits) or
  PROB_REL relative (bf16 logits);
* draw quantities (R, v*R, C(y-1), C(y)) of matching draws agree within
  CDF_DELTA.
"""

import numpy as np
import torch

import workloads
from oracle import lmhead as olm
from oracle import verify as ov

RATIO_EPS = 1e-5
CDF_DELTA = 1e-6
PROB_ABS = 1e-5
PROB_REL = 2e-3


def raw(t):
    return workloads.to_numpy_raw(t)


def oracle_single(w, seed, offset, sequences=None):
    temps = w["temperature"].cpu().numpy() if w.get("temperature") is not None else None
    return ov.spec_verify_single(raw(w["draft_logits"]), raw(w["target_logits"]),
                                 w["draft_tokens"].cpu().numpy(), temps, seed, offset,
                                 sequences=sequences)


def oracle_hier(w, seed, offset, window, sequences=None):
    temps = w["temperature"].cpu().numpy() if w.get("temperature") is not None else None
    return ov.spec_verify_hier(raw(w["ld_logits"]), raw(w["li_logits"]), raw(w["lf_logits"]),
                               w["draft_tokens"].cpu().numpy(), temps, seed, offset, window,
                               sequences=sequences)


def oracle_lmhead(w, seed, offset, sequences=None):
    temps = w["temperature"].cpu().numpy() if w.get("temperature") is not None else None
    return olm.spec_verify_lmhead_single(raw(w["h_draft"]), raw(w["h_target"]), raw(w["w_vocab"]),
                                         w["draft_tokens"].cpu().numpy(), temps, seed, offset,
                                         sequences=sequences)


def compare(gpu, ref, keys, sequences, bf16, report=None):
    """Bit-exact comparison of non-exempt sequences plus probability and draw
    tolerances.  Returns (number compared, number exempt)."""
    g = {k: gpu[k].cpu().numpy() for k in keys}
    exempt = [b for b in sequences if ov.near_tie(ref["infos"][b], RATIO_EPS, CDF_DELTA)]
    keep = [b for b in sequences if b not in exempt]
    for k in keys:
        bad = [b for b in keep if not np.array_equal(g[k][b], ref[k][b])]
        assert not bad, f"{k} differs at sequences {bad[:8]}: gpu {g[k][bad[0]]} " \
                        f"oracle {ref[k][bad[0]]}"
    if "diag_probs" in gpu:
        _check_probs(gpu, ref, keep, bf16, report)
    if report is not None:
        report["compared"] = report.get("compared", 0) + len(keep)
        report["exempt"] = report.get("exempt", 0) + len(exempt)
    return len(keep), len(exempt)


def _stage_infos(info):
    if "stage1" in info:
        return [info["stage1"], info["stage2"]]
    return [info]


def _check_probs(gpu, ref, keep, bf16, report):
    probs = gpu["diag_probs"].cpu().numpy()
    draws = gpu["diag_draws"].cpu().numpy()
    max_p = max_d = 0.0
    for b in keep:
        for s, info in enumerate(_stage_infos(ref["infos"][b])):
            n_t = len(info["tests"])
            # positions after a stage's stop were not tested: NaN
            rest = probs[b, s, n_t:]
            assert np.isnan(rest).all(), (b, s, rest)
            for j, (u, p, q) in enumerate(info["tests"]):
                gp, gq = probs[b, s, j]
                for o, gv in ((p, gp), (q, gq)):
                    err = abs(gv - o)
                    if bf16:
                        assert err <= PROB_REL * abs(o) + 1e-30, (b, s, j, gv, o)
                    else:
                        assert err <= PROB_ABS, (b, s, j, gv, o)
                    max_p = max(max_p, err / max(abs(o), 1e-30) if bf16 else err)
            d = info["draw"]
            if d is not None and np.isfinite(draws[b, s, 0]):
                R, t, clo, chi = draws[b, s]
                for gv, o in ((R, d["R"]), (t, d["t"]), (clo, d["c_lo"]), (chi, d["c_hi"])):
                    err = abs(gv - float(o))
                    assert err < CDF_DELTA, (b, s, gv, float(o))
                    max_d = max(max_d, err)
    if report is not None:
        report["max_prob_err"] = max(report.get("max_prob_err", 0.0), max_p)
        report["max_cdf_err"] = max(report.get("max_cdf_err", 0.0), max_d)


def to_device(w, dev):
    out = {}
    for k, v in w.items():
        out[k] = v.to(dev) if torch.is_tensor(v) else v
    return out
