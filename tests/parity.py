"""Helpers of the GPU parity tests: run the HIP path through the binding and
compare it with the CPU oracle on the same inputs.

Bars (as the tests state them):
* accepted lengths, emitted tokens, emitted counts and block tables are
  compared bit for bit, except for sequences the oracle marks as a near tie:
  an accept test with |u - p/q| < RATIO_EPS, or a draw whose threshold v*R lies
  within CDF_DELTA (probability units) of a CDF boundary of the chosen token;
* a near-tie sequence must still give one of the two outcomes the tie allows:
  the oracle's, or the oracle's with that one decision taken the other way
  (``alt``); only a tie whose other side is not one token (the R = 0 fallback)
  is left unchecked, and counted;
* at least a stated fraction of the sequences (``check_floor``) is checked
  against the oracle: bit for bit where the outcome is unique, against the
  two allowed outcomes where it is a near tie (at V = 128256 the residual draw
  often lands among tail tokens whose CDF steps are ~1e-6 wide, so ~10-20 %
  of the headline's sequences are near ties of the CDF band);
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


def _host(w):
    return {k: (v.cpu() if torch.is_tensor(v) else v) for k, v in w.items()}


def oracle_single(w, seed, offset, sequences=None, flips=None):
    temps = w["temperature"].cpu().numpy() if w.get("temperature") is not None else None
    return ov.spec_verify_single(raw(w["draft_logits"]), raw(w["target_logits"]),
                                 w["draft_tokens"].cpu().numpy(), temps, seed, offset,
                                 sequences=sequences, flips=flips)


def oracle_hier(w, seed, offset, window, sequences=None, flips=None):
    temps = w["temperature"].cpu().numpy() if w.get("temperature") is not None else None
    return ov.spec_verify_hier(raw(w["ld_logits"]), raw(w["li_logits"]), raw(w["lf_logits"]),
                               w["draft_tokens"].cpu().numpy(), temps, seed, offset, window,
                               sequences=sequences, flips=flips)


def oracle_lmhead(w, seed, offset, sequences=None, flips=None):
    temps = w["temperature"].cpu().numpy() if w.get("temperature") is not None else None
    return olm.spec_verify_lmhead_single(raw(w["h_draft"]), raw(w["h_target"]), raw(w["w_vocab"]),
                                         w["draft_tokens"].cpu().numpy(), temps, seed, offset,
                                         sequences=sequences, flips=flips)


def alt_single(w, seed, offset):
    """The ``alt`` argument of ``compare`` for a single-stage oracle run."""
    wc = _host(w)
    return lambda flips: oracle_single(wc, seed, offset, sequences=sorted(flips), flips=flips)


def alt_hier(w, seed, offset, window):
    wc = _host(w)
    return lambda flips: oracle_hier(wc, seed, offset, window, sequences=sorted(flips),
                                     flips=flips)


def alt_lmhead(w, seed, offset):
    wc = _host(w)
    return lambda flips: oracle_lmhead(wc, seed, offset, sequences=sorted(flips), flips=flips)


def compare(gpu, ref, keys, sequences, bf16, report=None, alt=None, ratio_eps=RATIO_EPS):
    """Bit-exact comparison of non-exempt sequences plus probability and draw
    tolerances.  Exempt (near-tie) sequences must equal the oracle's output or,
    given ``alt`` (flips -> oracle dict with those decisions taken the other
    way), that alternative; without ``alt`` they must equal the oracle's.
    Returns (number compared, number exempt)."""
    g = {k: gpu[k].cpu().numpy() for k in keys}
    events = {b: ov.near_tie_event(ref["infos"][b], ratio_eps, CDF_DELTA) for b in sequences}
    exempt = [b for b in sequences if events[b] is not None]
    keep = [b for b in sequences if events[b] is None]
    for k in keys:
        bad = [b for b in keep if not np.array_equal(g[k][b], ref[k][b])]
        assert not bad, f"{k} differs at sequences {bad[:8]}: gpu {g[k][bad[0]]} " \
                        f"oracle {ref[k][bad[0]]}"
    if "diag_probs" in gpu:
        _check_probs(gpu, ref, keep, bf16, report)

    def same(b, r):
        return all(np.array_equal(g[k][b], r[k][b]) for k in keys)

    flips = {b: events[b] for b in exempt if events[b]["flip"] is not None}
    other = alt(flips) if (alt is not None and flips) else None
    as_oracle = as_alt = unresolved = 0
    for b in exempt:
        if same(b, ref):
            as_oracle += 1
        elif other is not None and b in flips and same(b, other):
            as_alt += 1
        elif events[b]["flip"] is None:
            unresolved += 1
        else:
            raise AssertionError(
                f"near-tie sequence {b} ({events[b]}) matches neither the oracle nor the "
                f"outcome with that decision flipped: gpu {[g[k][b].tolist() for k in keys]} "
                f"oracle {[ref[k][b].tolist() for k in keys]}")
    if report is not None:
        report["compared"] = report.get("compared", 0) + len(keep)
        report["exempt"] = report.get("exempt", 0) + len(exempt)
        report["exempt_as_oracle"] = report.get("exempt_as_oracle", 0) + as_oracle
        report["exempt_as_flipped"] = report.get("exempt_as_flipped", 0) + as_alt
        report["exempt_unresolved"] = report.get("exempt_unresolved", 0) + unresolved
    return len(keep), len(exempt)


def check_floor(report, floor):
    """At least ``floor`` of the sequences were checked against the oracle:
    compared bit for bit, or (near ties) found equal to one of the two
    outcomes the tie allows; with fewer than 20 sequences in all, all but
    one.  Unresolved ties (the R = 0 fallback) do not count."""
    total = report.get("compared", 0) + report.get("exempt", 0)
    assert total > 0, report
    checked = total - report.get("exempt_unresolved", 0)
    need = floor * total if total >= 20 else total - 1
    assert checked >= need, \
        f"only {checked} of {total} sequences checked (floor {floor}): {report}"


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
