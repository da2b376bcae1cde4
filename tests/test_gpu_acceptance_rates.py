"""Acceptance frequencies of the full-size hierarchical verification (B=256,
k=8, V=128256 bf16, N_i=4) against the probabilities the oracle computes from
the same logits, within binomial bounds.

The drafts and logits are fixed; the GPU call is repeated with T Philox
offsets, so each trial draws fresh uniforms.  With float64 distributions Pd,
Pi, Pf of the oracle (row_distribution of the decoded logits):

* stage 1 accepts draft x_j, once reached, with probability
  m_j = min(1, Pi_j(x_j) / Pd_j(x_j)), independently per position, so
  P(a1 >= n) = m_0 ... m_{n-1}: the count of trials with a1 >= 1 and the sum
  of a1 are compared with their expectations;
* the first tentative token t_0 is x_0 with probability m_0, else the stage-1
  correction y ~ norm(max(0, Pi_0 - Pd_0)); stage 2 accepts a token v there
  with probability min(1, Pf_0(v) / Pi_0(v)), so the count of trials with
  a2 >= 1 has the expectation m_0 a(x_0) + (1 - m_0) sum_v r_v a(v) / R.

These are the standard rule's acceptance probabilities (the benchmark spec's
statement of the rule) evaluated from the oracle's distributions; the test
checks the GPU's decisions in aggregate at the full size, beside the
bit-exact comparison of sampled sequences elsewhere.
"""

import numpy as np
import pytest
import torch

import workloads
from oracle import numerics
from tests import parity as P

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TRIALS = 32
SIGMAS = 5.0


@pytest.fixture(scope="module")
def sv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lossless_token_verification_amd as m
    m.library()
    return m


def _dist(raw_rows, b, j, tau):
    return numerics.row_distribution(numerics.decode(raw_rows[b, j]), tau)


def test_full_size_acceptance_frequencies(sv):
    w = workloads.make("hier", 0, device=DEV)
    B, k = w["B"], w["k"]
    a1s, a2s = [], []
    for t in range(TRIALS):
        out = sv.spec_verify_hier(w["ld_logits"], w["li_logits"], w["lf_logits"],
                                  w["draft_tokens"], w["temperature"], window=w["window"],
                                  seed=0, offset=1000 + t)
        a1s.append(out["accept_len_inter"])
        a2s.append(out["accept_len_final"])
    torch.cuda.synchronize()
    a1 = torch.stack(a1s).cpu().numpy()   # [T, B]
    a2 = torch.stack(a2s).cpu().numpy()
    print(f"[acceptance] {TRIALS} trials of B={B} k={k}", flush=True)

    ld, li, lf = P.raw(w["ld_logits"].cpu()), P.raw(w["li_logits"].cpu()), P.raw(w["lf_logits"].cpu())
    x = w["draft_tokens"].cpu().numpy()
    temps = w["temperature"].cpu().numpy() if w.get("temperature") is not None else np.ones(B)

    m = np.zeros((B, k))
    e_a1 = np.zeros(B)
    var_a1 = np.zeros(B)
    e_s2 = np.zeros(B)
    for b in range(B):
        tau = float(temps[b])
        for j in range(k):
            pd, pi = _dist(ld, b, j, tau), _dist(li, b, j, tau)
            q, p = pd[x[b, j]], pi[x[b, j]]
            m[b, j] = 1.0 if q == 0.0 and p > 0.0 else (min(1.0, p / q) if q > 0.0 else 0.0)
            if j == 0:
                pi0, pd0 = pi, pd
        # distribution of a1: P(a1 = n) = m_0..m_{n-1} (1 - m_n), P(a1 = k) = prod m
        reach = np.concatenate([[1.0], np.cumprod(m[b])])          # P(a1 >= n), n = 0..k
        pn = reach[:-1] - reach[1:]
        pn = np.append(pn, reach[-1])
        n = np.arange(k + 1)
        e_a1[b] = (pn * n).sum()
        var_a1[b] = (pn * n * n).sum() - e_a1[b] ** 2
        # stage 2 at position 0
        pf0 = _dist(lf, b, 0, tau)
        with np.errstate(divide="ignore", invalid="ignore"):
            acc = np.where(pi0 > 0.0, np.minimum(1.0, pf0 / pi0), 0.0)
        r = np.maximum(0.0, pi0 - pd0)
        R = r.sum()
        corr = (r * acc).sum() / R if R > 0.0 else (pi0 * acc).sum()
        e_s2[b] = m[b, 0] * acc[x[b, 0]] + (1.0 - m[b, 0]) * corr

    def check(name, got, mean, var):
        bound = SIGMAS * np.sqrt(var) + 1.0
        print(f"[acceptance] {name}: got {got:.1f} expected {mean:.1f} bound {bound:.1f}", flush=True)
        assert abs(got - mean) <= bound, (name, got, mean, bound)

    m0 = m[:, 0]
    check("stage-1 accepts at position 0", float((a1 >= 1).sum()), TRIALS * m0.sum(),
          TRIALS * (m0 * (1 - m0)).sum())
    check("stage-1 accepted drafts", float(a1.sum()), TRIALS * e_a1.sum(), TRIALS * var_a1.sum())
    check("stage-2 accepts at position 0", float((a2 >= 1).sum()), TRIALS * e_s2.sum(),
          TRIALS * (e_s2 * (1 - e_s2)).sum())
    # not a degenerate workload: both stages accept and reject
    assert 0.05 < m0.mean() < 0.95 and 0.05 < e_s2.mean() < 0.95
