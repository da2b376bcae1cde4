"""Pins of the LM-head oracle (CPU).

The head's logits reduce to known quantities when W's rows are scaled unit
vectors: l[v] = c_v * h[pi(v)].  Then the LM-head verify must equal the
already pinned single-stage verify on those logits, which catches a transposed
head, the wrong hidden rows or positions, and a wrong vocabulary order.
"""

import numpy as np
import pytest

from oracle import lmhead, numerics, verify


def bf16_bits(x):
    """float -> bf16 bits by truncation (inputs here are exactly representable)."""
    f = np.asarray(x, dtype=np.float32)
    bits = (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    assert np.array_equal(numerics.decode_bf16(bits), f.astype(np.float64))
    return bits


def unit_head(V, d, rng):
    """W [V, d] with W[v] = c_v * e_{pi(v)}: c_v in {1, 2, 0.5}, pi onto [0, d)."""
    pi = np.concatenate([rng.permutation(d), rng.integers(0, d, V - d)])
    c = rng.choice([1.0, 2.0, 0.5], V)
    W = np.zeros((V, d), dtype=np.float32)
    W[np.arange(V), pi] = c
    return W, pi, c


@pytest.mark.parametrize("B,k,d,V", [(3, 4, 16, 21), (2, 2, 8, 8), (4, 0, 12, 15)])
def test_unit_head_reduces_to_single_stage(B, k, d, V):
    rng = np.random.default_rng(7 + B + k)
    # hidden values on a coarse grid so every logit is exact in bf16 and float64
    Hd = np.round(rng.normal(0, 2, (B, k, d)) * 8) / 8
    Ht = np.round(rng.normal(0, 2, (B, k + 1, d)) * 8) / 8
    W, pi, c = unit_head(V, d, rng)
    tokens = rng.integers(0, V, (B, k)).astype(np.int32)
    temps = np.array([1.0, 0.7, 0.0, 1.3][:B])
    got = lmhead.spec_verify_lmhead_single(bf16_bits(Hd), bf16_bits(Ht), bf16_bits(W), tokens,
                                           temps, 5, 9)
    ld = (Hd[:, :, pi] * c).astype(np.float32)
    lt = (Ht[:, :, pi] * c).astype(np.float32)
    ref = verify.spec_verify_single(ld, lt, tokens, temps, 5, 9)
    for key in ("accept_len", "num_emitted", "out_tokens", "num_drop"):
        assert np.array_equal(got[key], ref[key]), key


def test_logits_against_unit_head_and_linearity():
    rng = np.random.default_rng(3)
    d, V = 10, 13
    H = np.round(rng.normal(0, 1, (5, d)) * 16) / 16
    W, pi, c = unit_head(V, d, rng)
    L = lmhead.lmhead_logits(bf16_bits(H), bf16_bits(W), chunk=4)
    assert np.array_equal(L, H[:, pi] * c)
    # a head that is the sum of two unit heads gives the sum of their logits
    W2, pi2, c2 = unit_head(V, d, rng)
    L2 = lmhead.lmhead_logits(bf16_bits(H), bf16_bits(W + W2), chunk=5)
    assert np.allclose(L2, H[:, pi] * c + H[:, pi2] * c2, rtol=0, atol=1e-12)


def test_subset_of_sequences_and_shape_checks():
    rng = np.random.default_rng(11)
    B, k, d, V = 4, 3, 8, 9
    Hd = bf16_bits(np.round(rng.normal(0, 2, (B, k, d)) * 4) / 4)
    Ht = bf16_bits(np.round(rng.normal(0, 2, (B, k + 1, d)) * 4) / 4)
    W = bf16_bits(unit_head(V, d, rng)[0])
    tok = rng.integers(0, V, (B, k)).astype(np.int32)
    full = lmhead.spec_verify_lmhead_single(Hd, Ht, W, tok, None, 1, 2)
    part = lmhead.spec_verify_lmhead_single(Hd, Ht, W, tok, None, 1, 2, sequences=[1, 3])
    for b in (1, 3):
        assert np.array_equal(part["out_tokens"][b], full["out_tokens"][b])
    assert (part["accept_len"][[0, 2]] == -1).all()
    with pytest.raises(ValueError):
        lmhead.spec_verify_lmhead_single(Hd, Hd, W, tok, None, 1, 2)
