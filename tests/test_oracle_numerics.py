"""Pins of the oracle's decode and per-row distributions against library
routines (torch's bfloat16 conversion, SciPy's softmax) and closed forms."""

import numpy as np
import torch
from scipy import special

from oracle import numerics


def test_bf16_decode_exhaustive_against_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = numerics.decode_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().double().numpy()
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all()
    assert (ours[~nan] == ref[~nan]).all()
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_fp32_decode_is_exact():
    x = np.random.default_rng(0).normal(size=1000).astype(np.float32)
    assert (numerics.decode(x) == x.astype(np.float64)).all()


def test_softmax_matches_scipy():
    rng = np.random.default_rng(1)
    for tau in (0.3, 0.7, 1.0, 2.5):
        l = rng.normal(0, 4, size=5000)
        ref = special.softmax(l / tau)
        ours = numerics.row_distribution(l, tau)
        assert np.allclose(ours, ref, rtol=1e-12, atol=0)


def test_softmax_closed_forms():
    V = 777
    assert np.allclose(numerics.row_distribution(np.full(V, 3.25), 0.7), 1.0 / V, rtol=1e-15)
    l = np.zeros(10)
    l[4] = 2.0
    P = numerics.row_distribution(l, 0.5)
    e = np.exp(2.0 / 0.5)
    assert np.isclose(P[4], e / (e + 9), rtol=1e-14)
    assert np.allclose(np.delete(P, 4), 1.0 / (e + 9), rtol=1e-14)
    # large logits must not overflow (max subtracted first)
    assert np.isclose(numerics.row_distribution(np.array([1000.0, 999.0]), 1.0)[0],
                      1.0 / (1.0 + np.exp(-1.0)), rtol=1e-14)


def test_temperature_zero_is_first_argmax_and_limit():
    l = np.array([0.0, 2.0, -1.0, 2.0, 1.5])
    P = numerics.row_distribution(l, 0.0)
    assert P.tolist() == [0.0, 1.0, 0.0, 0.0, 0.0]
    l2 = np.array([0.0, 2.0, -1.0, 1.9, 1.5])
    P2 = numerics.row_distribution(l2, 1e-3)
    assert P2[1] == 1.0 and np.delete(P2, 1).max() < 1e-40
