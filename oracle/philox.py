"""Philox-4xW counter-based generator, restated from Salmon, Moraes, Dror, Shaw,
"Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11), section on Philox.

Test infrastructure only (see ``oracle/__init__``).

One Philox-4xW round maps the counter block (X0, X1, X2, X3) under the round key
(K0, K1) to

    (hi(M1*X2) ^ X1 ^ K0,  lo(M1*X2),  hi(M0*X0) ^ X3 ^ K1,  lo(M0*X0))

where hi/lo are the upper/lower W bits of the 2W-bit product.  The first round
uses the caller's key; before every later round the key is bumped by the Weyl
constants (K0 += C0, K1 += C1 mod 2^W).  Philox4x32-10 is W = 32 with ten rounds.

The same code serves W = 32 (uint64 NumPy arithmetic, products are exact below
2^64) and W = 64 (Python-int object arrays, exact 128-bit products).  The W = 64
instantiation exists only so that the round structure can be pinned against a
library (``numpy.random.Philox`` is Philox4x64-10); the W = 32 instance is
pinned by the authors' published known-answer vectors.

Uniform mapping used by the verifier (a reading, the pages fix none): a block is
drawn per (position j, sequence b, stage s, call offset), counter
(j, b, s, offset), key (seed & 0xffffffff, seed >> 32); word 0 gives the accept
uniform u = (w0 >> 8) * 2^-24 and word 1 the draw uniform v = (w1 >> 8) * 2^-24.
Both are exact in float32 and lie in [0, 1 - 2^-24].
"""

import numpy as np

# Published Philox constants (SC'11): multipliers and Weyl key increments.
PHILOX_4x32 = dict(width=32, mult=(0xD2511F53, 0xCD9E8D57), weyl=(0x9E3779B9, 0xBB67AE85))
PHILOX_4x64 = dict(width=64, mult=(0xD2E7470EE14C6C93, 0xCA5A826395121157),
                   weyl=(0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B))

STAGE_SINGLE = 0      # single-stage verify, and stage 1 (L_d -> L_i) of the hierarchy
STAGE_FINAL = 1       # stage 2 (L_i -> L_f) of the hierarchy


def _as_words(x, width):
    if width == 32:
        return np.asarray(x, dtype=np.uint64) & np.uint64(0xFFFFFFFF)
    arr = np.asarray(x, dtype=object)
    return np.vectorize(lambda v: int(v) & ((1 << 64) - 1), otypes=[object])(arr)


def philox4(counter, key, params=PHILOX_4x32, rounds=10):
    """Philox-4xW over broadcastable arrays.

    counter: sequence of 4 arrays (X0..X3); key: sequence of 2 arrays (K0, K1).
    Returns the 4 output words (uint64 arrays holding W-bit values for W = 32,
    object arrays of Python ints for W = 64).
    """
    w = params["width"]
    mask = (1 << w) - 1
    if w == 32:
        mask_a = np.uint64(mask)
        shift = np.uint64(32)
        m0, m1 = np.uint64(params["mult"][0]), np.uint64(params["mult"][1])
        c0, c1 = np.uint64(params["weyl"][0]), np.uint64(params["weyl"][1])
    else:
        mask_a, shift = mask, 64
        m0, m1 = params["mult"]
        c0, c1 = params["weyl"]
    x0, x1, x2, x3 = (_as_words(c, w) for c in counter)
    k0, k1 = (_as_words(k, w) for k in key)
    x0, x1, x2, x3, k0, k1 = np.broadcast_arrays(x0, x1, x2, x3, k0, k1)
    for r in range(rounds):
        if r > 0:
            k0 = (k0 + c0) & mask_a
            k1 = (k1 + c1) & mask_a
        p0 = m0 * x0          # exact: operands < 2^W
        p1 = m1 * x2
        hi0, lo0 = p0 >> shift, p0 & mask_a
        hi1, lo1 = p1 >> shift, p1 & mask_a
        x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
    return x0, x1, x2, x3


def block_words(j, b, stage, offset, seed):
    """Philox4x32-10 block for counter (j, b, stage, offset) under ``seed``."""
    seed = int(seed)
    key = (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    return philox4((j, b, stage, offset), key, PHILOX_4x32, 10)


def uniforms(j, b, stage, offset, seed):
    """(u, v) as float64 arrays: 24-bit uniforms from words 0 and 1."""
    w0, w1, _, _ = block_words(j, b, stage, offset, seed)
    scale = 2.0 ** -24
    u = (np.asarray(w0, dtype=np.uint64) >> np.uint64(8)).astype(np.float64) * scale
    v = (np.asarray(w1, dtype=np.uint64) >> np.uint64(8)).astype(np.float64) * scale
    return u, v
