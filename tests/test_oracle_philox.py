"""Pins of the oracle's Philox generator.

The round structure and key schedule are shared by all Philox-4xW widths; the
W = 64 instantiation is checked bit for bit against ``numpy.random.Philox``
(Philox4x64-10, a library routine), which pins the word order, the products,
the xors and the key bumps.  The W = 32 instance is pinned by the known-answer
vectors that the generator's authors publish with their Random123 library
(philox4x32, 10 rounds: zero counter and key, all-ones counter and key, and the
digits-of-pi counter and key).  Statistical checks cover the 24-bit uniforms
the verifier takes from it.
"""

import numpy as np
from scipy import stats

from oracle import philox


def _numpy_blocks(counter, key, n):
    """n consecutive Philox4x64-10 blocks from numpy, starting at ``counter``."""
    bg = np.random.Philox(counter=np.array(counter, dtype=np.uint64),
                          key=np.array(key, dtype=np.uint64))
    raw = bg.random_raw(4 * n)
    return [tuple(int(x) for x in raw[4 * i:4 * i + 4]) for i in range(n)]


def _ours64(counter, key):
    w = philox.philox4(tuple(int(c) for c in counter), tuple(int(k) for k in key),
                       philox.PHILOX_4x64, 10)
    return tuple(int(np.asarray(x).item()) for x in w)


def _add(counter, d):
    c0 = counter[0] + d
    return (c0 & (2 ** 64 - 1), counter[1] + (c0 >> 64), counter[2], counter[3])


# (counter, key, output) of Philox4x32-10, Random123 known-answer vectors
_KAT_4x32 = [
    ((0x00000000, 0x00000000, 0x00000000, 0x00000000), (0x00000000, 0x00000000),
     (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
    ((0xffffffff, 0xffffffff, 0xffffffff, 0xffffffff), (0xffffffff, 0xffffffff),
     (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
    ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
     (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
]


def test_philox4x32_known_answers():
    for counter, key, want in _KAT_4x32:
        w = philox.philox4(counter, key, philox.PHILOX_4x32, 10)
        assert tuple(int(np.asarray(x).item()) for x in w) == want


def test_round_structure_against_numpy_philox4x64():
    rng = np.random.default_rng(0)
    cases = [((0, 0, 0, 0), (0, 0))]
    for _ in range(12):
        cases.append((tuple(int(x) for x in rng.integers(0, 2 ** 63, 4)),
                      tuple(int(x) for x in rng.integers(0, 2 ** 63, 2))))
    cases.append(((2 ** 64 - 5, 3, 0, 7), (2 ** 64 - 1, 2 ** 64 - 1)))
    for counter, key in cases:
        got = _numpy_blocks(counter, key, 3)
        # numpy advances the counter before producing a block
        ours = [_ours64(_add(counter, d), key) for d in (1, 2, 3)]
        assert got == ours


def test_vectorised_32bit_matches_scalar_calls():
    j = np.arange(50, dtype=np.uint64)
    w = philox.block_words(j, 3, 1, 17, 0x1234567890AB)
    for i in (0, 7, 49):
        s = philox.block_words(np.uint64(i), 3, 1, 17, 0x1234567890AB)
        assert all(int(np.asarray(w[t])[i]) == int(np.asarray(s[t])) for t in range(4))
    assert all(int(np.max(x)) < 2 ** 32 for x in w)


def test_uniforms_range_and_resolution():
    j = np.arange(200000, dtype=np.uint64)
    u, v = philox.uniforms(j, 0, 0, 0, 0)
    for x in (u, v):
        assert x.min() >= 0.0 and x.max() <= 1.0 - 2.0 ** -24
        assert (x * 2 ** 24 == np.floor(x * 2 ** 24)).all()
        assert (x.astype(np.float32).astype(np.float64) == x).all()


def test_uniforms_chi_square():
    n = 1 << 20
    j = np.arange(n, dtype=np.uint64) % 4096
    b = np.arange(n, dtype=np.uint64) // 4096
    u, v = philox.uniforms(j, b, 1, 3, 99)
    for x in (u, v):
        cnt = np.bincount((x * 1024).astype(np.int64), minlength=1024)
        assert stats.chisquare(cnt).pvalue > 1e-4
    w = philox.block_words(j[:200000], b[:200000], 0, 0, 5)
    for word in w:
        word = np.asarray(word, dtype=np.uint64)
        for sh in (0, 8, 16, 24):
            cnt = np.bincount(((word >> np.uint64(sh)) & np.uint64(255)).astype(np.int64),
                              minlength=256)
            assert stats.chisquare(cnt).pvalue > 1e-4


def test_distinct_counters_give_distinct_blocks():
    j = np.arange(64, dtype=np.uint64)[:, None, None]
    b = np.arange(64, dtype=np.uint64)[None, :, None]
    s = np.arange(3, dtype=np.uint64)[None, None, :]
    w = philox.block_words(j, b, s, 0, 0)
    blocks = set(zip(*(np.asarray(x).ravel().tolist() for x in w)))
    assert len(blocks) == 64 * 64 * 3
    # seed and offset change the stream
    a = philox.block_words(np.uint64(1), 2, 0, 0, 0)
    assert a != philox.block_words(np.uint64(1), 2, 0, 1, 0)
    assert a != philox.block_words(np.uint64(1), 2, 0, 0, 1 << 32)
