"""Pins of the oracle's block-table rollback: a slot-level brute force (which
physical blocks still hold a live KV slot) and conservation invariants."""

import numpy as np
import pytest

from oracle import blocktable


def _random_state(rng, B, bs, max_blocks):
    lens = rng.integers(0, max_blocks * bs + 1, B)
    pool = rng.permutation(B * max_blocks)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    pos = 0
    for b in range(B):
        n = -(-int(lens[b]) // bs)
        table[b, :n] = pool[pos:pos + n]
        pos += n
    return table, lens.astype(np.int32)


@pytest.mark.parametrize("bs", [1, 3, 16])
def test_rollback_brute_force_and_invariants(bs):
    rng = np.random.default_rng(bs)
    B, max_blocks = 200, 9
    table, lens = _random_state(rng, B, bs, max_blocks)
    drop = np.array([rng.integers(0, L + 1) for L in lens], dtype=np.int32)
    max_freed = max_blocks
    t2, l2, freed, nf = blocktable.kv_blocktable_truncate(table, lens, drop, bs, max_freed)
    for b in range(B):
        L, Ln = int(lens[b]), int(lens[b] - drop[b])
        live_before = [table[b, s // bs] for s in range(L)]
        live_after = [table[b, s // bs] for s in range(Ln)]
        gone = []
        for blk in live_before:            # in slot (hence logical) order, deduplicated
            if blk not in live_after and blk not in gone:
                gone.append(blk)
        assert l2[b] == Ln
        assert nf[b] == len(gone)
        assert list(freed[b, :nf[b]]) == gone and (freed[b, nf[b]:] == -1).all()
        keep = -(-Ln // bs)
        assert (t2[b, :keep] == table[b, :keep]).all() and (t2[b, keep:] == -1).all()
        # conservation of the physical ids
        before = sorted(x for x in table[b] if x >= 0)
        after = sorted([x for x in t2[b] if x >= 0] + list(freed[b, :nf[b]]))
        assert before == after
        assert nf[b] <= -(-int(drop[b]) // bs)


def test_rollback_rejects_bad_input():
    table = np.array([[5, 6, -1]], dtype=np.int32)
    with pytest.raises(ValueError):
        blocktable.kv_blocktable_truncate(table, np.array([20]), np.array([21]), 16, 3)
    with pytest.raises(ValueError):
        blocktable.kv_blocktable_truncate(table, np.array([20]), np.array([-1]), 16, 3)
    with pytest.raises(ValueError):
        blocktable.kv_blocktable_truncate(table, np.array([49]), np.array([0]), 16, 3)
    with pytest.raises(ValueError):
        blocktable.kv_blocktable_truncate(table, np.array([32]), np.array([32]), 16, 1)


def test_rollback_edge_cases():
    table = np.array([[5, 6, 7], [1, -1, -1], [-1, -1, -1]], dtype=np.int32)
    lens = np.array([33, 16, 0])
    t2, l2, freed, nf = blocktable.kv_blocktable_truncate(table, lens, np.array([1, 16, 0]), 16, 2)
    assert l2.tolist() == [32, 0, 0]
    assert nf.tolist() == [1, 1, 0]
    assert freed.tolist() == [[7, -1], [1, -1], [-1, -1]]
    assert t2.tolist() == [[5, 6, -1], [-1, -1, -1], [-1, -1, -1]]
