"""Paged-KV block-table rollback after verification.

Test infrastructure only (see ``oracle/__init__``).

The HiSpec summary (section 2, bullets "Wiederverwendung von KV-Cache und
versteckten Zustaenden" and "Unterstuetzung fuer Batch-Inferenz") buffers the KV
entries of drafted tokens, removes the entries of discarded tokens before the
next phase without recomputation, and batches sequences with paged attention and
block tables so each sequence keeps its own accepted length without padding.

Reading: one block table and one length per sequence.  A sequence holding L KV
slots drops its last num_drop slots; logical blocks that no longer hold any slot
(indices ceil(L'/bs) .. ceil(L/bs)-1, L' = L - num_drop) are released: their
physical ids are listed in ascending logical order and their table entries
become -1.  Blocks still partly used are kept.
"""

import numpy as np


def ceil_div(a, b):
    return -(-a // b)


def kv_blocktable_truncate(block_table, seq_lens, num_drop, block_size, max_freed):
    """Returns (table', lens', freed [B, max_freed] (-1 padded), num_freed [B]).
    Raises ValueError on num_drop outside [0, L], on L beyond the table, or when
    more than max_freed blocks would be released."""
    table = np.array(block_table, dtype=np.int32, copy=True)
    lens = np.array(seq_lens, dtype=np.int32, copy=True)
    B, max_blocks = table.shape
    freed = np.full((B, max_freed), -1, dtype=np.int32)
    num_freed = np.zeros(B, dtype=np.int32)
    for b in range(B):
        L = int(lens[b])
        d = int(num_drop[b])
        if d < 0 or d > L:
            raise ValueError(f"sequence {b}: num_drop {d} outside [0, {L}]")
        if ceil_div(L, block_size) > max_blocks:
            raise ValueError(f"sequence {b}: length {L} exceeds the block table")
        new_len = L - d
        keep = ceil_div(new_len, block_size)
        used = ceil_div(L, block_size)
        n = used - keep
        if n > max_freed:
            raise ValueError(f"sequence {b}: {n} blocks to free > max_freed {max_freed}")
        freed[b, :n] = table[b, keep:used]
        table[b, keep:used] = -1
        num_freed[b] = n
        lens[b] = new_len
    return table, lens, freed, num_freed
