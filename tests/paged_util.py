"""Test helper: lay a contiguous cache out as a paged pool with a shuffled block table.

The pool holds every sequence's blocks at random places, plus spare blocks
that no table names; spare blocks and table entries past a sequence's last
needed block carry poison (NaN rows, id -1), so a kernel that reads what it
should not shows it in the result.
"""
from __future__ import annotations

import numpy as np


def nan_like(dtype):
    return np.uint16(0x7FC0) if dtype == np.uint16 else np.float32(np.nan)


def make_paged(cache: np.ndarray, lens, block_size: int, rng, *, spare: int = 3, room: int = 1):
    """Pool [num_blocks, g, B, d] and table int32 [b, max_blocks] standing for ``cache`` [b, g, cap, d].

    Sequence s gets ceil((lens[s] + room) / B) blocks (room: positions an append may still need);
    table entries after those are -1. Rows of the cache are copied for every position its blocks cover.
    """
    b, g, cap, d = cache.shape
    lens = np.asarray(lens)
    max_blocks = (cap + block_size - 1) // block_size
    need = [min(max_blocks, (int(lens[s]) + room + block_size - 1) // block_size) for s in range(b)]
    num_blocks = sum(need) + spare
    ids = rng.permutation(num_blocks).astype(np.int32)
    pool = np.full((num_blocks, g, block_size, d), nan_like(cache.dtype), dtype=cache.dtype)
    table = np.full((b, max_blocks), -1, dtype=np.int32)
    k = 0
    for s in range(b):
        for n in range(need[s]):
            blk = int(ids[k])
            k += 1
            table[s, n] = blk
            rows = cache[s, :, n * block_size:(n + 1) * block_size]
            pool[blk, :, :rows.shape[1]] = rows
    return pool, table


def scatter_rows(pool, table, cache, s, block_size):
    """Write every row of sequence s that its blocks cover from ``cache`` back into ``pool`` (numpy)."""
    for n in range(table.shape[1]):
        blk = table[s, n]
        if blk >= 0:
            rows = cache[s, :, n * block_size:(n + 1) * block_size]
            pool[blk, :, :rows.shape[1]] = rows
