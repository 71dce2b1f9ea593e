"""Paged global KV: the logical view of a page pool — TEST INFRASTRUCTURE ONLY.

[HF] abstract: the compressed global KV cache stays whole in HBM while a
server decodes batches of sequences of different lengths.  The pages fix no
memory layout for that; the reading used here (and by the library) is the
usual paged one: every per-position tensor of the cache lives in a pool of
pages of `page` positions, and a block table gives, for each sequence b and
logical block j, the page that holds positions j*page .. j*page + page - 1
(a negative entry: the block is unmapped and holds no positions).

Pinned by tests/test_oracle_paging.py: a hand-computed table of physical rows
for a tiny map, the identity map, and a pool scattered through a random
permutation that must come back unchanged.
"""
import numpy as np


def physical_row(block_table, page, b, p):
    """Physical pool row of sequence b's logical position p, or -1 when the
    block holding p is unmapped or beyond the table."""
    j = p // page
    if p < 0 or j >= block_table.shape[1]:
        return -1
    pg = int(block_table[b, j])
    if pg < 0:
        return -1
    return pg * page + p % page


def logical_view(pool, block_table, page, T):
    """Dense [B, T, ...] copy of a page pool [n_pages * page, ...] and the
    boolean map [B, T] of mapped positions (unmapped positions read as 0)."""
    pool = np.asarray(pool)
    block_table = np.asarray(block_table)
    B = block_table.shape[0]
    out = np.zeros((B, T) + pool.shape[1:], dtype=pool.dtype)
    mapped = np.zeros((B, T), dtype=bool)
    for b in range(B):
        for p in range(T):
            row = physical_row(block_table, page, b, p)
            if row >= 0:
                out[b, p] = pool[row]
                mapped[b, p] = True
    return out, mapped
