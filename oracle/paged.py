"""Paged KV cache: the mapping from (sequence, slot) to (page, row).

TEST INFRASTRUCTURE ONLY (part of the oracle; see the package docstring).

[LA] "Troubleshooting Common Deployment Faults", item 3, names paged KV
buffers (PagedAttention) as the remedy for a contiguous per-sequence cache
that fragments memory.  The pages fix no layout; the reading used here: a
pool of pages [n_pages, page_size, n_kv, hd] and a block table
[batch, max_pages] such that slot j of sequence b is row j % page_size of
page table[b, j // page_size].  Attention over a paged cache is attention
over the cache this mapping gathers.
"""

import numpy as np


def gather(pool, table, page_size):
    """pool [n_pages, P, n_kv, hd], table [B, max_pages] -> contiguous
    caches [B, max_pages * P, n_kv, hd] (float64)."""
    pool = np.asarray(pool, dtype=np.float64)
    table = np.asarray(table, dtype=np.int64)
    B, max_pages = table.shape
    out = np.empty((B, max_pages * page_size) + pool.shape[2:], dtype=np.float64)
    for b in range(B):
        for i in range(max_pages):
            out[b, i * page_size:(i + 1) * page_size] = pool[table[b, i]]
    return out


def scatter(cache, table, n_pages, page_size, fill=np.nan):
    """Inverse of :func:`gather` for the pages a table references: caches
    [B, S, n_kv, hd] -> a pool [n_pages, P, n_kv, hd] whose other pages hold
    ``fill``."""
    cache = np.asarray(cache, dtype=np.float64)
    table = np.asarray(table, dtype=np.int64)
    B, max_pages = table.shape
    pool = np.full((n_pages, page_size) + cache.shape[2:], fill)
    for b in range(B):
        for i in range(max_pages):
            pool[table[b, i]] = cache[b, i * page_size:(i + 1) * page_size]
    return pool
