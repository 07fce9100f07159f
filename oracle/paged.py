"""Paged latent cache for the oracle: where a sequence's rows live in a pool
of fixed-size pages.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Transformer and KV Cache Basics" (KV Cache section, Engineering) keeps its
cache in one preallocated buffer per sequence and names a growing memory pool
as the next step; the "Multi-Head Latent Attention" post's code (section 3.7)
also preallocates.  Reading: a paged cache is a
pool of rows cut into pages of P rows (page k = pool rows [k P, (k + 1) P));
each sequence lists its pages in a block table, and its position t is pool row
    table[b][t // P] * P + t % P.
Pages may be shared (a common prefix) and need not be in order.  What the
attention computes does not change: the rows of sequence b, in position
order, are the same rows a contiguous cache would hold.
"""

from __future__ import annotations

import numpy as np


def row_index(table, page_rows: int, b: int, t) -> np.ndarray:
    """Pool row of position(s) t of sequence b."""
    t = np.asarray(t, dtype=np.int64)
    tab = np.asarray(table, dtype=np.int64)
    return tab[b, t // page_rows] * page_rows + t % page_rows


def gather(pool, table, page_rows: int, seq_len) -> list:
    """The rows of every sequence in position order, read through the block
    table: a list of (seq_len[b], R) arrays."""
    pool = np.asarray(pool)
    return [pool[row_index(table, page_rows, b, np.arange(int(n)))]
            for b, n in enumerate(seq_len)]


def pages_needed(seq_len, page_rows: int) -> np.ndarray:
    """Pages sequence b occupies: ceil(seq_len[b] / P)."""
    return (np.asarray(seq_len, dtype=np.int64) + page_rows - 1) // page_rows
