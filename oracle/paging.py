"""Paged K/V — oracle side (test infrastructure only).

A serving engine keeps each sequence's K/V rows in fixed-size pages of one
pool and a per-sequence page table (the pages' serving regime: a batch of
requests whose caches grow independently).  The verification path computes
exactly what it computes on the contiguous rows; paging only relabels rows:
logical row x of sequence b is physical row
    table[b, x // page_size] * page_size + x % page_size.
`gather` undoes the relabelling, so every other oracle function applies to
its result unchanged.
"""
import numpy as np


def physical_row(table, b, x, page_size):
    return int(table[b, x // page_size]) * page_size + x % page_size


def gather(paged, table, b, n, page_size):
    """Sequence b's first n logical rows of a paged array, in order."""
    idx = [physical_row(table, b, x, page_size) for x in range(n)]
    return np.asarray(paged)[np.asarray(idx, dtype=np.int64)]
