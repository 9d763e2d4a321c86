"""Paged K/V layouts for tests and benchmarks (input generation only).

`to_paged` scatters each sequence's contiguous rows (its prefix, then its
tree rows) into fixed-size pages placed at random slots of one page pool, as
a serving engine's block allocator leaves them, and returns the page table.
It moves rows and computes nothing else.
"""
import numpy as np


def to_paged(k, v, kv_indptr, prefix_lens, T, page_size, rng, spare_pages=3):
    """k, v: [rows, Hkv, D] contiguous (sequence b at rows kv_indptr[b] ..).
    Returns (k_paged, v_paged, table [B, pages_per_seq] int32); pages are
    drawn without replacement from a pool holding `spare_pages` more pages
    than needed (unused pages and table slots hold random garbage / page 0)."""
    B = len(prefix_lens)
    need = [(int(prefix_lens[b]) + T + page_size - 1) // page_size for b in range(B)]
    pps = max(need)
    pool = sum(need) + spare_pages
    slots = rng.permutation(pool)
    table = np.zeros((B, pps), dtype=np.int32)
    kp = np.empty((pool * page_size,) + k.shape[1:], dtype=k.dtype)
    vp = np.empty_like(kp)
    kp[...] = rng.integers(0, 1 << 8, size=kp.shape).astype(k.dtype) if kp.dtype != np.float32 else \
        rng.standard_normal(kp.shape).astype(np.float32)
    vp[...] = kp[::-1]
    at = 0
    for b in range(B):
        n = int(prefix_lens[b]) + T
        base = int(kv_indptr[b])
        for j in range(need[b]):
            page = int(slots[at])
            at += 1
            table[b, j] = page
            lo = j * page_size
            hi = min(n, lo + page_size)
            kp[page * page_size: page * page_size + (hi - lo)] = k[base + lo: base + hi]
            vp[page * page_size: page * page_size + (hi - lo)] = v[base + lo: base + hi]
    return kp, vp, table
