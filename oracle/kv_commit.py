"""Committing the accepted path into the KV cache — oracle side (test
infrastructure only).

What the step does (lesson page, the "KV cache rollback" section and build
step 4, "KV accounting"): the verification forward has written K/V rows for
every tree node behind the sequence's prefix; once the walk is known, the
rows of the accepted nodes become the next positions of the cache and the
logical length moves past them, while the rows of rejected nodes are simply
left behind (rollback by logical length, no copy of them).  For a tree the
accepted nodes are not contiguous, so their rows are compacted:

  rows of sequence b: kv_indptr[b] + j, j = 0 .. L_b + T - 1
      prefix rows j < L_b, tree node i at row L_b + i
  path: node 0 (the root: the already committed token whose K/V this step
        computed), then accepted_nodes[b, 0 .. n-1], n = accept_len[b]
  after the step: row L_b + i holds what row L_b + path[i] held before,
                  i = 0 .. n; every other row is left as it was
  new length: L_b + n + 1 (the final sampled token has no K/V yet: it is the
              next step's root)

Readings where the pages are silent (each listed in the design notes):
  * the root row is part of the committed path (its K/V were computed by this
    verification forward, it is the token the previous step emitted);
  * accept_len < 0 (a poisoned sequence): only the root is committed;
  * the path must be strictly increasing node indices in [1, T) (a root path
    of a tree whose parents precede their children); otherwise nothing moves,
    the length becomes L_b + 1 and the sequence is flagged BAD_TREE;
  * kv_indptr[b] .. kv_indptr[b+1] must hold L_b + T rows inside
    [0, num_kv_rows); otherwise nothing moves, the length is -1 and the
    sequence is flagged BAD_KV_RANGE (the flag values of the boundary).

Plain numpy: every source row is read from a copy of the input before any
row is written, exactly as the definition says.
"""
import numpy as np

FLAG_BAD_TREE = 1
FLAG_BAD_KV_RANGE = 32


def kv_commit(k, v, kv_indptr, prefix_lens, accept_len, accepted_nodes, tree_rows):
    """k, v: [num_kv_rows, Hkv, D] arrays (any dtype, not modified).
    kv_indptr [B+1] int64, prefix_lens [B], accept_len [B], accepted_nodes [B, T].
    Returns (k_new, v_new, new_lens [B] int32, flags [B] uint32)."""
    k_in, v_in = np.asarray(k), np.asarray(v)
    k_out, v_out = k_in.copy(), v_in.copy()
    B = len(prefix_lens)
    T = int(tree_rows)
    rows = k_in.shape[0]
    new_lens = np.zeros(B, dtype=np.int32)
    flags = np.zeros(B, dtype=np.uint32)
    for b in range(B):
        L = int(prefix_lens[b])
        lo, hi = int(kv_indptr[b]), int(kv_indptr[b + 1])
        if lo < 0 or lo + L + T > hi or hi > rows:
            flags[b] = FLAG_BAD_KV_RANGE
            new_lens[b] = -1
            continue
        n = int(accept_len[b])
        path = [0] + [int(x) for x in accepted_nodes[b][:max(n, 0)]]
        ok = n < T and all(0 < path[i] < T for i in range(1, len(path))) and \
            all(path[i - 1] < path[i] for i in range(1, len(path)))
        if not ok:
            flags[b] = FLAG_BAD_TREE
            new_lens[b] = L + 1
            continue
        base = lo + L
        for i, node in enumerate(path):
            k_out[base + i] = k_in[base + node]
            v_out[base + i] = v_in[base + node]
        new_lens[b] = L + len(path)
    return k_out, v_out, new_lens, flags
