"""Tree attention, float64 — oracle side (test infrastructure only).

What is computed (EAGLE verification with tree attention: one target forward
over the whole draft tree in which every candidate attends only to its own
ancestors, see the EAGLE notes page, core mechanism §3 and §5 and the
"tree attention" term; the speculative-decoding lesson page describes it as
ordinary flash attention with a custom, tree-shaped non-causal mask):

  for sequence b, tree node i, query head h and its KV head h' = h // g:
      keys(i) = prefix rows 0..L_b-1  U  tree rows of the nodes on the
                path root -> ... -> i (the node itself included)
      O[b,i,h] = sum_j softmax_j(scale * Q[b,i,h] . K_j) V_j,  j in keys(i)

This is exactly causal attention at the last position of the token sequence
prefix + path(i).  The oracle gathers keys(i) explicitly and applies no mask;
inputs are exact float64 images of the stored bf16/fp32 values.

Readings taken where the pages are silent: a node sees itself; the scale is an
argument (1/sqrt(D) by convention); Q and K arrive already position-encoded;
query head h reads KV head h // (Hq/Hkv).
"""
import numpy as np

FLAG_BAD_TREE = 1


def tree_is_valid(parents) -> bool:
    p = [int(x) for x in parents]
    if not p or p[0] != -1:
        return False
    return all(0 <= p[i] < i for i in range(1, len(p)))


def root_path(parents, i: int):
    """Node ids from the root to i, in root-first order."""
    path = []
    n = int(i)
    while n >= 0:
        path.append(n)
        n = int(parents[n])
    return path[::-1]


def attend(qvec, krows, vrows, scale):
    """softmax(scale * K q) V for one query vector over explicit key rows."""
    s = scale * (krows @ qvec)
    s = s - s.max()
    w = np.exp(s)
    w = w / w.sum()
    return w @ vrows


def node_rows(kv_begin: int, prefix_len: int, parents, i: int):
    """Absolute KV row indices node i may attend to."""
    path = root_path(parents, i)
    tree = kv_begin + prefix_len + np.asarray(path, dtype=np.int64)
    return np.concatenate([np.arange(kv_begin, kv_begin + prefix_len, dtype=np.int64), tree])


def tree_attention(q, k, v, kv_indptr, prefix_lens, parents, scale):
    """Full oracle.  q [B,T,Hq,D], k/v [rows,Hkv,D] (float64).

    Returns (out [B,T,Hq,D] float64, flags [B] uint32).  A sequence whose
    parent array is not a tree in topological order gets flag bit 0 and NaN
    outputs.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, T, Hq, D = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    out = np.full((B, T, Hq, D), np.nan)
    flags = np.zeros(B, dtype=np.uint32)
    for b in range(B):
        if not tree_is_valid(parents[b]):
            flags[b] |= FLAG_BAD_TREE
            continue
        for i in range(T):
            rows = node_rows(int(kv_indptr[b]), int(prefix_lens[b]), parents[b], i)
            for h in range(Hq):
                kh = h // g
                out[b, i, h] = attend(q[b, i, h], k[rows, kh, :], v[rows, kh, :], scale)
    return out, flags


def node_head_output(qvec, k_head, v_head, prefix_len, parents, i, scale):
    """One output row from a single sequence's K/V of one KV head.

    k_head, v_head: [L + T, D] float64 rows of that sequence and KV head.
    Used to check sampled outputs of workloads too large to run in full.
    """
    rows = node_rows(0, int(prefix_len), parents, i)
    return attend(np.asarray(qvec, dtype=np.float64), k_head[rows], v_head[rows], scale)
