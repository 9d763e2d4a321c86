"""Pins for the oracle's tree attention (CPU only).

The oracle gathers each node's keys and runs plain attention.  It is pinned
against routines it does not use:
  * torch's scaled_dot_product_attention in float64 with a boolean mask whose
    tree part is built as the transitive closure of the parent relation
    (repeated boolean matrix products), and with GQA realised by repeating KV
    heads;
  * the chain special case: a chain tree is ordinary causal attention
    (scaled_dot_product_attention with is_causal=True over prefix + chain);
  * a one-row tree is plain decode attention;
  * closed forms: constant V rows give that constant; Q = 0 gives the mean of
    the visible V rows (prefix + depth + 1 of them).
"""
import numpy as np
import pytest
import torch

from oracle import attention as oa


def _random_tree(rng, T):
    par = [-1] + [int(rng.integers(0, i)) for i in range(1, T)]
    return np.asarray(par, dtype=np.int32)


def _case(rng, B=2, T=9, Hq=4, Hkv=2, D=16, lens=(13, 7), trees=None):
    q = rng.standard_normal((B, T, Hq, D))
    indptr = np.zeros(B + 1, dtype=np.int64)
    indptr[1:] = np.cumsum(np.asarray(lens) + T)
    k = rng.standard_normal((int(indptr[-1]), Hkv, D))
    v = rng.standard_normal((int(indptr[-1]), Hkv, D))
    if trees is None:
        trees = [_random_tree(rng, T) for _ in range(B)]
    return q, k, v, indptr, np.asarray(lens, dtype=np.int32), np.stack(trees)


def _closure_mask(parents):
    """anc[i, j] = j is i or an ancestor of i, via boolean matrix powers."""
    T = len(parents)
    adj = np.zeros((T, T), dtype=bool)
    for i in range(1, T):
        adj[i, parents[i]] = True
    reach = np.eye(T, dtype=bool)
    step = np.eye(T, dtype=bool)
    for _ in range(T):
        step = (step.astype(np.int64) @ adj.astype(np.int64)) > 0
        reach |= step
    return reach


def _sdpa_reference(q, k, v, indptr, lens, parents, scale):
    B, T, Hq, D = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    out = np.zeros_like(q)
    for b in range(B):
        L = int(lens[b])
        rows = slice(int(indptr[b]), int(indptr[b]) + L + T)
        kk = torch.from_numpy(k[rows]).permute(1, 0, 2).repeat_interleave(g, 0)   # [Hq, L+T, D]
        vv = torch.from_numpy(v[rows]).permute(1, 0, 2).repeat_interleave(g, 0)
        qq = torch.from_numpy(q[b]).permute(1, 0, 2)                              # [Hq, T, D]
        mask = np.zeros((T, L + T), dtype=bool)
        mask[:, :L] = True
        mask[:, L:] = _closure_mask(parents[b])
        o = torch.nn.functional.scaled_dot_product_attention(
            qq, kk, vv, attn_mask=torch.from_numpy(mask), scale=scale)
        out[b] = o.permute(1, 0, 2).numpy()
    return out


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_matches_masked_sdpa(seed):
    rng = np.random.default_rng(seed)
    q, k, v, indptr, lens, parents = _case(rng)
    scale = 1.0 / np.sqrt(q.shape[-1])
    got, flags = oa.tree_attention(q, k, v, indptr, lens, parents, scale)
    ref = _sdpa_reference(q, k, v, indptr, lens, parents, scale)
    assert not flags.any()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_chain_is_causal_attention():
    rng = np.random.default_rng(5)
    L, T, H, D = 11, 6, 3, 8
    chain = np.arange(-1, T - 1, dtype=np.int32)
    # full causal attention over prefix + chain; prefix queries are filler
    qfull = rng.standard_normal((H, L + T, D))
    k = rng.standard_normal((L + T, H, D))
    v = rng.standard_normal((L + T, H, D))
    scale = 0.37
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qfull), torch.from_numpy(k).permute(1, 0, 2),
        torch.from_numpy(v).permute(1, 0, 2), is_causal=True, scale=scale).numpy()
    q = qfull[:, L:, :].transpose(1, 0, 2)[None]          # [1, T, H, D]
    got, _ = oa.tree_attention(q, k, v, np.array([0, L + T]), np.array([L]), chain[None], scale)
    np.testing.assert_allclose(got[0], ref[:, L:, :].transpose(1, 0, 2), rtol=1e-12, atol=1e-12)


def test_single_row_tree_is_decode_attention():
    rng = np.random.default_rng(6)
    L, H, D = 40, 2, 16
    q = rng.standard_normal((1, 1, H, D))
    k = rng.standard_normal((L + 1, H, D))
    v = rng.standard_normal((L + 1, H, D))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q[0]).permute(1, 0, 2), torch.from_numpy(k).permute(1, 0, 2),
        torch.from_numpy(v).permute(1, 0, 2)).numpy()
    got, _ = oa.tree_attention(q, k, v, np.array([0, L + 1]), np.array([L]),
                               np.array([[-1]]), 1.0 / np.sqrt(D))
    np.testing.assert_allclose(got[0, 0], ref[:, 0, :], rtol=1e-12, atol=1e-12)


def test_constant_values_give_constant_output():
    rng = np.random.default_rng(7)
    q, k, v, indptr, lens, parents = _case(rng)
    const = rng.standard_normal(q.shape[-1])
    v[:] = const
    got, _ = oa.tree_attention(q, k, v, indptr, lens, parents, 0.25)
    np.testing.assert_allclose(got, np.broadcast_to(const, got.shape), rtol=1e-12, atol=1e-12)


def test_zero_query_gives_mean_of_visible_values():
    rng = np.random.default_rng(8)
    q, k, v, indptr, lens, parents = _case(rng)
    q[:] = 0.0
    got, _ = oa.tree_attention(q, k, v, indptr, lens, parents, 1.0)
    B, T, Hq, D = q.shape
    g = Hq // k.shape[1]
    for b in range(B):
        L = int(lens[b])
        base = int(indptr[b])
        for i in range(T):
            anc = {i}
            n = i
            while parents[b][n] >= 0:
                n = int(parents[b][n])
                anc.add(n)
            vis = list(range(base, base + L)) + [base + L + j for j in sorted(anc)]
            assert len(vis) == L + len(anc)
            for h in range(Hq):
                np.testing.assert_allclose(got[b, i, h], v[vis, h // g].mean(axis=0), rtol=1e-12,
                                           atol=1e-12)


def test_prefix_order_is_irrelevant():
    rng = np.random.default_rng(9)
    q, k, v, indptr, lens, parents = _case(rng, B=1, lens=(17,))
    got, _ = oa.tree_attention(q, k, v, indptr, lens, parents, 0.3)
    perm = rng.permutation(17)
    k2, v2 = k.copy(), v.copy()
    k2[:17], v2[:17] = k[perm], v[perm]
    got2, _ = oa.tree_attention(q, k2, v2, indptr, lens, parents, 0.3)
    np.testing.assert_allclose(got, got2, rtol=1e-12, atol=1e-12)


def test_invalid_tree_is_flagged():
    rng = np.random.default_rng(10)
    q, k, v, indptr, lens, parents = _case(rng)
    parents = parents.copy()
    parents[1, 4] = 6           # parent after child
    got, flags = oa.tree_attention(q, k, v, indptr, lens, parents, 0.3)
    assert flags[0] == 0 and flags[1] == oa.FLAG_BAD_TREE
    assert np.isnan(got[1]).all() and np.isfinite(got[0]).all()
