"""Pins for the oracle's KV commit (CPU only).

What fixes the commit, independently of how the oracle is written:
  * the lesson page's exercise for its KV accounting step: two sequences
    verified together, A accepts every draft of a chain, B rejects at the
    second draft; both lengths come out right and no committed row changes
    (on a chain the accepted rows are already in place);
  * the other implementation the lesson page's "KV cache rollback" section
    names: keep the tree's rows in a scratch buffer and append the accepted
    ones on acceptance.  Appending scratch[path] to the prefix, done here with
    numpy fancy indexing, must give the same committed rows;
  * a hand-built tree whose rows hold their own indices, so every expected
    value is read off the path;
  * overlapping sources and destinations (path 0, 2, 3: row 1 <- 2, 2 <- 3),
    where a row-by-row copy done in the opposite order would be wrong;
  * the boundary's edge conventions: poisoned sequences commit the root,
    invalid paths and KV ranges move nothing and are flagged.
"""
import numpy as np
import pytest

from oracle import kv_commit as okc


def _cache(lens, T, Hkv=2, D=4, seed=0):
    rng = np.random.default_rng(seed)
    indptr = np.zeros(len(lens) + 1, dtype=np.int64)
    indptr[1:] = np.cumsum(np.asarray(lens) + T)
    k = rng.standard_normal((int(indptr[-1]), Hkv, D))
    v = rng.standard_normal((int(indptr[-1]), Hkv, D))
    return k, v, indptr


def _nodes(paths, T):
    out = np.full((len(paths), T), -1, dtype=np.int32)
    for b, p in enumerate(paths):
        out[b, :len(p)] = p
    return out


def test_lesson_exercise_two_sequences_on_a_chain():
    N = 5                      # drafts per step, a chain: node i is draft i
    T = N + 1
    lens = [7, 12]
    k, v, indptr = _cache(lens, T)
    accept_len = np.array([N, 1], dtype=np.int32)   # A: all drafts; B: rejected at the second draft
    nodes = _nodes([list(range(1, N + 1)), [1]], T)
    k2, v2, new_lens, flags = okc.kv_commit(k, v, indptr, lens, accept_len, nodes, T)
    assert new_lens.tolist() == [lens[0] + N + 1, lens[1] + 2]
    assert flags.tolist() == [0, 0]
    # a chain's accepted rows are already where they belong: nothing changes
    assert np.array_equal(k2, k) and np.array_equal(v2, v)


@pytest.mark.parametrize("seed", range(6))
def test_matches_scratch_buffer_commit(seed):
    rng = np.random.default_rng(100 + seed)
    T = int(rng.integers(2, 20))
    B = 3
    lens = [int(x) for x in rng.integers(0, 30, size=B)]
    k, v, indptr = _cache(lens, T, seed=seed)
    paths, alen = [], []
    for b in range(B):
        n = int(rng.integers(0, T))
        p = sorted(rng.choice(np.arange(1, T), size=n, replace=False).tolist())
        paths.append(p)
        alen.append(n)
    nodes = _nodes(paths, T)
    k2, v2, new_lens, flags = okc.kv_commit(k, v, indptr, lens, np.array(alen, dtype=np.int32), nodes, T)
    assert flags.tolist() == [0] * B
    for b in range(B):
        lo, L = int(indptr[b]), lens[b]
        scratch_k = k[lo + L: lo + L + T]          # the tree's rows, node order
        scratch_v = v[lo + L: lo + L + T]
        sel = np.array([0] + paths[b], dtype=np.int64)
        want_k = np.concatenate([k[lo: lo + L], scratch_k[sel]])
        want_v = np.concatenate([v[lo: lo + L], scratch_v[sel]])
        n_keep = L + 1 + alen[b]
        assert new_lens[b] == n_keep
        assert np.array_equal(k2[lo: lo + n_keep], want_k)
        assert np.array_equal(v2[lo: lo + n_keep], want_v)
        # rows past the new length keep what they held (rolled back, not cleared)
        assert np.array_equal(k2[lo + n_keep: int(indptr[b + 1])], k[lo + n_keep: int(indptr[b + 1])])


def test_hand_built_tree_rows_hold_their_indices():
    # root 0 -> 1, 2; 1 -> 3, 4; 3 -> 5.  Path accepted: 1, 3, 5.
    T, L = 6, 3
    rows = L + T
    k = np.arange(rows, dtype=np.float64).reshape(rows, 1, 1) * np.ones((1, 2, 4))
    v = -k
    indptr = np.array([0, rows], dtype=np.int64)
    k2, v2, new_lens, flags = okc.kv_commit(k, v, indptr, [L], np.array([3]), _nodes([[1, 3, 5]], T), T)
    assert new_lens.tolist() == [L + 4] and flags.tolist() == [0]
    assert k2[:, 0, 0].tolist() == [0, 1, 2, 3, 4, 6, 8, 7, 8]   # rows L+2 <- L+3, L+3 <- L+5
    assert np.array_equal(v2, -k2)


def test_overlapping_sources_and_destinations():
    T, L = 5, 2
    rows = L + T
    k = np.arange(rows, dtype=np.float64).reshape(rows, 1, 1)
    k2, _, new_lens, _ = okc.kv_commit(k, k.copy(), np.array([0, rows]), [L], np.array([2]),
                                       _nodes([[2, 3]], T), T)
    # row L+1 <- L+2, row L+2 <- L+3 (the value row L+2 held before the call)
    assert k2[:, 0, 0].tolist() == [0, 1, 2, 4, 5, 5, 6]
    assert new_lens.tolist() == [L + 3]


def test_poisoned_sequence_commits_the_root_only():
    T, lens = 4, [3]
    k, v, indptr = _cache(lens, T)
    k2, v2, new_lens, flags = okc.kv_commit(k, v, indptr, lens, np.array([-1]), _nodes([[]], T), T)
    assert new_lens.tolist() == [4] and flags.tolist() == [0]
    assert np.array_equal(k2, k) and np.array_equal(v2, v)


@pytest.mark.parametrize("path", [[2, 2], [3, 1], [0, 1], [1, 4], [-1]])
def test_invalid_path_moves_nothing(path):
    T, lens = 4, [5]
    k, v, indptr = _cache(lens, T)
    k2, v2, new_lens, flags = okc.kv_commit(k, v, indptr, lens, np.array([len(path)]), _nodes([path], T), T)
    assert flags.tolist() == [okc.FLAG_BAD_TREE] and new_lens.tolist() == [6]
    assert np.array_equal(k2, k) and np.array_equal(v2, v)


def test_accept_len_not_below_tree_rows():
    T, lens = 3, [2]
    k, v, indptr = _cache(lens, T)
    _, _, new_lens, flags = okc.kv_commit(k, v, indptr, lens, np.array([3]), _nodes([[1, 2]], T), T)
    assert flags.tolist() == [okc.FLAG_BAD_TREE] and new_lens.tolist() == [3]


def test_bad_kv_range_moves_nothing():
    T, lens = 4, [5, 2]
    k, v, indptr = _cache(lens, T)
    bad = indptr.copy()
    bad[1] -= 1                          # sequence 0 now holds one row too few
    k2, v2, new_lens, flags = okc.kv_commit(k, v, bad, lens, np.array([1, 1]), _nodes([[2], [3]], T), T)
    assert flags.tolist() == [okc.FLAG_BAD_KV_RANGE, 0]
    assert new_lens[0] == -1 and new_lens[1] == lens[1] + 2
    lo = int(bad[0])
    assert np.array_equal(k2[lo: lo + lens[0] + T], k[lo: lo + lens[0] + T])
