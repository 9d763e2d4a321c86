"""Pins for the oracle's dynamic-tree expansion step (CPU only).

What fixes the step, independently of how the oracle is written:
  * values are log-probabilities: with every token a candidate (k >= V) and
    every candidate kept, the output is all (node, token) pairs ranked, and
    each value equals s_f + scipy's log_softmax(x_f / tau)[t];
  * a single frontier node at value 0 keeps its M most probable tokens in
    numpy's stable descending order of the logits;
  * per-node top-k is applied before the global ranking: a node whose k-th
    token is worse than another node's (k+1)-th still keeps k candidates
    while the other keeps only k (checked on a hand-built case);
  * invariances of the definition: adding a constant to a row's logits, or
    permuting the frontier rows together with their values, changes nothing
    but the parent indices;
  * a child's value never exceeds its parent's (log p <= 0), so values fall
    along every path;
  * inactive (-inf) frontier nodes and unusable rows are skipped, the latter
    flagged; short candidate lists are padded.
"""
import numpy as np
import pytest
from scipy.special import log_softmax

from oracle import tree_expand as ote


def _rng_case(seed, B=2, F=5, V=40, scale=2.0):
    rng = np.random.default_rng(seed)
    logits = (rng.standard_normal((B, F, V)) * scale).astype(np.float32)
    scores = -np.abs(rng.standard_normal((B, F))) * 3
    return logits, scores


@pytest.mark.parametrize("tau", [1.0, 0.7])
def test_all_candidates_are_log_probabilities(tau):
    logits, scores = _rng_case(1, F=3, V=12)
    B, F, V = logits.shape
    out = ote.expand(logits, scores, tau, V, F * V)
    for b in range(B):
        lp = log_softmax(logits[b].astype(np.float64) / tau, axis=-1)
        want = sorted(((scores[b, f] + lp[f, t], f, t) for f in range(F) for t in range(V)),
                      key=lambda c: (-c[0], c[1], c[2]))
        assert out["parent"][b].tolist() == [c[1] for c in want]
        assert out["token"][b].tolist() == [c[2] for c in want]
        np.testing.assert_allclose(out["value"][b], [c[0] for c in want], rtol=0, atol=1e-12)


def test_single_root_keeps_its_most_probable_tokens():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(300).astype(np.float32)
    x[17] = x[40] = x.max() + 1.0          # a tie at the top: the lower id first
    out = ote.expand(x[None, None, :], np.zeros((1, 1)), 1.0, 10, 6)
    order = np.argsort(-x.astype(np.float64), kind="stable")[:6]
    assert out["token"][0].tolist() == order.tolist()
    assert out["token"][0][:2].tolist() == [17, 40]
    assert out["parent"][0].tolist() == [0] * 6


def test_per_node_top_k_comes_before_the_global_ranking():
    # node 0 is confident: its 3rd token is still better than node 1's 1st;
    # with k = 2 node 0 contributes only two candidates
    V = 6
    x = np.full((1, 2, V), -10.0, dtype=np.float32)
    x[0, 0, :3] = [5.0, 4.9, 4.8]            # log p about -1.0, -1.1, -1.2
    x[0, 1, :] = 0.0                         # flat: log p = -log 6 = -1.79
    out = ote.expand(x, np.zeros((1, 2)), 1.0, 2, 4)
    assert out["parent"][0].tolist() == [0, 0, 1, 1]
    assert out["token"][0].tolist() == [0, 1, 0, 1]
    wide = ote.expand(x, np.zeros((1, 2)), 1.0, 3, 4)   # with k = 3 node 0's third token wins
    assert wide["parent"][0].tolist() == [0, 0, 0, 1]


def test_shift_and_permutation_invariance():
    logits, scores = _rng_case(3)
    logits = (np.round(logits * 1024) / 1024).astype(np.float32)   # a shift by 3.5 stays exact
    out = ote.expand(logits, scores, 1.0, 4, 7)
    shifted = logits + np.float32(3.5)
    out2 = ote.expand(shifted, scores, 1.0, 4, 7)
    assert out["token"].tolist() == out2["token"].tolist()
    assert out["parent"].tolist() == out2["parent"].tolist()
    np.testing.assert_allclose(out["value"], out2["value"], atol=1e-9)
    perm = np.array([3, 0, 4, 1, 2])
    out3 = ote.expand(logits[:, perm], scores[:, perm], 1.0, 4, 7)
    assert out3["token"].tolist() == out["token"].tolist()
    assert [[int(perm[p]) for p in row] for row in out3["parent"]] == out["parent"].tolist()


def test_children_never_exceed_their_parent():
    logits, scores = _rng_case(4, F=6, V=50)
    out = ote.expand(logits, scores, 1.0, 5, 12)
    for b in range(logits.shape[0]):
        for f, val in zip(out["parent"][b], out["value"][b]):
            assert val <= scores[b, f] + 1e-12


def test_inactive_unusable_and_short_lists():
    logits, scores = _rng_case(5, B=1, F=4, V=8)
    scores[0, 1] = -np.inf                  # inactive
    logits[0, 2, 3] = np.nan                # unusable row
    out = ote.expand(logits, scores, 1.0, 2, 10)
    assert out["flags"].tolist() == [ote.FLAG_NONFINITE]
    kept = [p for p in out["parent"][0] if p >= 0]
    assert sorted(set(kept)) == [0, 3] and len(kept) == 4
    assert out["parent"][0][4:].tolist() == [-1] * 6 and out["token"][0][4:].tolist() == [-1] * 6
    assert np.isneginf(out["value"][0][4:]).all()


def test_near_ties_are_counted_across_rows_only():
    x = np.zeros((1, 2, 4), dtype=np.float32)
    x[0, :, 0] = 1.0                         # both rows alike: cross-row ties
    out = ote.expand(x, np.zeros((1, 2)), 1.0, 4, 3)
    assert out["parent"][0].tolist() == [0, 1, 0]
    assert out["near_ties"][0] == 1          # the two rows' best tokens; row 0's equal tail is exact
    x1 = np.zeros((1, 1, 6), dtype=np.float32)   # one row, equal logits: exact ties, not counted
    assert ote.expand(x1, np.zeros((1, 1)), 1.0, 6, 5)["near_ties"][0] == 0


def _chain_of_steps(seed, B=2, V=50, steps=((4, 4), (3, 6), (2, 6))):
    rng = np.random.default_rng(seed)
    fr = np.zeros((B, 1))
    P, T, Vv = [], [], []
    for k, M in steps:
        F = fr.shape[1]
        x = (rng.standard_normal((B, F, V)) * 2).astype(np.float32)
        out = ote.expand(x, fr, 1.0, k, M)
        P.append(out["parent"]); T.append(out["token"]); Vv.append(out["value"].astype(np.float32))
        fr = out["value"]
    Mx = max(p.shape[1] for p in P)
    pad = lambda a, fill: np.stack([np.pad(x, ((0, 0), (0, Mx - x.shape[1])), constant_values=fill) for x in a])
    return pad(P, -1), pad(T, -1), pad(Vv, -np.inf)


def test_rerank_is_the_top_n_of_all_nodes_and_ancestor_closed():
    P, T, V = _chain_of_steps(21)
    D, B, M = P.shape
    N = 9
    out = ote.rerank(P, T, V, np.array([7, 8]), N)
    for b in range(B):
        # brute force: every node's value, the N largest (ties: earlier step, then rank)
        allv = sorted(((V[d, b, r], d, r) for d in range(D) for r in range(M) if P[d, b, r] >= 0),
                      key=lambda c: (-c[0], c[1], c[2]))[:N]
        assert out["rows"][b] == N + 1
        par, tok = out["parents"][b], out["tokens"][b]
        assert par[0] == -1 and tok[0] == [7, 8][b]
        assert all(0 <= par[i] < i for i in range(1, N + 1))          # a valid tree, parents first
        # each output row's path of tokens, rebuilt from the steps' parent links
        def path_tokens(d, r):
            toks = []
            while d >= 0:
                toks.append(int(T[d, b, r]))
                r = int(P[d, b, r])
                d -= 1
            return toks[::-1]
        def out_path(i):
            toks = []
            while i > 0:
                toks.append(int(tok[i]))
                i = int(par[i])
            return toks[::-1]
        assert sorted(map(tuple, (path_tokens(d, r) for _, d, r in allv))) == \
            sorted(map(tuple, (out_path(i) for i in range(1, N + 1))))


def test_rerank_keeps_everything_when_n_is_large():
    P, T, V = _chain_of_steps(22)
    out = ote.rerank(P, T, V, np.zeros(2, dtype=np.int32), 40)
    n = int((P >= 0).sum(axis=(0, 2))[0])
    assert out["rows"][0] == n + 1
    assert out["parents"][0][n + 1:].tolist() == [0] * (40 - n)      # padding rows: parent 0, token -1
    assert out["tokens"][0][n + 1:].tolist() == [-1] * (40 - n)


def test_short_rerank_output_is_a_padded_tree_for_verification():
    """Fewer candidates than rows: the rows past the kept nodes are padding
    that the acceptance walk accepts (no flag) with the result of the tree
    without them, and tree attention computes the real rows unchanged."""
    from oracle import accept as oacc
    from oracle import attention as oatt
    from oracle import philox
    P, T, V = _chain_of_steps(22)
    N = 40
    out = ote.rerank(P, T, V, np.array([3, 4], dtype=np.int32), N)
    rows = out["rows"]
    assert (rows < N + 1).all()
    rng = np.random.default_rng(5)
    B, Vv = 2, 50
    tgt = rng.standard_normal((B, N + 1, Vv)) * 2
    drf = tgt + rng.standard_normal((B, N + 1, Vv)) * 0.7
    toks = np.where(out["tokens"] >= 0, out["tokens"] % Vv, -1).astype(np.int32)
    toks[:, 0] = out["tokens"][:, 0]
    for temp in (1.0, 0.0):
        full = oacc.spec_accept(tgt, None if temp == 0 else drf, out["parents"], toks, temp, 11, 0)
        assert (full["flags"] & 7).tolist() == [0, 0]
        for b in range(B):
            n = int(rows[b])
            # the same uniforms: the sequence keeps its index in the batch
            alone = oacc.spec_accept(tgt[b:b + 1, :n], None if temp == 0 else drf[b:b + 1, :n],
                                     out["parents"][b:b + 1, :n], toks[b:b + 1, :n], temp, 11, 0,
                                     draw=lambda _b, nd, sl, bb=b: philox.uniform(11, 0, bb, nd, sl))
            assert full["accept_len"][b] == alone["accept_len"][0]
            assert full["out_tokens"][b, :n].tolist() == alone["out_tokens"][0].tolist()
    # attention: a padded row's parent is the root, a valid tree
    L, D = 16, 8
    k = rng.standard_normal((L + N + 1, D))
    v = rng.standard_normal((L + N + 1, D))
    q = rng.standard_normal(D)
    n = int(rows[0])
    for i in range(1, n):
        full_o = oatt.node_head_output(q, k, v, L, out["parents"][0], i, 0.3)
        part_o = oatt.node_head_output(q, k[:L + n], v[:L + n], L, out["parents"][0][:n], i, 0.3)
        assert np.allclose(full_o, part_o, rtol=0, atol=1e-14)
