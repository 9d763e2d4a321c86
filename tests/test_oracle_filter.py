"""Pins for the oracle's filtered distributions (top-k / top-p keep
thresholds, oracle/accept.py keep_threshold, and the walk over filtered rows;
CPU only).

What fixes them, independently of how the oracle is written:
  * hand-built rows whose kept sets follow from the definitions, ties
    included (a tie at the boundary keeps every tied token);
  * the transformers library's TopKLogitsWarper / TopPLogitsWarper (applied
    in that order, after the temperature) keep the same tokens on random
    rows away from the nucleus boundary;
  * exact enumeration: with children drawn from the filtered draft rows,
    the emitted token's law equals the filtered target distribution.
"""
import numpy as np
import pytest
from scipy.special import softmax as sp_softmax

from oracle import accept as oacc
from oracle import philox
from test_oracle_accept import _tables, enumerate_outcomes


def _kept(row, tau, k, p):
    th, near = oacc.keep_threshold(row, tau, k, p)
    return np.asarray(row) >= th, near


def test_hand_built_thresholds():
    x = np.log([0.5, 0.3, 0.15, 0.05])
    cases = [  # (top_k, top_p, kept)
        (0, 0.75, [1, 1, 0, 0]),      # 0.5 < 0.75 <= 0.8
        (0, 0.9, [1, 1, 1, 0]),       # 0.8 < 0.9 <= 0.95
        (0, 0.4, [1, 0, 0, 0]),
        (2, 0.0, [1, 1, 0, 0]),
        (3, 0.0, [1, 1, 1, 0]),
        (2, 0.6, [1, 0, 0, 0]),       # top-p over the two kept: 0.5 / 0.8 = 0.625 >= 0.6
        (2, 0.7, [1, 1, 0, 0]),       # ... 0.625 < 0.7
        (0, 1.0, [1, 1, 1, 1]),       # 1 = off
        (4, 0.0, [1, 1, 1, 1]),       # k = V keeps everything
        (0, 0.0, [1, 1, 1, 1]),
    ]
    for k, p, want in cases:
        kept, near = _kept(x, 1.0, k, p)
        assert kept.astype(int).tolist() == want, (k, p)
        assert not near
    # temperature: at tau = 0.5 the distribution is (25, 9, 2.25, 0.25) / 36.5
    kept, _ = _kept(x, 0.5, 0, 0.9)
    assert kept.astype(int).tolist() == [1, 1, 0, 0]        # 25 / 36.5 = 0.68 < 0.9 <= 34 / 36.5 = 0.93
    # ties at the boundary are kept whole
    y = np.log([0.4, 0.2, 0.2, 0.2])
    assert _kept(y, 1.0, 2, 0.0)[0].all()                   # the 2nd largest value is tied three times
    assert _kept(y, 1.0, 0, 0.5)[0].all()                   # mass above 0.2 is 0.4 < 0.5
    assert _kept(y, 1.0, 0, 0.3)[0].astype(int).tolist() == [1, 0, 0, 0]
    # -inf entries: k beyond the finite ones keeps everything
    z = np.array([1.0, -np.inf, 0.0, -np.inf])
    assert oacc.keep_threshold(z, 1.0, 3, 0.0)[0] == -np.inf


def test_boundary_within_the_margin_is_a_near_tie():
    x = np.log([0.5, 0.3, 0.2])
    assert oacc.keep_threshold(x, 1.0, 0, 0.8 - 0.5e-6)[1]      # kept mass 0.8 within 1e-6 above p
    assert oacc.keep_threshold(x, 1.0, 0, 0.8 + 0.5e-6)[1]      # mass above the boundary 0.8 within 1e-6 below p
    assert not oacc.keep_threshold(x, 1.0, 0, 0.8 - 2e-6)[1]
    assert not oacc.keep_threshold(x, 1.0, 0, 0.8 + 2e-6)[1]
    assert not oacc.keep_threshold(x, 1.0, 2, 0.0)[1]           # top-k is a count: never near


def test_matches_the_transformers_warpers():
    torch = pytest.importorskip("torch")
    tr = pytest.importorskip("transformers")
    rng = np.random.default_rng(4)
    checked = 0
    for trial in range(300):
        V = int(rng.integers(2, 400))
        row = rng.standard_normal(V) * rng.uniform(0.5, 4.0)
        tau = float(rng.choice([1.0, 0.7, 1.3]))
        k = int(rng.choice([0, 1, 2, 5, 20, V - 1, V + 3]))
        p = float(rng.choice([0.0, 0.3, 0.8, 0.95, 1.0]))
        kept, near = _kept(row, tau, k, p)
        if near:
            continue
        scores = torch.from_numpy(row / tau).view(1, -1)
        if k > 0:
            scores = tr.TopKLogitsWarper(top_k=min(k, V))(None, scores)
        if 0.0 < p < 1.0:
            scores = tr.TopPLogitsWarper(top_p=p)(None, scores)
        ref = torch.isfinite(scores).view(-1).numpy()
        assert kept.tolist() == ref.tolist(), (trial, V, k, p, tau)
        checked += 1
    assert checked > 250


def _filtered(rows_fn, tau, k, p):
    def rows(path):
        t, d = rows_fn(path)
        out = []
        for r in (t, d):
            th, _ = oacc.keep_threshold(r, tau, k, p)
            out.append(np.where(r < th, -np.inf, r))
        return tuple(out)
    return rows


@pytest.mark.parametrize("parents,V,k,p,tau", [
    ([-1, 0, 0, 0], 5, 3, 0.0, 1.0),
    ([-1, 0, 0, 0], 5, 0, 0.8, 1.0),
    ([-1, 0, 0, 1], 4, 3, 0.9, 0.8),
])
def test_lossless_exact_enumeration_with_filters(parents, V, k, p, tau):
    """Children i.i.d. from the filtered draft row of their parent; the first
    emitted token follows the filtered target row of the root exactly."""
    parents = np.asarray(parents)
    T = len(parents)
    rows = _filtered(_tables(V, 11, noise=1.0), tau, k, p)
    kids = oacc.tree_children(parents)
    first = np.zeros(V)

    def assign(c, tokens, weight):
        if c == T:
            paths = {0: ()}
            for n in range(1, T):
                paths[n] = paths[int(parents[n])] + (int(tokens[n]),)
            tgt = np.stack([rows(paths[n])[0] for n in range(T)])
            drf = np.stack([rows(paths[n])[1] for n in range(T)])

            def run(draw):
                path, final, _, _ = oacc.walk_sampled(lambda n: tgt[n], lambda n: drf[n], parents, tokens, tau,
                                                      lambda n, s: draw(0, n, s))
                return ([int(tokens[x]) for x in path] + [int(final)])[0]
            for out, pr in enumerate_outcomes(run).items():
                first[out] += weight * pr
            return
        par = int(parents[c])
        toks, n = [], par
        while n > 0:
            toks.append(int(tokens[n]))
            n = int(parents[n])
        pd = sp_softmax(rows(tuple(reversed(toks)))[1] / tau)
        for t in range(V):
            if pd[t] > 0:
                tokens[c] = t
                assign(c + 1, tokens, weight * pd[t])
        tokens[c] = 0

    assign(1, np.zeros(T, dtype=np.int64), 1.0)
    q_root = sp_softmax(rows(())[0] / tau)
    assert (q_root == 0).any()                    # the filter does cut tokens here
    np.testing.assert_allclose(first, q_root, rtol=0, atol=1e-12)
    assert kids[0]


def test_spec_accept_filters_both_rows_and_counts_boundary_ties():
    rng = np.random.default_rng(7)
    B, T, V = 3, 6, 40
    parents = np.tile(np.array([-1, 0, 0, 1, 1, 2]), (B, 1))
    tgt = rng.standard_normal((B, T, V)) * 2
    drf = tgt + rng.standard_normal((B, T, V)) * 0.8
    tokens = rng.integers(0, V, size=(B, T)).astype(np.int32)
    for k, p in ((5, 0.0), (0, 0.7), (8, 0.9)):
        got = oacc.spec_accept(tgt, drf, parents, tokens, 1.0, 3, 0, top_k=k, top_p=p)
        mt, md = tgt.copy(), drf.copy()
        for b in range(B):
            for n in range(T):
                for rows in (mt, md):
                    th, _ = oacc.keep_threshold(rows[b, n], 1.0, k, p)
                    rows[b, n] = np.where(rows[b, n] < th, -np.inf, rows[b, n])
        ref = oacc.spec_accept(mt, md, parents, tokens, 1.0, 3, 0)
        for key in ("accept_len", "accepted_nodes", "out_tokens", "flags"):
            assert np.array_equal(got[key], ref[key]), (k, p, key)
    # a root row whose nucleus boundary sits exactly on p: one near tie at
    # depth 0, slot 0 (every decision at the root depends on it)
    row = np.log([0.5, 0.3, 0.2])
    t1 = np.tile(row, (1, 2, 1))
    res = oacc.spec_accept(t1, t1, np.array([[-1, 0]]), np.array([[0, 0]]), 1.0, 3, 0, top_p=0.8)
    assert res["near_ties"][0] >= 1
    assert (res["first_near_depth"][0], res["first_near_slot"][0]) == (0, 0)
    # greedy ignores the filters
    g = oacc.spec_accept(tgt, None, parents, tokens, 0.0, 3, 0, top_k=1, top_p=0.5)
    g0 = oacc.spec_accept(tgt, None, parents, tokens, 0.0, 3, 0)
    assert np.array_equal(g["out_tokens"], g0["out_tokens"])
    assert philox.SAMPLE_SLOT
