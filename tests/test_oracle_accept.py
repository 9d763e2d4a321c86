"""Pins for the oracle's multi-round speculative sampling (CPU only).

What fixes the walk, independently of how the oracle is written:
  * losslessness (the lesson page's Leviathan invariant; the EAGLE notes
    page's claim that the output distribution equals the target's): exact
    enumeration over every draft-token draw and every branch of every
    uniform, on tiny vocabularies, drives the oracle's own code and must give
    the target distribution to 1e-12 (first token, and the second token given
    the first);
  * the same, statistically, over Philox offsets (chi-square, as the lesson's
    build step 5 describes);
  * the chain closed form E[emitted] = (1 - a^(N+1)) / (1 - a) under a
    constant per-token acceptance rate a (lesson page, "what sets the
    speedup"), exactly by enumeration and by Monte Carlo;
  * greedy mode equals textbook greedy decoding of the target along the tree;
  * special cases: identical target and draft always accept the first child;
    disjoint supports reject every child;
  * the edge conventions of the lesson's accept() and residual() helpers.
"""
from collections import defaultdict

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax
from scipy.stats import chi2 as chi2_dist

from oracle import accept as oacc
from oracle import philox


# ---------------------------------------------------------------------------
# exact enumeration of the oracle's decision tree
# ---------------------------------------------------------------------------
class _Driver:
    """Feeds the walk symbolic uniforms and follows a script of branch choices."""

    def __init__(self, script):
        self.script = script
        self.pos = 0
        self.prob = 1.0
        self.points = []

    def decide(self, p_true):
        p_true = min(max(p_true, 0.0), 1.0)
        if self.pos < len(self.script):
            take = self.script[self.pos]
        else:
            take = False
            self.points.append((self.pos, p_true))
        self.pos += 1
        self.prob *= p_true if take else (1.0 - p_true)
        return take

    def draw(self, b, node, slot):
        return _SymU(self)


class _SymU:
    """A uniform on [lo, hi) whose comparisons branch with exact probabilities."""

    def __init__(self, drv):
        self.drv, self.lo, self.hi = drv, 0.0, 1.0

    def below(self, x):
        width = self.hi - self.lo
        p = 0.0 if width <= 0 else (min(max(x, self.lo), self.hi) - self.lo) / width
        take = self.drv.decide(p)
        if take:
            self.hi = min(self.hi, x)
        else:
            self.lo = max(self.lo, x)
        return take

    def __lt__(self, x):
        return self.below(float(x))

    def __mul__(self, s):
        return _Scaled(self, float(s))

    __rmul__ = __mul__


class _Scaled:
    def __init__(self, u, s):
        self.u, self.s = u, s

    def __lt__(self, x):            # u * s < x  <=>  u < x / s
        return self.u.below(float(x) / self.s)


def enumerate_outcomes(run):
    """Exact distribution of run(draw) over all uniform branches."""
    dist = defaultdict(float)
    stack = [[]]
    while stack:
        script = stack.pop()
        drv = _Driver(script)
        out = run(drv.draw)
        if drv.prob > 0:
            dist[out] += drv.prob
        for pos, p_true in drv.points:
            if p_true > 0:
                stack.append(script + [False] * (pos - len(script)) + [True])
    return dist


# a tiny autoregressive "target" and "draft": logits depend only on the token path
def _tables(V, seed, spread=1.5, noise=0.8):
    cache = {}

    def rows(path):
        key = tuple(path)
        if key not in cache:
            h = abs(hash((seed,) + key)) % (2 ** 32)
            r = np.random.default_rng(h)
            t = r.standard_normal(V) * spread
            d = t + r.standard_normal(V) * noise
            cache[key] = (t, d)
        return cache[key]
    return rows


def _tree_outcomes(parents, V, rows, tau=1.0, want=2, without_replacement=False):
    """Exact joint law of the first `want` emitted tokens (None = stopped).
    Siblings are i.i.d. draws from the parent's draft distribution, or, with
    without_replacement, drawn one after the other from it without
    replacement (and verified by the walk's without-replacement rule)."""
    T = len(parents)
    kids = oacc.tree_children(parents)
    depth_path = {0: ()}
    for c in range(1, T):
        depth_path[c] = None
    total = defaultdict(float)

    # enumerate child tokens: each child ~ parent's draft distribution, i.i.d.
    def assign(c, tokens, weight):
        if c == T:
            paths = {0: ()}
            for n in range(1, T):
                paths[n] = paths[int(parents[n])] + (int(tokens[n]),)
            tgt = np.stack([rows(paths[n])[0] for n in range(T)])
            drf = np.stack([rows(paths[n])[1] for n in range(T)])

            def run(draw):
                path, final, _, _ = oacc.walk_sampled(
                    lambda n: tgt[n], lambda n: drf[n], parents, tokens, tau,
                    lambda n, s: draw(0, n, s), without_replacement)
                emitted = [int(tokens[c]) for c in path] + [int(final)]
                emitted += [None] * want
                return tuple(emitted[:want])
            for out, pr in enumerate_outcomes(run).items():
                total[out] += weight * pr
            return
        par = int(parents[c])
        ppath = ()
        n = par
        toks = []
        while n > 0:
            toks.append(int(tokens[n]))
            n = int(parents[n])
        ppath = tuple(reversed(toks))
        pd = sp_softmax(rows(ppath)[1] / tau)
        if without_replacement:   # earlier siblings' tokens are gone, the rest renormalised
            used = [int(tokens[o]) for o in range(1, c) if int(parents[o]) == par]
            pd = pd.copy()
            pd[used] = 0.0
            pd = pd / pd.sum()
        for t in range(V):
            if pd[t] == 0:
                continue
            tokens[c] = t
            assign(c + 1, tokens, weight * pd[t])
        tokens[c] = 0

    assign(1, np.zeros(T, dtype=np.int64), 1.0)
    return total


@pytest.mark.parametrize("parents,V,seed", [
    ([-1, 0, 0, 0], 4, 1),          # three i.i.d. siblings at the root
    ([-1, 0, 0, 1, 1], 3, 2),       # depth 2, two siblings per level
    ([-1, 0, 1, 0], 5, 3),          # chain + sibling
])
def test_lossless_exact_enumeration(parents, V, seed):
    rows = _tables(V, seed)
    dist = _tree_outcomes(np.asarray(parents), V, rows)
    assert abs(sum(dist.values()) - 1.0) < 1e-12
    q_root = sp_softmax(rows(())[0])
    first = np.zeros(V)
    for (a, _), pr in dist.items():
        first[a] += pr
    np.testing.assert_allclose(first, q_root, rtol=0, atol=1e-12)
    # second token, given the first was emitted as an accepted draft
    for a in range(V):
        cont = np.zeros(V)
        for (x, y), pr in dist.items():
            if x == a and y is not None:
                cont[y] += pr
        if cont.sum() > 1e-9:
            np.testing.assert_allclose(cont / cont.sum(), sp_softmax(rows((a,))[0]),
                                       rtol=0, atol=1e-10)


def test_lossless_exact_with_temperature():
    rows = _tables(4, 11)
    tau = 0.7
    dist = _tree_outcomes(np.asarray([-1, 0, 0]), 4, rows, tau=tau, want=1)
    first = np.zeros(4)
    for (a,), pr in dist.items():
        first[a] += pr
    np.testing.assert_allclose(first, sp_softmax(rows(())[0] / tau), atol=1e-12)


def _chain_case(N, B, rng):
    """Chain of N draft nodes with q = (0.3, 0.7), p = (0.5, 0.5) at every node."""
    V = 2
    T = N + 1
    parents = np.tile(np.arange(-1, N, dtype=np.int32), (B, 1))
    tgt = np.tile(np.log(np.array([0.3, 0.7])), (B, T, 1))
    drf = np.tile(np.log(np.array([0.5, 0.5])), (B, T, 1))
    tokens = rng.integers(0, V, size=(B, T)).astype(np.int32)      # drafts ~ p
    return tgt, drf, parents, tokens


def test_chain_closed_form_exact():
    N, alpha = 5, 0.8
    parents = np.arange(-1, N)
    # enumerate draft tokens (uniform over {0,1}) and decisions
    exp_emitted = 0.0
    q = np.log(np.array([0.3, 0.7]))
    p = np.log(np.array([0.5, 0.5]))
    for mask in range(2 ** N):
        tokens = np.array([0] + [(mask >> i) & 1 for i in range(N)])

        def run(draw):
            path, final, _, _ = oacc.walk_sampled(lambda n: q, lambda n: p, parents, tokens, 1.0,
                                                  lambda n, s: draw(0, n, s))
            return len(path) + 1
        for n_emit, pr in enumerate_outcomes(run).items():
            exp_emitted += pr * n_emit / 2 ** N
    assert abs(exp_emitted - (1 - alpha ** (N + 1)) / (1 - alpha)) < 1e-12


def test_chain_closed_form_monte_carlo():
    N, alpha, B = 5, 0.8, 3000
    rng = np.random.default_rng(42)
    tgt, drf, parents, tokens = _chain_case(N, B, rng)
    res = oacc.spec_accept(tgt, drf, parents, tokens, 1.0, seed=0x5EED, offset=3)
    emitted = res["accept_len"] + 1
    mean = (1 - alpha ** (N + 1)) / (1 - alpha)
    se = emitted.std(ddof=1) / np.sqrt(B)
    assert abs(emitted.mean() - mean) < 4.5 * se


def test_chi_square_over_philox_offsets():
    """Root with three i.i.d. siblings; first emitted token vs q_root."""
    V, B = 6, 12000
    rng = np.random.default_rng(3)
    t_row = rng.standard_normal(V) * 1.5
    d_row = t_row + rng.standard_normal(V) * 0.9
    q = sp_softmax(t_row)
    p = sp_softmax(d_row)
    parents = np.tile(np.array([-1, 0, 0, 0], dtype=np.int32), (B, 1))
    tokens = np.zeros((B, 4), dtype=np.int32)
    tokens[:, 1:] = rng.choice(V, size=(B, 3), p=p)
    tgt = np.tile(t_row, (B, 4, 1))
    drf = np.tile(d_row, (B, 4, 1))
    res = oacc.spec_accept(tgt, drf, parents, tokens, 1.0, seed=0x5EED0004, offset=0)
    counts = np.bincount(res["out_tokens"][:, 0], minlength=V)
    stat = ((counts - B * q) ** 2 / (B * q)).sum()
    assert stat < chi2_dist.ppf(0.999, V - 1), (stat, counts, B * q)


def test_greedy_equals_greedy_decoding():
    V = 7
    rows = _tables(V, 99)

    def greedy_decode(k):
        seq = []
        for _ in range(k):
            seq.append(int(np.argmax(rows(tuple(seq))[0])))
        return seq

    g = greedy_decode(5)
    rng = np.random.default_rng(0)
    for trial in range(40):
        # a random tree that contains the greedy path to a random depth,
        # with distractor siblings before and after it
        d = int(rng.integers(0, 5))
        parents, tokens = [-1], [0]
        cur = 0
        for lvl in range(d + 1):
            others = [t for t in range(V) if t != g[lvl]]
            rng.shuffle(others)
            nd = int(rng.integers(0, 3))
            opts = others[:nd]
            on_path = lvl < d
            if on_path:
                pos = int(rng.integers(0, nd + 1))
                opts = opts[:pos] + [g[lvl]] + opts[pos:]
            ids = []
            for t in opts:
                parents.append(cur)
                tokens.append(t)
                ids.append(len(parents) - 1)
            if on_path:
                cur = ids[opts.index(g[lvl])]
        T = len(parents)
        paths = {0: ()}
        for n in range(1, T):
            paths[n] = paths[parents[n]] + (tokens[n],)
        tgt = np.stack([rows(paths[n])[0] for n in range(T)])[None]
        res = oacc.spec_accept(tgt, None, np.array([parents]), np.array([tokens]), 0.0, 0, 0)
        n_acc = int(res["accept_len"][0])
        assert n_acc == d
        assert list(res["out_tokens"][0, :n_acc + 1]) == g[:n_acc + 1]


def test_greedy_tie_break_lowest_id():
    tgt = np.zeros((1, 2, 5))
    tgt[0, 0, [1, 3]] = 2.0
    res = oacc.spec_accept(tgt, None, np.array([[-1, 0]]), np.array([[0, 3]]), 0.0, 0, 0)
    assert res["accept_len"][0] == 0 and res["out_tokens"][0, 0] == 1


def test_identical_distributions_accept_first_child():
    rng = np.random.default_rng(1)
    T, V = 7, 9
    parents = np.array([[-1, 0, 0, 1, 1, 3, 3]])
    rows = rng.standard_normal((1, T, V))
    tokens = rng.integers(0, V, size=(1, T)).astype(np.int32)
    for off in range(20):
        res = oacc.spec_accept(rows, rows, parents, tokens, 1.0, seed=5, offset=off)
        assert list(res["accepted_nodes"][0, :3]) == [1, 3, 5]
        assert res["accept_len"][0] == 3


def test_disjoint_supports_reject_every_child():
    V = 6
    t_row = np.array([0.0, 0.5, 1.0, -np.inf, -np.inf, -np.inf])
    d_row = np.array([-np.inf, -np.inf, -np.inf, 0.0, 0.2, 0.1])
    parents = np.array([[-1, 0, 0, 0]])
    tokens = np.array([[0, 3, 4, 5]])
    tgt = np.tile(t_row, (1, 4, 1))
    drf = np.tile(d_row, (1, 4, 1))
    finals = []
    for off in range(200):
        res = oacc.spec_accept(tgt, drf, parents, tokens, 1.0, seed=9, offset=off)
        assert res["accept_len"][0] == 0
        finals.append(res["out_tokens"][0, 0])
    assert set(finals) <= {0, 1, 2} and len(set(finals)) == 3


def test_edge_conventions():
    # p(t) == 0 with q_res(t) > 0: accepted and flagged (lesson's accept(): p <= 0 -> True)
    tgt = np.log(np.array([[[0.5, 0.5, 1e-300], [0.1, 0.9, 1e-300]]]))
    drf = np.array([[[0.0, 0.0, -np.inf], [0.0, 0.0, 0.0]]])
    res = oacc.spec_accept(tgt, drf, np.array([[-1, 0]]), np.array([[0, 2]]), 1.0, 1, 0)
    assert res["accept_len"][0] == 1 and res["flags"][0] & oacc.FLAG_P_ZERO
    # zero residual mass: q == p, the child must be rejected... impossible (ratio 1);
    # use q == p and a token of zero target mass so the test rejects, then
    # the residual max(0, q - p) is zero and q is used again (lesson's residual()).
    row = np.log(np.array([0.5, 0.5, 1e-300]))
    row[2] = -np.inf
    tgt = np.stack([row, row, row])[None]
    drf = tgt.copy()
    res = oacc.spec_accept(tgt, drf, np.array([[-1, 0, 0]]), np.array([[0, 2, 1]]), 1.0, 1, 0)
    # first child has q(t)=p(t)=0 -> p==0 rule, q_res(t)=0 -> rejected; residual is 0 -> reset
    assert res["flags"][0] & oacc.FLAG_P_ZERO
    assert res["flags"][0] & oacc.FLAG_DEGENERATE_RESIDUAL
    assert res["accept_len"][0] == 1 and res["accepted_nodes"][0, 0] == 2


def test_invalid_inputs_are_flagged_and_poisoned():
    rng = np.random.default_rng(0)
    B, T, V = 4, 4, 8
    tgt = rng.standard_normal((B, T, V))
    drf = rng.standard_normal((B, T, V))
    parents = np.tile(np.array([-1, 0, 0, 1]), (B, 1))
    tokens = np.tile(np.array([0, 1, 2, 3]), (B, 1))
    parents[1, 3] = 3                       # self parent
    tokens[2, 2] = V                        # out of range
    tgt[3, 1, 4] = np.nan                   # non-finite row
    res = oacc.spec_accept(tgt, drf, parents, tokens, 1.0, 2, 0)
    assert res["flags"][0] == 0 and res["accept_len"][0] >= 0
    assert res["flags"][1] == oacc.FLAG_BAD_TREE
    assert res["flags"][2] == oacc.FLAG_BAD_TOKEN
    assert res["flags"][3] == oacc.FLAG_NONFINITE
    for b in (1, 2, 3):
        assert res["accept_len"][b] == -1
        assert (res["accepted_nodes"][b] == -1).all() and (res["out_tokens"][b] == -1).all()
    # an all -inf row is unusable too; a leaf's draft row is never read
    tgt2 = tgt[:1].copy()
    drf2 = drf[:1].copy()
    drf2[0, 3, :] = np.nan                  # node 3 is a leaf: ignored
    assert oacc.spec_accept(tgt2, drf2, parents[:1], tokens[:1], 1.0, 2, 0)["flags"][0] == 0
    tgt2[0, 2, :] = -np.inf
    assert oacc.spec_accept(tgt2, drf2, parents[:1], tokens[:1], 1.0, 2, 0)["flags"][0] == \
        oacc.FLAG_NONFINITE


def test_inv_cdf_definition():
    w = np.array([0.0, 0.25, 0.0, 0.5, 0.25])
    assert oacc.inv_cdf(w, 0.0)[0] == 1
    assert oacc.inv_cdf(w, 0.2499)[0] == 1
    assert oacc.inv_cdf(w, 0.25)[0] == 3          # strict: running sum must exceed u*S
    assert oacc.inv_cdf(w, 0.75)[0] == 4
    assert oacc.inv_cdf(w * 3.0, 0.5)[0] == 3     # unnormalised weights


# ---------------------------------------------------------------------------
# near-tie flags (several correct results: a decision within 1e-6 of its
# threshold is flagged, lesson page build step 5 / EAGLE notes page core
# mechanism §5 for the rule it guards).  The margins are relative to the
# weights' total for an inverse-CDF sample and absolute for the ratio test
# (r and the ratio are both on the [0, 1) scale there); both are strict.
# ---------------------------------------------------------------------------
def test_inv_cdf_near_tie_flags():
    w = np.array([0.25, 0.25, 0.5])
    cases = [                       # (u, token, near): boundary between tokens 0 and 1 at 0.25
        (0.25 - 2e-6, 0, False),
        (0.25 - 0.5e-6, 0, True),
        (0.25, 1, True),            # exactly on it: strict > picks token 1, margin 0
        (0.25 + 0.5e-6, 1, True),
        (0.25 + 2e-6, 1, False),
        (0.5 + 0.5e-6, 2, True),    # boundary between tokens 1 and 2: lower side of token 2
        (0.5 - 0.5e-6, 1, True),    # ... upper side of token 1
        (0.375, 1, False),          # the middle of token 1
    ]
    for scale in (1.0, 3.0, 1e3, 1e-3):     # relative to the total, not absolute
        for u, tok, near in cases:
            assert oacc.inv_cdf(w * scale, u) == (tok, near), (scale, u)
    # strict: with a total of exactly 1 and the lower boundary 0, a margin of
    # exactly 1e-6 is not a near tie, anything below it is
    w2 = np.array([0.5, 0.5])
    assert oacc.inv_cdf(w2, 1e-6) == (0, False)
    assert oacc.inv_cdf(w2, np.nextafter(1e-6, 0.0)) == (0, True)
    # a token whose weight is below 2e-6 of the total is always a near tie
    # (both of its boundaries lie within 1e-6 of any draw that lands on it)
    w3 = np.array([0.5, 1.5e-6, 0.5])
    w3 = w3 / w3.sum()
    for f in (0.1, 0.5, 0.9):
        u = (w3[0] + f * w3[1])
        assert oacc.inv_cdf(w3, u) == (1, True)
    w4 = np.array([0.5, 3e-6, 0.5])
    w4 = w4 / w4.sum()
    assert oacc.inv_cdf(w4, w4[0] + 0.5 * w4[1]) == (1, False)


def _scripted(draws):
    def draw(node, slot):
        return draws[(node, slot)]
    return draw


def test_ratio_test_near_tie_flags():
    """Root with one child of token 0; q = (0.3, 0.7), p = (0.5, 0.5): the
    ratio is 0.6; the child is a leaf, so its bonus sample follows."""
    q = np.log([0.3, 0.7])
    p = np.log([0.5, 0.5])
    parents = np.array([-1, 0])
    tokens = np.array([0, 0])
    for r, acc, near in [(0.6 - 2e-6, True, 0), (0.6 - 0.5e-6, True, 1), (0.6 + 0.5e-6, False, 1),
                         (0.6 + 2e-6, False, 0)]:
        where = []
        path, final, fl, nt = oacc.walk_sampled(lambda n: q, lambda n: p, parents, tokens, 1.0,
                                                _scripted({(0, 0): r, (0, philox.SAMPLE_SLOT): 0.5,
                                                           (1, philox.SAMPLE_SLOT): 0.5}), where=where)
        assert (path == [1]) == acc and nt == near and fl == 0, r
        assert where == ([(0, 0)] if near else [])
        if not acc:
            assert final == 1       # the residual max(0, q - p) = (0, 0.2) puts all its mass on token 1
    # absolute margin: a ratio of 1e-3 is flagged for r within 1e-6 of it
    q_small = np.log([1e-3 * 0.5, 1 - 1e-3 * 0.5])
    for r, near in [(1e-3 + 0.5e-6, 1), (1e-3 - 0.5e-6, 1), (1e-3 + 2e-6, 0)]:
        _, _, _, nt = oacc.walk_sampled(lambda n: q_small, lambda n: p, parents, tokens, 1.0,
                                        _scripted({(0, 0): r, (0, philox.SAMPLE_SLOT): 0.7,
                                                   (1, philox.SAMPLE_SLOT): 0.7}))
        assert nt == near, r
    # strict: q(t) = 0 makes the ratio 0; r = 1e-6 exactly is not a near tie
    q_zero = np.array([-np.inf, 0.0])
    for r, near in [(1e-6, 0), (np.nextafter(1e-6, 0.0), 1)]:
        path, _, _, nt = oacc.walk_sampled(lambda n: q_zero, lambda n: p, parents, tokens, 1.0,
                                           _scripted({(0, 0): r, (0, philox.SAMPLE_SLOT): 0.5}))
        assert path == [] and nt == near, r


def test_near_tie_is_measured_against_the_current_residual():
    """Two siblings, tokens 2 then 1; q = (0.4, 0.35, 0.25), p = (0.2, 0.3, 0.5).
    The first is rejected (ratio 0.5, r = 0.9); the residual is then
    norm(max(0, q - p)) = (0.8, 0.2, 0), so the second sibling's ratio is
    0.2 / 0.3 = 2/3, not q(1)/p(1) = 7/6."""
    q = np.log([0.4, 0.35, 0.25])
    p = np.log([0.2, 0.3, 0.5])
    parents = np.array([-1, 0, 0])
    tokens = np.array([0, 2, 1])
    for r, acc, near in [(2 / 3 - 0.5e-6, True, 1), (2 / 3 + 0.5e-6, False, 1), (2 / 3 + 2e-6, False, 0),
                         (7 / 6 - 1.0, True, 0)]:
        where = []
        path, _, _, nt = oacc.walk_sampled(lambda n: q, lambda n: p, parents, tokens, 1.0,
                                           _scripted({(0, 0): 0.9, (0, 1): r, (0, philox.SAMPLE_SLOT): 0.31,
                                                      (2, philox.SAMPLE_SLOT): 0.31}), where=where)
        assert (path == [2]) == acc and nt == near, r
        assert where == ([(0, 1)] if near else [])


def test_first_near_tie_is_located_on_the_walk():
    """Chain root -> 1 -> 2 (tokens 0, 0), q = (0.3, 0.7), p = (0.5, 0.5):
    node 1 is accepted far from its threshold, node 2's test is a near tie
    (rejected), then the residual sample; spec_accept reports depth 1, slot 0.
    A near tie on a terminal sample reports slot -1."""
    V = 2
    tgt = np.tile(np.log([0.3, 0.7]), (1, 3, 1))
    drf = np.tile(np.log([0.5, 0.5]), (1, 3, 1))
    parents = np.array([[-1, 0, 1]])
    tokens = np.array([[0, 0, 0]])
    draws = {(0, 0, 0): 0.1, (0, 1, 0): 0.6 + 0.5e-6, (0, 1, philox.SAMPLE_SLOT): 0.5}
    res = oacc.spec_accept(tgt, drf, parents, tokens, 1.0, 0, 0, draw=lambda b, n, s: draws[(b, n, s)])
    assert res["accept_len"][0] == 1 and res["out_tokens"][0, :2].tolist() == [0, 1]
    assert res["near_ties"][0] == 1
    assert (res["first_near_depth"][0], res["first_near_slot"][0]) == (1, 0)
    # both tests accepted far away; the bonus sample at leaf 2 lands 0.5e-6
    # above the boundary at 0.3 between tokens 0 and 1
    draws = {(0, 0, 0): 0.1, (0, 1, 0): 0.2, (0, 2, philox.SAMPLE_SLOT): 0.3 + 0.5e-6}
    res = oacc.spec_accept(tgt, drf, parents, tokens, 1.0, 0, 0, draw=lambda b, n, s: draws[(b, n, s)])
    assert res["accept_len"][0] == 2 and res["out_tokens"][0].tolist() == [0, 0, 1]
    assert (res["first_near_depth"][0], res["first_near_slot"][0]) == (2, -1)
    # no near tie anywhere
    draws = {(0, 0, 0): 0.1, (0, 1, 0): 0.2, (0, 2, philox.SAMPLE_SLOT): 0.5}
    res = oacc.spec_accept(tgt, drf, parents, tokens, 1.0, 0, 0, draw=lambda b, n, s: draws[(b, n, s)])
    assert res["near_ties"][0] == 0 and (res["first_near_depth"][0], res["first_near_slot"][0]) == (-1, -1)
    assert V == tgt.shape[-1]


def _expected_accept_len(q_rows, p_rows, parents, tokens):
    """Probability flow through a tree whose tokens are fixed: the i-th child
    of n is accepted with probability a_i * prod_{j<i} (1 - a_j), where
    a_i = min(1, q_i(t_i) / p(t_i)) and q_i is the residual left after the
    i-1 rejections before it (the rule of the EAGLE notes page, core
    mechanism §5).  Returns E[accepted nodes]."""
    T = len(parents)
    kids = [[c for c in range(1, T) if parents[c] == n] for n in range(T)]

    def flow(n):
        q, p = q_rows[n], p_rows[n]
        res, reach, total = q.copy(), 1.0, 0.0
        for c in kids[n]:
            t = tokens[c]
            a = min(1.0, res[t] / p[t])
            total += reach * a * (1.0 + flow(c))
            reach *= 1.0 - a
            res = np.maximum(0.0, res - p)
            res = res / res.sum()
        return total
    return flow(0)


def test_expected_accept_length_of_a_fixed_tree():
    """Pin P8: the walk's mean accepted length over Philox uniforms equals the
    probability flow of a fixed three-level tree with distinct rows per node."""
    # chosen so that a walk without the residual update (E = 2.29) or with a
    # residual taken afresh from q at every rejection (E = 2.22) is far off
    rng = np.random.default_rng(13)
    V = 6
    parents = np.array([-1, 0, 0, 0, 0, 1, 1, 5, 2])
    tokens = np.array([0, 1, 3, 2, 0, 2, 0, 5, 4])
    T = len(parents)
    tgt = rng.standard_normal((T, V)) * 1.5
    drf = tgt + rng.standard_normal((T, V)) * 1.5
    q_rows = [sp_softmax(r) for r in tgt]
    p_rows = [sp_softmax(r) for r in drf]
    want = _expected_accept_len(q_rows, p_rows, parents, tokens)
    B, K = 64, 60
    lens = []
    for off in range(K):
        res = oacc.spec_accept(np.tile(tgt, (B, 1, 1)), np.tile(drf, (B, 1, 1)), np.tile(parents, (B, 1)),
                               np.tile(tokens, (B, 1)), 1.0, 77, off)
        lens.append(res["accept_len"])
    lens = np.concatenate(lens).astype(np.float64)
    se = lens.std(ddof=1) / np.sqrt(len(lens))
    assert abs(want - 1.9778) < 1e-3
    assert abs(lens.mean() - want) < 4.5 * se, (lens.mean(), want, se)


def test_residual_closed_form_matches_iteration():
    """The GPU's division-free form of the cumulative residual:
    after i rejections q_res = max(0, q - C_i p) / s_i with C_1 = 0, s_1 = 1,
    C_{i+1} = C_i + s_i, s_{i+1} = sum max(0, q - C_{i+1} p)."""
    rng = np.random.default_rng(12)
    for _ in range(200):
        V = int(rng.integers(2, 40))
        q = sp_softmax(rng.standard_normal(V) * 2)
        p = sp_softmax(rng.standard_normal(V) * 2)
        q_res = q.copy()
        C, s = 0.0, 1.0
        for _ in range(6):
            np.testing.assert_allclose(q_res, np.maximum(0.0, q - C * p) / s, atol=1e-12)
            nxt = np.maximum(0.0, q_res - p)
            z = nxt.sum()
            if z == 0:
                break
            q_res = nxt / z
            C = C + s
            s = np.maximum(0.0, q - C * p).sum()


def _random_tree(rng, T):
    return np.asarray([-1] + [int(rng.integers(0, i)) for i in range(1, T)], dtype=np.int32)


@pytest.mark.parametrize("temperature", [1.0, 0.0])
def test_padding_rows_give_the_truncated_trees_result(temperature):
    """Trees of different sizes in one batch: padding a tree with rows of
    token -1 (NaN logits, never read) gives, sequence by sequence, exactly
    the result of the tree without them (run with no padding at all and the
    same uniforms)."""
    rng = np.random.default_rng(41 + int(temperature))
    B, T, V = 6, 12, 40
    sizes = [12, 7, 3, 1, 2, 11]
    par = np.stack([_random_tree(rng, T) for _ in range(B)])
    tok = rng.integers(0, V, size=(B, T)).astype(np.int32)
    tgt = rng.standard_normal((B, T, V)) * 2
    drf = tgt + rng.standard_normal((B, T, V)) * 0.8
    par_p, tok_p, tgt_p, drf_p = par.copy(), tok.copy(), tgt.copy(), drf.copy()
    for b, n in enumerate(sizes):
        tok_p[b, n:] = -1
        par_p[b, n:] = 0
        tgt_p[b, n:] = np.nan
        drf_p[b, n:] = np.nan
    seed, off = 0x5EED0009, 3
    padded = oacc.spec_accept(tgt_p, None if temperature == 0 else drf_p, par_p, tok_p, temperature, seed, off)
    for b, n in enumerate(sizes):
        alone = oacc.spec_accept(tgt[b:b + 1, :n], None if temperature == 0 else drf[b:b + 1, :n],
                                 par[b:b + 1, :n], tok[b:b + 1, :n], temperature, seed, off,
                                 draw=lambda _bb, node, slot, _b=b: philox.uniform(seed, off, _b, node, slot))
        assert padded["accept_len"][b] == alone["accept_len"][0]
        assert padded["flags"][b] == alone["flags"][0] and padded["near_ties"][b] == alone["near_ties"][0]
        for key in ("accepted_nodes", "out_tokens"):
            assert padded[key][b, :n].tolist() == alone[key][0].tolist()
            assert (padded[key][b, n:] == -1).all()


def test_padding_must_be_a_suffix():
    rng = np.random.default_rng(43)
    T, V = 6, 20
    par = _random_tree(rng, T)[None]
    tok = np.array([[0, 3, -1, 4, -1, -1]], dtype=np.int32)   # a real row after a padding row
    tgt = rng.standard_normal((1, T, V))
    out = oacc.spec_accept(tgt, tgt, par, tok, 1.0, 1, 0)
    assert out["flags"].tolist() == [oacc.FLAG_BAD_TREE] and out["accept_len"].tolist() == [-1]


@pytest.mark.parametrize("parents,V,seed,tau", [
    ([-1, 0, 0, 0], 4, 1, 1.0),         # three siblings drawn without replacement at the root
    ([-1, 0, 0, 0, 0], 4, 4, 0.8),      # as many siblings as tokens: the last one is forced
    ([-1, 0, 0, 1, 1], 3, 2, 1.0),      # depth 2, two siblings per level
])
def test_lossless_exact_without_replacement(parents, V, seed, tau):
    """Siblings drawn without replacement and verified against the draft with
    the tried tokens removed and renormalised: the emitted tokens follow the
    target exactly (exact enumeration of tokens and uniforms)."""
    rows = _tables(V, seed)
    dist = _tree_outcomes(np.asarray(parents), V, rows, tau=tau, without_replacement=True)
    assert abs(sum(dist.values()) - 1.0) < 1e-12
    first = np.zeros(V)
    for (a, _), pr in dist.items():
        first[a] += pr
    np.testing.assert_allclose(first, sp_softmax(rows(())[0] / tau), rtol=0, atol=1e-12)
    for a in range(V):
        cont = np.zeros(V)
        for (x, y), pr in dist.items():
            if x == a and y is not None:
                cont[y] += pr
        if cont.sum() > 1e-9:
            np.testing.assert_allclose(cont / cont.sum(), sp_softmax(rows((a,))[0] / tau), rtol=0, atol=1e-10)


def test_with_replacement_rule_is_not_lossless_for_distinct_siblings():
    """The plain rule applied to siblings drawn without replacement is biased
    (which is why the renormalised rule exists): the exact first-token law
    then differs from the target."""
    rows = _tables(3, 5)
    par = np.asarray([-1, 0, 0])
    T = 3
    # distinct siblings drawn without replacement, verified with the i.i.d. rule
    total = defaultdict(float)
    t_root, d_root = rows(())
    pd = sp_softmax(d_root)
    for t1 in range(3):
        for t2 in range(3):
            if t2 == t1:
                continue
            w = pd[t1] * pd[t2] / (1.0 - pd[t1])
            tokens = np.array([0, t1, t2])
            tgt = np.stack([t_root, rows((t1,))[0], rows((t2,))[0]])
            drf = np.stack([d_root, rows((t1,))[1], rows((t2,))[1]])

            def run(draw, tokens=tokens, tgt=tgt, drf=drf):
                path, final, _, _ = oacc.walk_sampled(lambda n: tgt[n], lambda n: drf[n], par, tokens, 1.0,
                                                      lambda n, s: draw(0, n, s))
                return int(tokens[path[0]]) if path else int(final)
            for out, pr in enumerate_outcomes(run).items():
                total[out] += w * pr
    first = np.array([total[a] for a in range(3)])
    assert np.abs(first - sp_softmax(t_root)).max() > 1e-3
