"""One expansion step of a dynamic draft tree (EAGLE-2) — oracle side (test
infrastructure only).

What the step does (EAGLE notes page, the EAGLE-2 section: the draft model's
confidence tracks the acceptance rate, so the tree grows where the
cumulative confidence of a path is high; the tree-drafting section: greedy
drafting takes each node's top-k children by probability):

  frontier node f of sequence b carries the log-probability s_f of the path
  that reaches it (the root: 0) and the draft model's next-token logits x_f;
  with p_f = softmax(x_f / tau):
    candidates: for every active frontier node (s_f > -inf; NaN counts as
                inactive) its k most probable tokens (largest logit first,
                ties to the lower id)
    value of a candidate (f, t): s_f + log p_f(t)
    kept: the M candidates of largest value, ranked by value, ties to the
          lower frontier index, then the lower token id
  the kept candidates become the next frontier (their values its s), and
  the tree gains them as children of their frontier nodes.

Readings where the pages are silent (each listed in the design notes):
  * log p_f(t) = (x_t - max x)/tau - log sum_v exp((x_v - max x)/tau);
  * fewer than M candidates with a finite value: the rest of the output is
    padded with parent -1, token -1, value -inf;
  * a frontier row holding NaN or +inf is unusable: its node is skipped and the
    sequence is flagged (NONFINITE);
  * near ties: a ranking decision between two candidates whose values differ by
    less than 1e-6 (absolute, the values are log-probabilities) is counted;
    parity is defined up to such decisions.

Plain numpy in float64; the ranking is a full sort of all candidates.
"""
import numpy as np

FLAG_NONFINITE = 4
NEAR = 1e-6


def row_logprobs(x, tau):
    """log softmax(x / tau) in float64, or None for an unusable row."""
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any() or np.isposinf(x).any() or np.isneginf(x).all():
        return None
    m = x.max()
    z = np.exp((x - m) / tau).sum()
    return (x - m) / tau - np.log(z)


def top_k_tokens(x, k):
    """The k largest logits' ids, largest first, ties to the lower id."""
    x = np.asarray(x, dtype=np.float64)
    order = np.lexsort((np.arange(len(x)), -x))     # by -x, then by id
    return order[:k]


def expand(logits, scores, tau, k, M):
    """logits [B, F, V], scores [B, F] (float, -inf = inactive) ->
    dict(parent [B, M] int32, token [B, M] int32, value [B, M] float64,
         flags [B] uint32, near_ties [B] int32)."""
    logits = np.asarray(logits)
    B, F, V = logits.shape
    parent = np.full((B, M), -1, dtype=np.int32)
    token = np.full((B, M), -1, dtype=np.int32)
    value = np.full((B, M), -np.inf)
    flags = np.zeros(B, dtype=np.uint32)
    near = np.zeros(B, dtype=np.int32)
    for b in range(B):
        cands = []
        for f in range(F):
            s = float(scores[b][f])
            if not s > -np.inf:                     # -inf or NaN: an inactive node
                continue
            lp = row_logprobs(logits[b, f], tau)
            if lp is None:
                flags[b] |= FLAG_NONFINITE
                continue
            for t in top_k_tokens(logits[b, f], min(k, V)):
                cands.append((s + lp[t], f, int(t)))
        cands = [c for c in cands if c[0] > -np.inf]
        cands.sort(key=lambda c: (-c[0], c[1], c[2]))
        for i, (val, f, t) in enumerate(cands[:M]):
            parent[b, i], token[b, i], value[b, i] = f, t, val
        # ranking decisions that depend on less than NEAR: neighbours in the
        # order up to and including the boundary between kept and dropped
        # (two tokens of one row with equal logits tie exactly, and the token
        # ids decide; they are not counted)
        for i in range(min(len(cands), M + 1) - 1):
            (v0, f0, t0), (v1, f1, t1) = cands[i], cands[i + 1]
            same = f0 == f1 and logits[b, f0, t0] == logits[b, f1, t1]
            if v0 - v1 < NEAR and not same:
                near[b] += 1
    return dict(parent=parent, token=token, value=value, flags=flags, near_ties=near)


def rerank(parent, token, value, root_tokens, N):
    """Final draft tree from D expansion steps (EAGLE notes page, the EAGLE-2
    section: nodes are kept by the cumulative confidence of their paths).

    parent/token/value [D, B, M]: step d's kept candidates (step 0 expands the
    root, so its parents are 0; step d > 0 indexes step d-1's kept list;
    parent -1 = no candidate).  The N nodes of largest value are kept, ties to
    the earlier step, then the better rank in the step; a node's value never
    exceeds its parent's, so the kept set contains every kept node's parent.
    Output rows: 0 = the root (parent -1, token root_tokens[b]), then the
    kept nodes in (step, rank) order, so parents precede children.
    Returns dict(parents [B, N+1], tokens [B, N+1], rows [B]); rows past
    `rows` are padding rows, parent 0 and token -1 (the padding of a tree
    that shares a batch with larger ones: a valid parent, token -1)."""
    parent = np.asarray(parent)
    value = np.asarray(value, dtype=np.float64)
    D, B, M = parent.shape
    parents = np.zeros((B, N + 1), dtype=np.int32)
    parents[:, 0] = -1
    tokens = np.full((B, N + 1), -1, dtype=np.int32)
    rows = np.zeros(B, dtype=np.int32)
    for b in range(B):
        cands = [(value[d, b, r], d, r) for d in range(D) for r in range(M) if parent[d, b, r] >= 0]
        cands.sort(key=lambda c: (-c[0], c[1], c[2]))
        kept = sorted((d, r) for _, d, r in cands[:N])
        index = {}
        parents[b, 0], tokens[b, 0] = -1, int(root_tokens[b])
        for i, (d, r) in enumerate(kept, start=1):
            index[(d, r)] = i
            parents[b, i] = 0 if d == 0 else index[(d - 1, int(parent[d, b, r]))]
            tokens[b, i] = int(token[d, b, r])
        rows[b] = 1 + len(kept)
    return dict(parents=parents, tokens=tokens, rows=rows)
