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
