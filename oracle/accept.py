"""Multi-round speculative sampling over a draft tree — oracle side
(test infrastructure only).

Notation: q = target distribution, p = draft distribution (the lesson page's
Leviathan section uses this pair; the EAGLE notes page writes p and p-hat).

What the walk does (EAGLE notes page, core mechanism §5 and the "multi-round
speculative sampling" term; lesson page, "Concept" and build steps 1-3):

  start at the root; at the current node n with children c_1 < c_2 < ... :
    q_res = softmax(target[n] / tau),  p_n = softmax(draft[n] / tau)
    for each child c_i in ascending node index:
        draw r; accept c_i if r < q_res(t) / p_n(t), t = tokens[c_i]
          -> emit t, move to c_i, start over there
        otherwise q_res <- norm(max(0, q_res - p_n)) and try the next child
    all children rejected: emit a sample of q_res and stop
  a node without children: emit a sample of q_n (the bonus token) and stop

Greedy mode (tau == 0, EAGLE's lossless greedy verification): a_n = argmax of
target[n] (lowest id on ties); accept the first child whose token is a_n,
otherwise emit a_n and stop; at a leaf emit a_n.

Readings where the pages are silent or disagree (each listed in the design
notes):
  * every sibling is tested against the same parent draft row p_n;
  * the residual update is cumulative over the rejected siblings;
  * p_n(t) == 0: accept iff q_res(t) > 0 (the lesson's accept() returns True
    for p <= 0; the two differ only when q_res(t) == 0 too) — flagged;
  * residual mass 0: fall back to q_n (the lesson's residual() returns q) —
    flagged;
  * comparison is strict, r on the 24-bit grid of the Philox uniform;
  * temperature divides both target and draft logits;
  * samples are drawn by inverse CDF over ascending token ids: the smallest v
    whose running sum exceeds u * (total sum).

Outputs per sequence: accept_len, accepted_nodes (root path, -1 padded),
out_tokens (tokens of the accepted nodes followed by the final token, -1
padded), flags, near_ties (decisions on the walk whose margin is below 1e-6:
|r - q_res(t)/p_n(t)| for a test, |running sum - u * total| / total for a
sample).  A sequence with an invalid tree, an out-of-range token or an
unusable logits row (NaN, +inf, or all -inf) is flagged and its integer
outputs are all -1.

Trees of different sizes in one batch (a serving batch) are padded to the
same row count: rows whose token is -1 are padding.  They must form a suffix
of the rows (else the tree is invalid), still need a valid parent, are never
children of anything and their logits rows are never read; the result is the
one for the tree without them.
"""
import numpy as np

from . import philox

FLAG_BAD_TREE = 1
FLAG_BAD_TOKEN = 2
FLAG_NONFINITE = 4
FLAG_P_ZERO = 8
FLAG_DEGENERATE_RESIDUAL = 16
NEAR_TIE = 1e-6


def _is_number(x) -> bool:
    return isinstance(x, (float, int, np.floating))


def real_rows(tokens, T):
    """Rows of the tree proper: those before the first padding row (token -1
    at a row >= 1).  Padding lets trees of different sizes share a batch."""
    for i in range(1, T):
        if int(tokens[i]) == -1:
            return i
    return T


def tree_children(parents, nreal=None):
    T = len(parents)
    nreal = T if nreal is None else nreal
    kids = [[] for _ in range(T)]
    for c in range(1, nreal):
        kids[int(parents[c])].append(c)
    return kids


def softmax_t(row, tau: float):
    z = np.asarray(row, dtype=np.float64) / tau
    z = z - z.max()
    w = np.exp(z)
    return w / w.sum()


def row_is_usable(row) -> bool:
    r = np.asarray(row, dtype=np.float64)
    if np.isnan(r).any() or np.isposinf(r).any():
        return False
    return bool(np.isfinite(r).any())


def inv_cdf(w, u):
    """Smallest id v with sum_{v' <= v} w[v'] > u * sum(w), ids ascending.

    Returns (v, near_tie).  If rounding leaves no such v, the last id with
    positive weight is returned.
    """
    w = np.asarray(w, dtype=np.float64)
    cum = np.cumsum(w)
    total = cum[-1]
    thr = u * total
    if _is_number(thr):
        v = int(np.searchsorted(cum, thr, side="right"))
    else:                               # symbolic uniform (exact enumeration tests)
        v = len(cum)
        for j in range(len(cum)):
            if thr < cum[j]:
                v = j
                break
    if v >= len(cum):
        return int(np.nonzero(w > 0)[0][-1]), False
    near = False
    if _is_number(thr):
        lower = cum[v - 1] if v > 0 else 0.0
        near = (cum[v] - thr) < NEAR_TIE * total or (thr - lower) < NEAR_TIE * total
    return v, near


def keep_threshold(row, tau, top_k=0, top_p=0.0):
    """Keep-threshold of a filtered distribution (a request's top-k / top-p
    sampling filters; the EAGLE notes page's tree drafting samples k children
    per node).  Returns (theta, near): the filtered distribution keeps the
    tokens whose logit is at least theta and renormalises softmax(row / tau)
    over them.

      top-k (0 < top_k < V): theta = the top_k-th largest logit, duplicates
        counted, so every token tied with it is kept; otherwise no cut.
      top-p (0 < top_p < 1), among the tokens top-k keeps: a token is kept
        iff the mass of the tokens with a strictly larger logit is below
        top_p times the kept mass; theta = the smallest kept logit.
    near: the nucleus boundary is within 1e-6 of the mass target, i.e. the
    kept mass minus top_p * Z, or top_p * Z minus the mass strictly above the
    boundary value, is below 1e-6 * Z."""
    x = np.asarray(row, dtype=np.float64)
    V = len(x)
    theta = -np.inf
    if 0 < top_k < V:
        theta = np.sort(x)[::-1][top_k - 1]
    near = False
    if 0.0 < top_p < 1.0:
        w = np.where(x >= theta, np.exp((x - x.max()) / tau), 0.0)
        order = np.argsort(-x, kind="stable")
        run = np.cumsum(w[order])
        z = run[-1]
        i = min(int(np.searchsorted(run, top_p * z, side="left")), V - 1)
        u = x[order][i]
        above, upto = w[x > u].sum(), w[x >= u].sum()
        near = bool((upto - top_p * z) < NEAR_TIE * z or (top_p * z - above) < NEAR_TIE * z)
        theta = u
    return theta, near


def walk_sampled(target_rows, draft_rows, parents, tokens, tau, draw, without_replacement=False, where=None,
                 row_near=None):
    """Sequential multi-round walk of one tree.

    target_rows(n) / draft_rows(n) return node n's logits rows (float64);
    draw(node, slot) returns the uniform for that decision.
    without_replacement: the siblings were drawn from p_n without
    replacement (the k sampled children of the EAGLE notes page, core
    mechanism), so sibling i is tested against p_n with the tokens of the
    siblings tried before it removed and the rest renormalised (all zero if
    nothing is left); the residual update uses that same distribution.
    where: if a list, every near-tie decision appends (depth, slot) to it:
    depth = accepted nodes before the decision (the node deciding sits at
    that depth of the path), slot = the sibling ordinal of a test, or -1 for
    the terminal sample.
    row_near(n) -> (target, draft): near ties of the filter boundaries of node
    n's rows (filtered distributions), counted when the walk visits n (the
    draft row's only when n has children), as slot 0 of that node: every
    decision there depends on them.
    Returns (path, final_token, flags, near_ties).
    """
    kids = tree_children(parents, real_rows(tokens, len(parents)))
    flags = 0
    near = 0
    path = []
    cur = 0
    while True:
        q = softmax_t(target_rows(cur), tau)
        if row_near is not None:
            nq, nd = row_near(cur)
            fnear = int(nq) + (int(nd) if kids[cur] else 0)
            if fnear:
                near += fnear
                if where is not None:
                    where.append((len(path), 0))
        if not kids[cur]:
            final, nt = inv_cdf(q, draw(cur, philox.SAMPLE_SLOT))
            near += int(nt)
            if nt and where is not None:
                where.append((len(path), -1))
            return path, final, flags, near
        p = softmax_t(draft_rows(cur), tau)
        q_res = q
        accepted = None
        tried = []
        for i, c in enumerate(kids[cur]):
            r = draw(cur, i)
            t = int(tokens[c])
            p_i = p
            if without_replacement and tried:
                p_i = p.copy()
                p_i[tried] = 0.0
                left = p_i.sum()
                p_i = p_i / left if left > 0.0 else np.zeros_like(p)
            if p_i[t] == 0.0:
                flags |= FLAG_P_ZERO
                ok = q_res[t] > 0.0
            else:
                ratio = q_res[t] / p_i[t]
                ok = r < ratio
                if _is_number(r) and abs(r - ratio) < NEAR_TIE:
                    near += 1
                    if where is not None:
                        where.append((len(path), i))
            if ok:
                accepted = c
                break
            tried.append(t)
            q_res = np.maximum(0.0, q_res - p_i)
            z = q_res.sum()
            if z == 0.0:
                flags |= FLAG_DEGENERATE_RESIDUAL
                q_res = q
            else:
                q_res = q_res / z
        if accepted is None:
            final, nt = inv_cdf(q_res, draw(cur, philox.SAMPLE_SLOT))
            near += int(nt)
            if nt and where is not None:
                where.append((len(path), -1))
            return path, final, flags, near
        path.append(accepted)
        cur = accepted


def walk_greedy(target_rows, parents, tokens):
    kids = tree_children(parents, real_rows(tokens, len(parents)))
    path = []
    cur = 0
    while True:
        a = int(np.argmax(np.asarray(target_rows(cur))))  # first maximum = lowest id
        nxt = next((c for c in kids[cur] if int(tokens[c]) == a), None)
        if nxt is None:
            return path, a, 0, 0
        path.append(nxt)
        cur = nxt


def validate_sequence(target, draft, parents, tokens, tau) -> int:
    """Flags that make a sequence unusable (outputs poisoned)."""
    T, V = target.shape
    if not (len(parents) == T and int(parents[0]) == -1
            and all(0 <= int(parents[i]) < i for i in range(1, T))):
        return FLAG_BAD_TREE
    nreal = real_rows(tokens, T)
    if any(int(tokens[c]) != -1 for c in range(nreal, T)):   # padding must be a suffix
        return FLAG_BAD_TREE
    flags = 0
    if any(not (0 <= int(tokens[c]) < V) for c in range(1, nreal)):
        flags |= FLAG_BAD_TOKEN
    kids = tree_children(parents, nreal)
    for n in range(nreal):                # padding rows are never read
        if not row_is_usable(target[n]):
            flags |= FLAG_NONFINITE
        if tau > 0 and kids[n] and not row_is_usable(draft[n]):
            flags |= FLAG_NONFINITE
    return flags


def spec_accept(target, draft, parents, tokens, temperature, seed, offset, draw=None, without_replacement=False,
                top_k=0, top_p=0.0):
    """Oracle for one verification step over a batch of trees.

    target, draft: [B,T,V] float64 logits (draft may be None when
    temperature == 0).  draw(b, node, slot) overrides the Philox uniforms.
    top_k, top_p (temperature > 0): every target and draft row is replaced by
    its filtered distribution (keep_threshold: logits below the threshold
    become -inf) before the walk; the children must have been drawn from the
    filtered draft rows.
    Returns a dict of numpy arrays: accept_len [B], accepted_nodes [B,T],
    out_tokens [B,T], flags [B], near_ties [B], and where the walk's first
    near-tie decision sits: first_near_depth [B] (accepted nodes before it,
    -1 if none) and first_near_slot [B] (sibling ordinal of a test, -1 for
    the terminal sample).  Up to that decision the result is fixed by the
    arithmetic; past it another rounding could take the other branch.
    """
    target = np.asarray(target, dtype=np.float64)
    B, T, V = target.shape
    tau = float(temperature)
    res = {
        "accept_len": np.full(B, -1, dtype=np.int32),
        "accepted_nodes": np.full((B, T), -1, dtype=np.int32),
        "out_tokens": np.full((B, T), -1, dtype=np.int32),
        "flags": np.zeros(B, dtype=np.uint32),
        "near_ties": np.zeros(B, dtype=np.int32),
        "first_near_depth": np.full(B, -1, dtype=np.int32),
        "first_near_slot": np.full(B, -1, dtype=np.int32),
    }
    for b in range(B):
        drf = None if draft is None else np.asarray(draft[b], dtype=np.float64)
        bad = validate_sequence(target[b], drf, parents[b], tokens[b], tau)
        if bad:
            res["flags"][b] = bad
            continue
        if tau == 0.0:
            path, final, fl, near = walk_greedy(lambda n: target[b, n], parents[b], tokens[b])
        else:
            if draw is None:
                def u(n, s, _b=b):
                    return philox.uniform(seed, offset, _b, n, s)
            else:
                def u(n, s, _b=b):
                    return draw(_b, n, s)
            where = []
            tgt_b, row_near = target[b], None
            if top_k > 0 or 0.0 < top_p < 1.0:
                tgt_b, drf, nears = tgt_b.copy(), drf.copy(), np.zeros((T, 2), dtype=bool)
                for n in range(T):
                    for r, rows in ((0, tgt_b), (1, drf)):
                        if row_is_usable(rows[n]):   # rows never read may hold anything
                            th, nears[n, r] = keep_threshold(rows[n], tau, top_k, top_p)
                            rows[n] = np.where(rows[n] < th, -np.inf, rows[n])
                row_near = lambda n, _nears=nears: (_nears[n, 0], _nears[n, 1])
            path, final, fl, near = walk_sampled(lambda n, _t=tgt_b: _t[n], lambda n, _d=drf: _d[n],
                                                 parents[b], tokens[b], tau, u, without_replacement, where,
                                                 row_near)
            if where:
                res["first_near_depth"][b], res["first_near_slot"][b] = where[0]
        res["accept_len"][b] = len(path)
        res["accepted_nodes"][b, :len(path)] = path
        res["out_tokens"][b, :len(path)] = [int(tokens[b][c]) for c in path]
        res["out_tokens"][b, len(path)] = final
        res["flags"][b] = fl
        res["near_ties"][b] = near
    return res
