"""Shared helpers of the GPU parity tests: move seeded inputs to the device,
run the library through its C ABI, and compare with the oracle."""
import sys

import numpy as np

import synth
from synth import inputs as si

ATTN_TOL = {"bf16": 2e-3, "f32": 1e-5}
# every output buffer starts out holding these, so a row or an entry that a
# kernel never writes cannot pass for a result: an attention output is a
# convex combination of value rows, never 3e38; -7 is no node, token, count
# or length; flags never hold bits 8-31
ATTN_SENTINEL = np.float32(3.0e38)
INT_SENTINEL = -7
FLAGS_SENTINEL = 0x5A5A5A00


def sentinel_accept_outputs(B, T):
    import torch
    full = lambda shape, v: torch.full(shape, v, dtype=torch.int32, device="cuda")
    return {"accept_len": full((B,), INT_SENTINEL), "accepted_nodes": full((B, T), INT_SENTINEL),
            "out_tokens": full((B, T), INT_SENTINEL), "flags": full((B,), FLAGS_SENTINEL),
            "near_ties": full((B,), INT_SENTINEL)}


def host_accept(outputs):
    out = {k: v.cpu().numpy() for k, v in outputs.items()}
    out["flags"] = out["flags"].astype(np.uint32)
    assert not (out["flags"] & 0xFFFFFF00).any(), "flags not written"
    return out


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(arr, dtype=None):
    import torch
    a = np.ascontiguousarray(arr)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def row_error(got, ref):
    """Per output row: max_d |o - o_ref| / max_d |o_ref| (rows along the last axis)."""
    return np.abs(got - ref).max(axis=-1) / np.abs(ref).max(axis=-1)


def make_verifier(spec, T):
    import eagle_draft_tree_attention_amd as ev
    return ev.Verifier(spec.batch, spec.q_heads, spec.kv_heads, spec.head_dim, T, spec.vocab,
                       kv_dtype=spec.dtype, logits_dtype=spec.ldtype)


def run_attention(ver, inp, scale=None, parents=None, kv_indptr=None, prefix_lens=None):
    import torch
    spec = inp.spec
    D = spec.head_dim
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    par = inp.parents if parents is None else parents
    ind = inp.kv_indptr if kv_indptr is None else kv_indptr
    lens = inp.prefix_lens if prefix_lens is None else prefix_lens
    B, T = inp.q.shape[:2]
    out = torch.full((B, T, spec.q_heads, spec.head_dim), float(ATTN_SENTINEL), dtype=torch.float32, device="cuda")
    flags = torch.full((B,), FLAGS_SENTINEL, dtype=torch.int32, device="cuda")
    out, flags = ver.tree_attention(dev(inp.q, spec.dtype), dev(inp.k, spec.dtype), dev(inp.v, spec.dtype),
                                    dev(ind), lens, dev(par), scale, out=out, flags=flags)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert not (got == ATTN_SENTINEL).any(), "attention output rows left unwritten"
    flags = flags.cpu().numpy().astype(np.uint32)
    assert not (flags & 0xFFFFFF00).any(), "attention flags not written"
    return got.astype(np.float64), flags


def run_accept(ver, inp, temperature, seed, offset, target=None, draft=None, parents=None, tokens=None, **kw):
    import torch
    spec = inp.spec
    tgt = inp.target if target is None else target
    drf = inp.draft if draft is None else draft
    par = inp.parents if parents is None else parents
    tok = inp.tokens if tokens is None else tokens
    B, T = np.asarray(par).shape
    res = ver.spec_accept(dev(tgt, spec.ldtype), dev(drf, spec.ldtype), dev(par), dev(tok), temperature,
                          seed, offset, outputs=sentinel_accept_outputs(B, T), **kw)
    torch.cuda.synchronize()
    return host_accept(res)


def _children(parents, tokens):
    """Children of every row, ascending (padding rows, token -1 at a row >= 1,
    are never children)."""
    T = len(parents)
    kids = [[] for _ in range(T)]
    for c in range(1, T):
        if int(tokens[c]) != -1:
            kids[int(parents[c])].append(c)
    return kids


def _check_walk(got, b, parents, tokens, V, context):
    """The GPU's outputs of sequence b describe a walk of its tree: accepted
    nodes form a root path, out_tokens are their tokens plus one final token
    in [0, V), and everything past them is -1."""
    n = int(got["accept_len"][b])
    T = len(parents)
    kids = _children(parents, tokens)
    cur = 0
    for i in range(n):
        node = int(got["accepted_nodes"][b][i])
        assert node in kids[cur], f"{context} seq {b}: accepted node {node} is not a child of {cur}"
        assert int(got["out_tokens"][b][i]) == int(tokens[node]), f"{context} seq {b}: token of node {node}"
        cur = node
    assert 0 <= int(got["out_tokens"][b][n]) < V, f"{context} seq {b}: final token out of range"
    assert (got["accepted_nodes"][b][n:] == -1).all() and (got["out_tokens"][b][n + 1:] == -1).all(), \
        f"{context} seq {b}: outputs past the walk are not -1"
    assert n < T


def compare_accept(got, ref, context="", parents=None, tokens=None, vocab=None):
    """Compare the GPU's acceptance outputs with the oracle's, sequence by
    sequence.

    Where the oracle's walk has no near tie (a decision within 1e-6 of its
    threshold), every output is bit-exact: accept_len, accepted_nodes,
    out_tokens, flags and the near-tie count.  Where it has one, the walks
    must agree on everything decided before it:
      * a near tie on the terminal sample: the accepted path and its tokens
        are identical and only the final token may differ;
      * a near tie on the test of sibling i at depth d: the first d accepted
        nodes are identical, and the GPU did not accept one of the siblings
        before i there;
    and a sequence whose results differ must carry a near tie on the GPU's
    side too (the decision that went the other way lay within the GPU's own
    1e-6 margin).  Given the tree (parents, tokens, vocab), the GPU's outputs
    of such a sequence must still describe a valid walk.

    Returns the number of sequences whose results differ (excused by a near
    tie)."""
    B = ref["accept_len"].shape[0]
    excused = 0
    for b in range(B):
        n_ref, n_got = int(ref["accept_len"][b]), int(got["accept_len"][b])
        same = (n_got == n_ref
                and np.array_equal(got["accepted_nodes"][b], ref["accepted_nodes"][b])
                and np.array_equal(got["out_tokens"][b], ref["out_tokens"][b]))
        if same:
            assert got["flags"][b] == ref["flags"][b], f"{context} seq {b}: flags {got['flags'][b]} vs {ref['flags'][b]}"
            assert int(got["near_ties"][b]) == int(ref["near_ties"][b]), (
                f"{context} seq {b}: near ties {got['near_ties'][b]} vs {ref['near_ties'][b]}")
            continue
        d, slot = int(ref["first_near_depth"][b]), int(ref["first_near_slot"][b])
        msg = (f"{context} seq {b}: GPU {n_got} {got['accepted_nodes'][b][:max(n_got, 0)].tolist()} "
               f"{got['out_tokens'][b][:max(n_got, 0) + 1].tolist()} vs oracle {n_ref} "
               f"{ref['accepted_nodes'][b][:max(n_ref, 0)].tolist()} {ref['out_tokens'][b][:max(n_ref, 0) + 1].tolist()}")
        assert d >= 0, msg + ", and the oracle's walk has no near tie"
        assert int(got["near_ties"][b]) > 0, msg + ", and the GPU reports no near tie"
        assert n_got >= d, msg + f": diverged before the near tie at depth {d}"
        assert np.array_equal(got["accepted_nodes"][b][:d], ref["accepted_nodes"][b][:d]) and \
            np.array_equal(got["out_tokens"][b][:d], ref["out_tokens"][b][:d]), msg + f": diverged before depth {d}"
        if slot < 0:      # the terminal sample: only the final token may differ
            assert n_got == n_ref and np.array_equal(got["accepted_nodes"][b], ref["accepted_nodes"][b]) and \
                np.array_equal(got["out_tokens"][b][:n_ref], ref["out_tokens"][b][:n_ref]), \
                msg + ": the near tie was the terminal sample, yet the path differs"
        elif n_got > d and parents is not None:
            node = 0 if d == 0 else int(ref["accepted_nodes"][b][d - 1])
            kids = _children(parents[b], tokens[b])[node]
            child = int(got["accepted_nodes"][b][d])
            assert child in kids and kids.index(child) >= slot, (
                msg + f": the GPU accepted sibling {kids.index(child) if child in kids else child} at depth {d}, "
                      f"before the near tie at sibling {slot}")
        if parents is not None:
            _check_walk(got, b, parents[b], tokens[b], vocab, context)
        excused += 1
    return excused


def excused_bound(sequences):
    """How many compared sequences may differ through a near tie: a flip
    needs the GPU's and the oracle's roundings to straddle a threshold, far
    rarer than the near tie itself (margins below 1e-6)."""
    return 1 + sequences // 100


def small_spec(name, dtype="bf16", B=1, Hq=8, Hkv=8, D=128, lens=(1000,), levels=(4, 6, 10), rule="rank",
               V=1000, sigma_t=3.0, sigma_d=0.7, temperature=1.0, seed=7, zipf=0.0, tree=None):
    recipe = tree if tree is not None else ("levels", tuple(levels), rule)
    if len(lens) == 1 and B > 1:
        lens = tuple(lens) * B
    return si.WorkloadSpec(name, dtype, B, Hq, Hkv, D, tuple(lens), recipe, V,
                           sigma_t, sigma_d, zipf=zipf, temperature=temperature, seed=seed)


def oracle_rows_sampled(spec, inp, out, samples, scale):
    """Check sampled output rows (b, node, head) against the oracle computed
    from one KV head's rows, regenerated from the seed."""
    from oracle import attention as oa
    errs = []
    cache = {}
    g = spec.q_heads // spec.kv_heads
    q64 = inp.q64()
    for (b, i, h) in samples:
        key = (b, h // g)
        if key not in cache:
            kb, vb = si.kv_head_block(spec, inp.T, b, h // g)
            cache = {key: (si.as_f64(kb, spec.dtype), si.as_f64(vb, spec.dtype))}
        k64, v64 = cache[key]
        ref = oa.node_head_output(q64[b, i, h], k64, v64, spec.prefix_lens[b], inp.parents[b], i, scale)
        errs.append(float(np.abs(out[b, i, h] - ref).max() / np.abs(ref).max()))
    return np.asarray(errs)
