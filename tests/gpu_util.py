"""Shared helpers of the GPU parity tests: move seeded inputs to the device,
run the library through its C ABI, and compare with the oracle."""
import sys

import numpy as np

import synth
from synth import inputs as si

ATTN_TOL = {"bf16": 2e-3, "f32": 1e-5}


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
    out, flags = ver.tree_attention(dev(inp.q, spec.dtype), dev(inp.k, spec.dtype), dev(inp.v, spec.dtype),
                                    dev(ind), lens, dev(par), scale)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), flags.cpu().numpy().astype(np.uint32)


def run_accept(ver, inp, temperature, seed, offset, target=None, draft=None, parents=None, tokens=None):
    import torch
    spec = inp.spec
    tgt = inp.target if target is None else target
    drf = inp.draft if draft is None else draft
    par = inp.parents if parents is None else parents
    tok = inp.tokens if tokens is None else tokens
    res = ver.spec_accept(dev(tgt, spec.ldtype), dev(drf, spec.ldtype), dev(par), dev(tok), temperature,
                          seed, offset)
    torch.cuda.synchronize()
    out = {k: v.cpu().numpy() for k, v in res.items()}
    out["flags"] = out["flags"].astype(np.uint32)
    return out


def compare_accept(got, ref, context=""):
    """Integers bit-exact; a sequence that differs must carry a near-tie flag
    on one side (decisions within 1e-6 of their threshold).  Returns the
    number of such flagged divergences."""
    B = ref["accept_len"].shape[0]
    diverged = 0
    for b in range(B):
        same = (got["accept_len"][b] == ref["accept_len"][b]
                and np.array_equal(got["accepted_nodes"][b], ref["accepted_nodes"][b])
                and np.array_equal(got["out_tokens"][b], ref["out_tokens"][b]))
        if not same:
            assert ref["near_ties"][b] > 0 or got["near_ties"][b] > 0, (
                f"{context} seq {b}: GPU {got['accept_len'][b]} {got['out_tokens'][b]} vs oracle "
                f"{ref['accept_len'][b]} {ref['out_tokens'][b]}, no near tie")
            diverged += 1
            continue
        assert got["flags"][b] == ref["flags"][b], f"{context} seq {b}: flags {got['flags'][b]} vs {ref['flags'][b]}"
        assert abs(int(got["near_ties"][b]) - int(ref["near_ties"][b])) <= 1, f"{context} seq {b} near ties"
    return diverged


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
