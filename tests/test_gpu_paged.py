"""GPU parity with paged K/V (per-sequence page tables over one page pool, as
a serving engine's block allocator leaves them).  The GPU runs on the paged
layout, the oracle on the contiguous rows: paging only relabels rows, so the
attention outputs must match the oracle to the usual tolerance and the
contiguous GPU call bit for bit; the committed cache, gathered back through
the table by the oracle, must equal the oracle's commit byte for byte."""
import zlib

import numpy as np
import pytest

import synth
from gpu_util import (ATTN_SENTINEL, ATTN_TOL, FLAGS_SENTINEL, dev, log, make_verifier, oracle_rows_sampled, row_error,
                      run_attention, small_spec)
from oracle import attention as oa
from oracle import kv_commit as okc
from oracle import paging as opg
from synth.paging import to_paged

pytestmark = pytest.mark.gpu

CASES = [
    (small_spec("paged_bf16_p64", B=3, Hq=16, Hkv=4, lens=(1000, 77, 0), levels=(4, 6, 10)), 64),
    (small_spec("paged_bf16_p128_splits", B=2, Hq=32, Hkv=8, lens=(3000, 1500), levels=(10,) * 6), 128),
    (small_spec("paged_bf16_d64_p256", B=2, Hq=8, Hkv=2, D=64, lens=(640, 64), levels=(4, 6, 10)), 256),
    (small_spec("paged_bf16_chain_p64", B=2, Hq=8, Hkv=2, lens=(1500, 130), tree=("chain", 7)), 64),
    (small_spec("paged_f32_fma_p64", dtype="f32", B=2, Hq=4, Hkv=2, D=64, lens=(300, 0), levels=(4, 4, 2),
                rule="uniform"), 64),
]


def _run_paged(ver, inp, kp, vp, table, P):
    import torch
    spec = inp.spec
    B, T = inp.q.shape[:2]
    out = torch.full((B, T, spec.q_heads, spec.head_dim), float(ATTN_SENTINEL), dtype=torch.float32, device="cuda")
    flags = torch.full((B,), FLAGS_SENTINEL, dtype=torch.int32, device="cuda")
    out, flags = ver.tree_attention(dev(inp.q, spec.dtype), dev(kp, spec.dtype), dev(vp, spec.dtype), None,
                                    inp.prefix_lens, dev(inp.parents), 1.0 / np.sqrt(spec.head_dim),
                                    out=out, flags=flags, page_table=dev(table), page_size=P)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert not (got == ATTN_SENTINEL).any(), "attention output rows left unwritten"
    return got.astype(np.float64), flags.cpu().numpy().astype(np.uint32)


@pytest.mark.parametrize("spec,P", CASES, ids=[c[0].name for c in CASES])
def test_paged_attention(spec, P):
    log(f"[paged attention] {spec.name} page {P}")
    inp = synth.make_inputs(spec, with_logits=False)
    rng = np.random.default_rng(zlib.crc32(spec.name.encode()))
    kp, vp, table = to_paged(inp.k, inp.v, inp.kv_indptr, inp.prefix_lens, inp.T, P, rng)
    ver = make_verifier(spec, inp.T)
    got, flags = _run_paged(ver, inp, kp, vp, table, P)
    ref, rflags = oa.tree_attention(inp.q64(), inp.k64(), inp.v64(), inp.kv_indptr, inp.prefix_lens,
                                    inp.parents, 1.0 / np.sqrt(spec.head_dim))
    assert np.array_equal(flags, rflags.astype(np.uint32))
    err = row_error(got, ref)
    log(f"    max row error {err.max():.3e}")
    assert err.max() <= ATTN_TOL[spec.dtype]
    contiguous, _ = run_attention(ver, inp)
    assert np.array_equal(got, contiguous), "paged and contiguous results differ"
    ver.close()


def test_page_outside_the_pool_is_flagged():
    import eagle_draft_tree_attention_amd as ev
    spec = small_spec("paged_bad", B=2, Hq=8, Hkv=2, lens=(500, 300), levels=(4, 6))
    inp = synth.make_inputs(spec, with_logits=False)
    rng = np.random.default_rng(5)
    kp, vp, table = to_paged(inp.k, inp.v, inp.kv_indptr, inp.prefix_lens, inp.T, 64, rng)
    table[0, 3] = kp.shape[0] // 64          # one past the last page
    ver = make_verifier(spec, inp.T)
    got, flags = _run_paged(ver, inp, kp, vp, table, 64)
    assert flags.tolist() == [ev.FLAG_BAD_KV_RANGE, 0]
    assert np.isnan(got[0]).all()
    ref, _ = oa.tree_attention(inp.q64()[1:], inp.k64(), inp.v64(), inp.kv_indptr[1:], inp.prefix_lens[1:],
                               inp.parents[1:], 1.0 / np.sqrt(spec.head_dim))
    assert row_error(got[1:], ref).max() <= ATTN_TOL["bf16"]
    ver.close()


def test_serving_batch_paged_sampled():
    """The 32-sequence serving batch with 64-row pages: sampled rows against
    the oracle, every row against the contiguous call bit for bit."""
    spec = synth.config_spec(5)
    log(f"[paged attention] {spec.name}: generating inputs")
    inp = synth.make_inputs(spec, with_logits=False)
    kp, vp, table = to_paged(inp.k, inp.v, inp.kv_indptr, inp.prefix_lens, inp.T, 64, np.random.default_rng(6))
    ver = make_verifier(spec, inp.T)
    got, flags = _run_paged(ver, inp, kp, vp, table, 64)
    assert (flags == 0).all()
    contiguous, _ = run_attention(ver, inp)
    assert np.array_equal(got, contiguous)
    rng = np.random.default_rng(7)
    samples = sorted({(int(rng.integers(0, spec.batch)), int(rng.integers(0, inp.T)), int(rng.integers(0, spec.q_heads)))
                      for _ in range(40)}, key=lambda s: (s[0], s[2] // spec.group, s[1], s[2]))
    errs = oracle_rows_sampled(spec, inp, got, samples, 1.0 / np.sqrt(spec.head_dim))
    log(f"    max row error {errs.max():.3e} over {len(samples)} sampled rows")
    assert errs.max() <= ATTN_TOL[spec.dtype]
    ver.close()


@pytest.mark.parametrize("dtype,P", [("bf16", 64), ("f32", 128)])
def test_paged_kv_commit(dtype, P):
    import torch
    import eagle_draft_tree_attention_amd as ev
    from test_gpu_kv_commit import _case, _nodes, _root_path, _tree
    rng = np.random.default_rng(11 + P)
    lens, T, Hkv, D = [37, 0, 300, 129], 21, 4, 128
    k, v, indptr = _case(rng, lens, T, Hkv, D, dtype)
    paths = [_root_path(_tree(rng, T), int(rng.integers(0, T))) for _ in lens]
    paths[1] = [1, 2, 3]                       # may be invalid for its tree: only the path matters here
    alen = np.asarray([len(p) for p in paths], dtype=np.int32)
    nodes = _nodes(paths, T)
    kp, vp, table = to_paged(k, v, indptr, lens, T, P, rng)
    ver = ev.Verifier(len(lens), Hkv, Hkv, D, T, 1000, kv_dtype=dtype, logits_dtype="f32")
    view = np.int16 if dtype == "bf16" else np.int32
    tk, tv = dev(kp.view(view)), dev(vp.view(view))
    new_lens, flags = ver.kv_commit(tk, tv, None, lens, dev(alen), dev(nodes), page_table=dev(table), page_size=P)
    torch.cuda.synchronize()
    kk, vv = tk.cpu().numpy().view(kp.dtype), tv.cpu().numpy().view(vp.dtype)
    k2, v2, nl2, fl2 = okc.kv_commit(k, v, indptr, lens, alen, nodes, T)
    assert new_lens.cpu().numpy().tolist() == nl2.tolist()
    assert flags.cpu().numpy().astype(np.uint32).tolist() == fl2.tolist()
    for b, L in enumerate(lens):
        n = L + T
        assert np.array_equal(opg.gather(kk, table, b, n, P), k2[indptr[b]: indptr[b] + n]), b
        assert np.array_equal(opg.gather(vv, table, b, n, P), v2[indptr[b]: indptr[b] + n]), b
    ver.close()
