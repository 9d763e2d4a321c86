"""GPU parity of tree attention (through the C ABI) against the fp64 oracle.

Element-by-element at sizes the oracle finishes in seconds (several 64-key
tiles, ragged tails, multi-split and single-split sequences in one call,
every MFMA row-tile variant, the FMA path); sampled rows at the full
workload sizes in the launch configuration the benchmark times.
Tolerance: row-normwise max |o - o_ref| / max |o_ref| <= 2e-3 for bf16 inputs
(fp32 accumulation), 1e-5 for fp32.
"""
import numpy as np
import pytest

import synth
from gpu_util import ATTN_TOL, log, make_verifier, oracle_rows_sampled, row_error, run_attention, small_spec
from oracle import attention as oa

pytestmark = pytest.mark.gpu

CASES = [
    small_spec("fp32_fma_ragged", dtype="f32", B=2, Hq=4, Hkv=2, D=64, lens=(300, 0), levels=(4, 4, 2),
               rule="uniform"),
    small_spec("fp32_fma_d128_gqa", dtype="f32", B=1, Hq=8, Hkv=2, D=128, lens=(257,), levels=(3, 3)),
    small_spec("bf16_mb1_two_seqs", B=2, Hq=8, Hkv=8, lens=(1000, 77), levels=(4, 6, 10)),
    small_spec("bf16_mb2_gqa", B=1, Hq=16, Hkv=4, lens=(777,), levels=(4, 6, 10)),
    small_spec("bf16_mb3_gqa", B=1, Hq=16, Hkv=4, lens=(513,), levels=(10, 10, 10, 10)),
    small_spec("bf16_mb4_gqa", B=1, Hq=32, Hkv=4, lens=(1100,), levels=(4, 8, 12)),
    small_spec("bf16_two_row_tiles", B=3, Hq=32, Hkv=2, lens=(513, 1024, 0), levels=(5, 10, 15)),
    small_spec("bf16_small_R_fma", B=1, Hq=2, Hkv=2, lens=(200,), levels=(2, 2)),
    small_spec("bf16_d64", B=2, Hq=8, Hkv=2, D=64, lens=(640, 64), levels=(4, 6, 10)),
    small_spec("bf16_chain", B=1, Hq=8, Hkv=2, lens=(900,), tree=("chain", 12)),
    small_spec("bf16_root_only", B=2, Hq=16, Hkv=1, lens=(129, 5), tree=("chain", 0)),
    small_spec("bf16_full_tree_64", B=1, Hq=4, Hkv=4, lens=(333,), levels=(8, 15, 20, 20)),
    # at most 32 rows per KV head: wave pairs split the keys of each tile
    small_spec("bf16_key_halves_chain8", B=2, Hq=8, Hkv=2, lens=(1500, 130), tree=("chain", 7)),
    small_spec("bf16_key_halves_d64_r20", B=1, Hq=12, Hkv=3, D=64, lens=(700,), levels=(2, 2)),
    small_spec("bf16_key_halves_r16_short", B=2, Hq=16, Hkv=1, lens=(20, 0), tree=("chain", 0)),
]


def _check(spec, inp, got, flags):
    scale = 1.0 / np.sqrt(spec.head_dim)
    ref, rflags = oa.tree_attention(inp.q64(), inp.k64(), inp.v64(), inp.kv_indptr, inp.prefix_lens,
                                    inp.parents, scale)
    assert np.array_equal(flags, rflags.astype(np.uint32))
    err = row_error(got, ref)
    log(f"    max row error {err.max():.3e} (tol {ATTN_TOL[spec.dtype]})")
    assert err.max() <= ATTN_TOL[spec.dtype]


@pytest.mark.parametrize("spec", CASES, ids=lambda s: s.name)
def test_attention_matches_oracle(spec):
    log(f"[attention] {spec.name}")
    inp = synth.make_inputs(spec, with_logits=False)
    ver = make_verifier(spec, inp.T)
    got, flags = run_attention(ver, inp)
    _check(spec, inp, got, flags)
    again, _ = run_attention(ver, inp)
    assert np.array_equal(got, again), "not bitwise deterministic"
    ver.close()


MERGE_CASES = [c for c in CASES if c.name in ("bf16_mb1_two_seqs", "bf16_two_row_tiles", "bf16_d64", "bf16_chain",
                                               "bf16_key_halves_chain8")]


@pytest.mark.parametrize("spec", MERGE_CASES, ids=lambda s: s.name)
def test_attention_separate_merge_kernel(spec, monkeypatch):
    """The split merge as its own kernel (the path taken when the attention
    workgroups cannot all be resident at once) against the oracle and
    against the merge done inside the attention kernel."""
    log(f"[attention] separate merge kernel: {spec.name}")
    inp = synth.make_inputs(spec, with_logits=False)
    ver = make_verifier(spec, inp.T)
    fused, _ = run_attention(ver, inp)
    plan = ver.last_attention_plan()
    assert plan.total_splits > spec.batch and plan.merge_in_kernel == 1
    ver.close()
    monkeypatch.setenv("EAGLE_VERIFY_ATTN_FUSED_MERGE", "0")
    ver = make_verifier(spec, inp.T)
    got, flags = run_attention(ver, inp)
    plan = ver.last_attention_plan()
    assert plan.merge_in_kernel == 0 and plan.merge_workgroups > 0
    ver.close()
    _check(spec, inp, got, flags)
    assert row_error(got, fused).max() <= ATTN_TOL[spec.dtype]


def _with_gaps(inp, gap):
    """The same sequences with `gap` unused rows before each KV block (filled
    with large values that a wrong row offset would pick up)."""
    import dataclasses
    B = inp.spec.batch
    sizes = np.diff(inp.kv_indptr)
    k = np.empty((int(sizes.sum()) + gap * B,) + inp.k.shape[1:], dtype=inp.k.dtype)
    v = np.empty_like(k)
    k[:] = synth.to_bf16_bits(np.float64(300.0)) if inp.k.dtype == np.uint16 else np.float32(300.0)
    v[:] = k
    ind = np.zeros(B + 1, dtype=np.int64)
    for b in range(B):
        start = int(ind[b]) + gap
        k[start:start + sizes[b]] = inp.k[inp.kv_indptr[b]:inp.kv_indptr[b + 1]]
        v[start:start + sizes[b]] = inp.v[inp.kv_indptr[b]:inp.kv_indptr[b + 1]]
        ind[b] = start
        ind[b + 1] = start + sizes[b]
    return dataclasses.replace(inp, k=k, v=v, kv_indptr=ind)


def test_attention_unpacked_kv_layout():
    """KV blocks that are not packed back to back: the first tile, requested
    early from the packed offset, is requested again from kv_indptr."""
    spec = small_spec("unpacked", B=3, Hq=8, Hkv=2, lens=(700, 64, 300), levels=(4, 6, 10))
    log("[attention] unpacked KV layout")
    inp = synth.make_inputs(spec, with_logits=False)
    moved = _with_gaps(inp, gap=37)
    ver = make_verifier(spec, inp.T)
    got, flags = run_attention(ver, moved)
    ver.close()
    _check(spec, moved, got, flags)
    assert np.array_equal(flags, np.zeros(3, dtype=np.uint32))


def test_attention_tiny_config_exact():
    spec = synth.config_spec(0)
    log("[attention] tiny fp32 workload")
    inp = synth.make_inputs(spec)
    ver = make_verifier(spec, inp.T)
    got, flags = run_attention(ver, inp)
    _check(spec, inp, got, flags)
    ver.close()


def test_invalid_sequences_are_flagged_and_poisoned():
    spec = small_spec("bad", B=4, Hq=8, Hkv=2, lens=(600, 300, 300, 64), levels=(4, 6, 10))
    log("[attention] invalid sequences")
    inp = synth.make_inputs(spec, with_logits=False)
    par = inp.parents.copy()
    par[1, 7] = 9                       # parent after child
    par[3, 0] = 0                       # root must be -1
    ind = inp.kv_indptr.copy()
    ind[3] = ind[2] + 10                 # sequence 2 no longer holds L + T rows
    ver = make_verifier(spec, inp.T)
    got, flags = run_attention(ver, inp, parents=par, kv_indptr=ind)
    from eagle_draft_tree_attention_amd import FLAG_BAD_KV_RANGE, FLAG_BAD_TREE
    assert flags[0] == 0
    assert flags[1] == FLAG_BAD_TREE
    assert flags[2] == FLAG_BAD_KV_RANGE
    assert flags[3] & FLAG_BAD_TREE
    assert np.isnan(got[1]).all() and np.isnan(got[2]).all() and np.isnan(got[3]).all()
    scale = 1.0 / np.sqrt(spec.head_dim)
    ref, _ = oa.tree_attention(inp.q64()[:1], inp.k64(), inp.v64(), inp.kv_indptr[:2], inp.prefix_lens[:1],
                               inp.parents[:1], scale)
    assert row_error(got[:1], ref).max() <= ATTN_TOL["bf16"]
    ver.close()


def _samples(spec, inp, rng, n=10):
    T, Hq = inp.T, spec.q_heads
    depth = np.zeros(T, dtype=int)
    for i in range(1, T):
        depth[i] = depth[inp.parents[0][i]] + 1
    out = []
    for b in range(spec.batch):
        nodes = {0, T - 1, int(np.argmax(depth))} | set(int(x) for x in rng.integers(0, T, n))
        for i in sorted(nodes):
            for h in sorted({0, Hq - 1, int(rng.integers(0, Hq))}):
                out.append((b, i, h))
    g = spec.q_heads // spec.kv_heads
    return sorted(out, key=lambda s: (s[0], s[2] // g, s[1], s[2]))


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_attention_full_size_sampled(cfg):
    spec = synth.config_spec(cfg)
    log(f"[attention] full size {spec.name}: generating inputs")
    inp = synth.make_inputs(spec, with_logits=False)
    ver = make_verifier(spec, inp.T)
    log(f"[attention] full size {spec.name}: running")
    got, flags = run_attention(ver, inp)
    ver.close()
    assert (flags == 0).all()
    assert np.isfinite(got).all()
    # every output is (up to the bf16 rounding of the weights) a convex
    # combination of value rows
    v64 = inp.v64()
    vmax, vmin = v64.max(), v64.min()
    del v64
    slack = 0.01 * max(abs(vmax), abs(vmin))
    assert got.max() <= vmax + slack and got.min() >= vmin - slack
    samples = _samples(spec, inp, np.random.default_rng(cfg))
    log(f"[attention] full size {spec.name}: oracle on {len(samples)} sampled rows")
    errs = oracle_rows_sampled(spec, inp, got, samples, 1.0 / np.sqrt(spec.head_dim))
    log(f"    max row error {errs.max():.3e}")
    assert errs.max() <= ATTN_TOL[spec.dtype]
