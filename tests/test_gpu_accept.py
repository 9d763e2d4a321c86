"""GPU parity of multi-round speculative sampling (through the C ABI) against
the scalar fp64 oracle on the same Philox stream.

Integers (accept_len, accepted_nodes, out_tokens), flags and near-tie counts
must match bit for bit; a sequence may only differ past the first decision on
the oracle's walk that came within 1e-6 of its threshold (a near tie), and
must agree on everything decided before it (tests/gpu_util.py,
compare_accept).  Every test bounds how many sequences differ.  Besides
parity: losslessness statistics over Philox offsets (chi-square vs the target
distribution; chain closed form), determinism, and the edge cases.
"""
import numpy as np
import pytest
from scipy.special import softmax as sp_softmax
from scipy.stats import chi2 as chi2_dist

import synth
from gpu_util import compare_accept, dev, excused_bound, log, make_verifier, run_accept, small_spec
from eagle_draft_tree_attention_amd import verify as ev
from oracle import accept as oacc

pytestmark = pytest.mark.gpu

SEED = 0x5EED0000


@pytest.fixture(params=["node_parallel", "fused"])
def accept_path(request, monkeypatch):
    """Vocabularies up to 32768 go to the node-parallel kernels when the
    batch exceeds the fused kernel's co-resident capacity;
    EAGLE_VERIFY_NODE_PARALLEL=1 / 0 (read per call) forces either path, so
    both are checked on the same cases."""
    monkeypatch.setenv("EAGLE_VERIFY_NODE_PARALLEL", "1" if request.param == "node_parallel" else "0")
    return request.param

CASES = [
    small_spec("bf16_t1", B=8, V=1000, levels=(4, 6, 10)),
    small_spec("bf16_t07_unaligned_rows", B=4, V=5003, levels=(10, 10, 10), temperature=0.7),
    small_spec("f32_multi_chunk", dtype="f32", B=3, V=20000, levels=(4, 4, 4, 4)),
    small_spec("bf16_low_alpha_many_rounds", B=8, V=20000, sigma_d=2.5, levels=(10, 10)),
    small_spec("bf16_greedy", B=8, V=3000, temperature=0.0, levels=(4, 6, 10)),
    small_spec("bf16_chain", B=6, V=4096, tree=("chain", 9)),
    small_spec("bf16_star", B=6, V=2000, tree=("star", 12), sigma_d=1.5),
]


def _oracle(inp, temperature, offset, **over):
    tgt = over.get("target")
    drf = over.get("draft")
    from synth.inputs import as_f64
    t64 = inp.target64() if tgt is None else as_f64(tgt, inp.spec.ldtype)
    d64 = inp.draft64() if drf is None else as_f64(drf, inp.spec.ldtype)
    par = over.get("parents", inp.parents)
    tok = over.get("tokens", inp.tokens)
    return oacc.spec_accept(t64, None if temperature == 0 else d64, par, tok, temperature, SEED, offset)


@pytest.mark.parametrize("spec", CASES, ids=lambda s: s.name)
def test_accept_matches_oracle(spec, accept_path):
    log(f"[accept] {spec.name}")
    inp = synth.make_inputs(spec, with_kv=False)
    ver = make_verifier(spec, inp.T)
    diverged = 0
    for off in range(12):
        got = run_accept(ver, inp, spec.temperature, SEED, off)
        ref = _oracle(inp, spec.temperature, off)
        diverged += compare_accept(got, ref, f"{spec.name} offset {off}", inp.parents, inp.tokens, spec.vocab)
    log(f"    near-tie divergences: {diverged}")
    assert diverged <= excused_bound(12 * spec.batch)
    # the path the fixture asked for is the one that ran
    paths = ver.last_accept_paths()
    if accept_path == "node_parallel" and spec.vocab <= 32768:
        assert paths == ev.ACCEPT_PATH_NODE_PARALLEL
    else:
        assert paths & ev.ACCEPT_PATH_NODE_PARALLEL == 0 and paths != 0
    again = run_accept(ver, inp, spec.temperature, SEED, 11)
    for key in again:
        assert np.array_equal(again[key], got[key]), "not bitwise deterministic"
    ver.close()


@pytest.mark.parametrize("cfg,temp", [(0, 1.0), (1, 1.0), (1, 0.0), (2, 1.0), (3, 1.0), (4, 1.0), (5, 1.0),
                                      (5, 0.0)])
def test_accept_full_configs(cfg, temp):
    spec = synth.config_spec(cfg, temperature=temp)
    log(f"[accept] full size {spec.name} temperature {temp}")
    inp = synth.make_inputs(spec, with_kv=False)
    ver = make_verifier(spec, inp.T)
    diverged = 0
    for off in range(3):
        got = run_accept(ver, inp, temp, SEED + cfg, off)
        ref = oacc.spec_accept(inp.target64(), None if temp == 0 else inp.draft64(), inp.parents, inp.tokens,
                               temp, SEED + cfg, off)
        diverged += compare_accept(got, ref, f"{spec.name} offset {off}", inp.parents, inp.tokens, spec.vocab)
        log(f"    offset {off}: accept_len {got['accept_len'].tolist()} near ties {got['near_ties'].tolist()}")
    log(f"    near-tie divergences: {diverged}")
    assert diverged <= excused_bound(3 * spec.batch)
    ver.close()


def _custom(B, T, V, dtype="f32"):
    return small_spec("custom", dtype=dtype, B=B, V=V, tree=("chain", T - 1))


def test_edge_cases_flags_and_poison(accept_path):
    import eagle_draft_tree_attention_amd as ev
    log("[accept] edge cases")
    B, T, V = 8, 4, 64
    rng = np.random.default_rng(0)
    spec = _custom(B, T, V)
    inp = synth.make_inputs(spec.with_(q_heads=1, kv_heads=1, prefix_lens=(1,) * B), with_kv=False)
    tgt = (rng.standard_normal((B, T, V)) * 2).astype(np.float32)
    drf = (tgt + rng.standard_normal((B, T, V)) * 0.5).astype(np.float32)
    par = np.tile(np.array([-1, 0, 0, 1], dtype=np.int32), (B, 1))
    tok = np.tile(np.array([0, 5, 9, 3], dtype=np.int32), (B, 1))
    par[1, 3] = 3                                   # bad tree
    tok[2, 2] = V                                   # bad token
    tgt[3, 1, 7] = np.nan                           # unusable target row
    tgt[4, 2, :] = -np.inf                          # all -inf target row
    drf[5, 3, :] = np.nan                           # draft row of a leaf: never read
    tgt[6, 0, :] = -np.inf                          # -inf but for one NaN (root target row)
    tgt[6, 0, 11] = np.nan
    drf[7, 1, :] = -np.inf                          # the same in an internal node's draft row
    drf[7, 1, 40] = np.nan
    ver = make_verifier(spec.with_(batch=B), T)
    got = run_accept(ver, inp, 1.0, SEED, 0, target=tgt, draft=drf, parents=par, tokens=tok)
    ref = oacc.spec_accept(tgt.astype(np.float64), drf.astype(np.float64), par, tok, 1.0, SEED, 0)
    assert got["flags"].tolist() == ref["flags"].tolist() == [0, ev.FLAG_BAD_TREE, ev.FLAG_BAD_TOKEN,
                                                             ev.FLAG_NONFINITE, ev.FLAG_NONFINITE, 0,
                                                             ev.FLAG_NONFINITE, ev.FLAG_NONFINITE]
    assert compare_accept(got, ref, "edge", par, tok, V) == 0
    for b in (1, 2, 3, 4, 6, 7):
        assert got["accept_len"][b] == -1 and (got["out_tokens"][b] == -1).all()
    ver.close()


@pytest.mark.parametrize("V", [3, 16])   # per-token loads, and whole 16-byte groups
def test_p_zero_and_degenerate_residual(V, accept_path):
    import eagle_draft_tree_attention_amd as ev
    log(f"[accept] p = 0 and zero residual, V={V}")
    spec = _custom(2, 3, V)
    inp = synth.make_inputs(spec.with_(q_heads=1, kv_heads=1, prefix_lens=(1, 1)), with_kv=False)
    row = np.full(V, -np.inf, dtype=np.float32)
    row[:2] = np.log(0.5)
    tgt = np.stack([np.stack([row] * 3)] * 2)
    drf = tgt.copy()
    par = np.array([[-1, 0, 0], [-1, 0, 0]], dtype=np.int32)
    tok = np.array([[0, 2, 1], [0, 2, 2]], dtype=np.int32)
    ver = make_verifier(spec.with_(batch=2), 3)
    got = run_accept(ver, inp, 1.0, SEED, 0, target=tgt, draft=drf, parents=par, tokens=tok)
    ref = oacc.spec_accept(tgt.astype(np.float64), drf.astype(np.float64), par, tok, 1.0, SEED, 0)
    assert compare_accept(got, ref, "p0", par, tok, V) == 0
    assert got["flags"][0] & ev.FLAG_P_ZERO and got["flags"][0] & ev.FLAG_DEGENERATE_RESIDUAL
    assert got["accept_len"][0] == 1 and got["accepted_nodes"][0, 0] == 2
    # sequence 1: both children rejected (q = 0 at their token), residual 0 -> sample from q
    assert got["accept_len"][1] == 0 and got["out_tokens"][1, 0] in (0, 1)
    assert got["flags"][1] & ev.FLAG_DEGENERATE_RESIDUAL
    ver.close()


def test_root_only_tree_draws_bonus_from_target(accept_path):
    log("[accept] T = 1")
    V, B = 7, 64
    spec = small_spec("root_only", dtype="f32", B=B, V=V, tree=("chain", 0))
    inp = synth.make_inputs(spec.with_(q_heads=1, kv_heads=1, prefix_lens=(1,) * B), with_kv=False)
    ver = make_verifier(spec, 1)
    counts = np.zeros(V)
    diverged = 0
    for off in range(40):
        got = run_accept(ver, inp, 1.0, SEED, off)
        ref = _oracle(inp, 1.0, off)
        diverged += compare_accept(got, ref, f"root-only {off}", inp.parents, inp.tokens, V)
        assert (got["accept_len"] == 0).all()
        for b in range(B):
            counts[got["out_tokens"][b, 0]] += 1
    assert diverged <= excused_bound(40 * B)
    ver.close()


def test_lossless_statistics_over_offsets(accept_path):
    """Root with three i.i.d. draft children: the first emitted token follows
    the target distribution (chi-square), and every run equals the oracle."""
    log("[accept] chi-square over Philox offsets")
    V, B, K = 6, 256, 40
    rng = np.random.default_rng(3)
    t_row = (rng.standard_normal(V) * 1.5).astype(np.float32)
    d_row = (t_row + rng.standard_normal(V) * 0.9).astype(np.float32)
    q = sp_softmax(t_row.astype(np.float64))
    p = sp_softmax(d_row.astype(np.float64))
    spec = small_spec("stats", dtype="f32", B=B, V=V, tree=("star", 3))
    inp = synth.make_inputs(spec.with_(q_heads=1, kv_heads=1, prefix_lens=(1,) * B), with_kv=False)
    par = np.tile(np.array([-1, 0, 0, 0], dtype=np.int32), (B, 1))
    tgt = np.tile(t_row, (B, 4, 1))
    drf = np.tile(d_row, (B, 4, 1))
    ver = make_verifier(spec, 4)
    counts = np.zeros(V)
    diverged = 0
    for off in range(K):
        tok = np.zeros((B, 4), dtype=np.int32)
        tok[:, 1:] = rng.choice(V, size=(B, 3), p=p)
        got = run_accept(ver, inp, 1.0, SEED, off, target=tgt, draft=drf, parents=par, tokens=tok)
        ref = oacc.spec_accept(tgt.astype(np.float64), drf.astype(np.float64), par, tok, 1.0, SEED, off)
        diverged += compare_accept(got, ref, f"stats offset {off}", par, tok, V)
        counts += np.bincount(got["out_tokens"][:, 0], minlength=V)
    n = B * K
    stat = ((counts - n * q) ** 2 / (n * q)).sum()
    log(f"    chi2 {stat:.2f} (99.9% critical {chi2_dist.ppf(0.999, V - 1):.2f}), near-tie divergences {diverged}")
    assert diverged <= excused_bound(n)
    assert stat < chi2_dist.ppf(0.999, V - 1)
    ver.close()


def test_chain_closed_form_on_gpu(accept_path):
    """E[emitted] = (1 - a^(N+1)) / (1 - a) for a chain with acceptance rate a."""
    log("[accept] chain closed form")
    N, B, K, alpha = 5, 256, 16, 0.8
    spec = small_spec("chain_cf", dtype="f32", B=B, V=2, tree=("chain", N))
    inp = synth.make_inputs(spec.with_(q_heads=1, kv_heads=1, prefix_lens=(1,) * B), with_kv=False)
    tgt = np.tile(np.log(np.array([0.3, 0.7], dtype=np.float32)), (B, N + 1, 1))
    drf = np.tile(np.log(np.array([0.5, 0.5], dtype=np.float32)), (B, N + 1, 1))
    par = np.tile(np.arange(-1, N, dtype=np.int32), (B, 1))
    rng = np.random.default_rng(9)
    ver = make_verifier(spec, N + 1)
    emitted = []
    for off in range(K):
        tok = rng.integers(0, 2, size=(B, N + 1)).astype(np.int32)
        got = run_accept(ver, inp, 1.0, SEED, off, target=tgt, draft=drf, parents=par, tokens=tok)
        emitted.append(got["accept_len"] + 1)
    e = np.concatenate(emitted)
    mean = (1 - alpha ** (N + 1)) / (1 - alpha)
    log(f"    mean emitted {e.mean():.4f} vs {mean:.4f}")
    assert abs(e.mean() - mean) < 4.5 * e.std(ddof=1) / np.sqrt(len(e))
    ver.close()


def test_large_batch_in_fused_slices(monkeypatch):
    """B*T*chunks beyond what the fused kernel can keep co-resident: the
    batch is verified in slices of whole sequences (the uniforms keep the
    sequence's index in the whole batch)."""
    monkeypatch.setenv("EAGLE_VERIFY_NODE_PARALLEL", "0")
    spec = small_spec("large_batch", B=40, V=32000, levels=(10,) * 6, sigma_d=1.2)
    log(f"[accept] {spec.name}")
    inp = synth.make_inputs(spec, with_kv=False)
    ver = make_verifier(spec, inp.T)
    diverged = 0
    for off in range(2):
        got = run_accept(ver, inp, 1.0, SEED, off)
        ref = _oracle(inp, 1.0, off)
        diverged += compare_accept(got, ref, f"large batch offset {off}", inp.parents, inp.tokens, spec.vocab)
    assert diverged <= excused_bound(2 * spec.batch)
    assert ver.last_accept_paths() & ev.ACCEPT_PATH_FUSED
    ver.close()


def test_large_batch_in_one_node_parallel_launch():
    """The same 40-sequence batch on the node-parallel kernels: one workgroup
    per node, no residency requirement, so no slices."""
    spec = small_spec("large_batch_np", B=40, V=32000, levels=(10,) * 6, sigma_d=1.2)
    log(f"[accept] {spec.name}")
    inp = synth.make_inputs(spec, with_kv=False)
    ver = make_verifier(spec, inp.T)
    diverged = 0
    for off in range(2):
        got = run_accept(ver, inp, 1.0, SEED, off)
        ref = _oracle(inp, 1.0, off)
        diverged += compare_accept(got, ref, f"large batch offset {off}", inp.parents, inp.tokens, spec.vocab)
    assert diverged <= excused_bound(2 * spec.batch)
    assert ver.last_accept_paths() == ev.ACCEPT_PATH_NODE_PARALLEL   # chosen without the override
    ver.close()


def test_mixed_invalid_inputs_report_every_flag(accept_path):
    import eagle_draft_tree_attention_amd as ev
    log("[accept] bad token together with an unusable row")
    B, T, V = 2, 4, 64
    rng = np.random.default_rng(5)
    spec = _custom(B, T, V)
    inp = synth.make_inputs(spec.with_(q_heads=1, kv_heads=1, prefix_lens=(1,) * B), with_kv=False)
    tgt = rng.standard_normal((B, T, V)).astype(np.float32)
    drf = rng.standard_normal((B, T, V)).astype(np.float32)
    par = np.tile(np.array([-1, 0, 0, 1], dtype=np.int32), (B, 1))
    tok = np.tile(np.array([0, 5, 9, 3], dtype=np.int32), (B, 1))
    tok[1, 3] = -2
    tgt[1, 2, 0] = np.inf
    ver = make_verifier(spec.with_(batch=B), T)
    got = run_accept(ver, inp, 1.0, SEED, 0, target=tgt, draft=drf, parents=par, tokens=tok)
    ref = oacc.spec_accept(tgt.astype(np.float64), drf.astype(np.float64), par, tok, 1.0, SEED, 0)
    assert got["flags"].tolist() == ref["flags"].tolist() == [0, ev.FLAG_BAD_TOKEN | ev.FLAG_NONFINITE]
    assert compare_accept(got, ref, "mixed", par, tok, V) == 0
    ver.close()


def _pad(spec, inp, sizes):
    """Trees of different sizes in one batch: rows past sizes[b] become padding
    (token -1, parent 0, NaN logits that must never be read)."""
    par, tok = inp.parents.copy(), inp.tokens.copy()
    tgt, drf = inp.target.copy(), inp.draft.copy()
    nan = np.uint16(0x7FC0) if spec.ldtype == "bf16" else np.float32(np.nan)
    for b, n in enumerate(sizes):
        tok[b, n:] = -1
        par[b, n:] = 0
        tgt[b, n:] = nan
        drf[b, n:] = nan
    return par, tok, tgt, drf


@pytest.mark.parametrize("temp", [1.0, 0.0])
def test_trees_of_different_sizes_in_one_batch(temp, accept_path):
    spec = small_spec("padded", B=6, V=3000, levels=(10, 10, 10))
    log(f"[accept] trees of different sizes, temperature {temp}")
    inp = synth.make_inputs(spec, with_kv=False)
    sizes = [inp.T, 20, 9, 4, 2, 1]
    par, tok, tgt, drf = _pad(spec, inp, sizes)
    ver = make_verifier(spec, inp.T)
    diverged = 0
    for off in range(4):
        got = run_accept(ver, inp, temp, SEED, off, target=tgt, draft=drf, parents=par, tokens=tok)
        ref = oacc.spec_accept(synth.inputs.as_f64(tgt, spec.ldtype), None if temp == 0 else synth.inputs.as_f64(drf, spec.ldtype),
                               par, tok, temp, SEED, off)
        assert (ref["flags"] & 7).tolist() == [0] * spec.batch
        diverged += compare_accept(got, ref, f"padded offset {off}", par, tok, spec.vocab)
        for b, n in enumerate(sizes):
            assert got["accept_len"][b] < n
    assert diverged <= excused_bound(4 * spec.batch)
    ver.close()


def test_general_path_with_padded_trees():
    """One sequence needs more workgroups than the fused kernel can keep
    resident (61 rows x 64 vocabulary chunks): the three-kernel path, with
    trees of different sizes."""
    spec = small_spec("general", B=2, V=520000, levels=(10,) * 6, sigma_d=1.2)
    log(f"[accept] {spec.name}: three-kernel path, V {spec.vocab}")
    inp = synth.make_inputs(spec, with_kv=False)
    sizes = [inp.T, 23]
    par, tok, tgt, drf = _pad(spec, inp, sizes)
    ver = make_verifier(spec, inp.T)
    diverged = 0
    for temp in (1.0, 0.0):
        for off in range(2):
            got = run_accept(ver, inp, temp, SEED, off, target=tgt, draft=drf, parents=par, tokens=tok)
            ref = oacc.spec_accept(synth.inputs.as_f64(tgt, spec.ldtype),
                                   None if temp == 0 else synth.inputs.as_f64(drf, spec.ldtype), par, tok, temp, SEED, off)
            diverged += compare_accept(got, ref, f"general temperature {temp} offset {off}", par, tok, spec.vocab)
    assert diverged <= excused_bound(4 * spec.batch)
    ver.close()


def _tokens_without_replacement(spec, inp, rng, temp):
    """Children's tokens drawn from their parent's draft row without
    replacement (siblings distinct), in sibling order."""
    d64 = synth.inputs.as_f64(inp.draft, spec.ldtype)
    tok = inp.tokens.copy()
    for b in range(spec.batch):
        kids = oacc.tree_children(inp.parents[b])
        for n, ch in enumerate(kids):
            if not ch:
                continue
            p = sp_softmax(d64[b, n] / temp)
            tok[b, ch] = rng.choice(spec.vocab, size=len(ch), replace=False, p=p)
    return tok


WR_CASES = [
    small_spec("wr_bf16_t1", B=8, V=1000, levels=(4, 6, 10)),
    small_spec("wr_bf16_t07_multi_chunk", B=3, V=20000, levels=(10, 10, 10), temperature=0.7),
    small_spec("wr_bf16_low_alpha_many_rounds", B=6, V=3000, sigma_d=2.5, levels=(12, 12)),
    small_spec("wr_f32_star", dtype="f32", B=4, V=64, tree=("star", 40), sigma_d=1.5),
]


@pytest.mark.parametrize("spec", WR_CASES, ids=lambda s: s.name)
def test_siblings_without_replacement(spec):
    log(f"[accept] without replacement: {spec.name}")
    inp = synth.make_inputs(spec, with_kv=False)
    tok = _tokens_without_replacement(spec, inp, np.random.default_rng(3), spec.temperature)
    ver = make_verifier(spec, inp.T)
    diverged = 0
    for off in range(6):
        got = run_accept(ver, inp, spec.temperature, SEED, off, tokens=tok, without_replacement=True)
        ref = oacc.spec_accept(inp.target64(), inp.draft64(), inp.parents, tok, spec.temperature, SEED, off,
                               without_replacement=True)
        diverged += compare_accept(got, ref, f"{spec.name} offset {off}", inp.parents, tok, spec.vocab)
    log(f"    near-tie divergences: {diverged}")
    assert diverged <= excused_bound(6 * spec.batch)
    ver.close()


def test_without_replacement_with_repeated_tokens():
    """i.i.d. siblings (tokens may repeat) under the without-replacement rule:
    a repeated token has draft probability 0 there."""
    spec = small_spec("wr_repeats", dtype="f32", B=6, V=6, tree=("star", 8), sigma_d=1.0)
    inp = synth.make_inputs(spec, with_kv=False)
    ver = make_verifier(spec, inp.T)
    diverged = 0
    for off in range(4):
        got = run_accept(ver, inp, 1.0, SEED, off, without_replacement=True)
        ref = oacc.spec_accept(inp.target64(), inp.draft64(), inp.parents, inp.tokens, 1.0, SEED, off,
                               without_replacement=True)
        diverged += compare_accept(got, ref, f"repeats offset {off}", inp.parents, inp.tokens, spec.vocab)
    assert diverged <= excused_bound(4 * spec.batch)
    ver.close()


def test_without_replacement_on_the_three_kernel_path():
    """Sequences too large for the fused kernel (61 rows x 64 vocabulary
    chunks): siblings drawn without replacement, many residual rounds, one
    sequence with repeated tokens, and top-k / top-p filters on top."""
    spec = small_spec("wr_general", B=2, V=520000, levels=(10,) * 6, sigma_d=2.0)
    log(f"[accept] without replacement, three-kernel path: V {spec.vocab}")
    inp = synth.make_inputs(spec, with_kv=False)
    tok = _tokens_without_replacement(spec, inp, np.random.default_rng(4), 1.0)
    tok[1] = inp.tokens[1]                     # i.i.d. siblings: tokens may repeat
    ver = make_verifier(spec, inp.T)
    t64, d64 = inp.target64(), inp.draft64()
    diverged = 0
    for k, p, offs in ((0, 0.0, 3), (50, 0.95, 1)):
        for off in range(offs):
            got = run_accept(ver, inp, 1.0, SEED, off, tokens=tok, without_replacement=True, top_k=k, top_p=p)
            ref = oacc.spec_accept(t64, d64, inp.parents, tok, 1.0, SEED, off, without_replacement=True,
                                   top_k=k, top_p=p)
            diverged += compare_accept(got, ref, f"wr general k {k} p {p} offset {off}", inp.parents, tok,
                                       spec.vocab)
    assert diverged <= excused_bound(4 * spec.batch)
    ver.close()


def test_expected_accept_length_of_a_fixed_tree_on_gpu(accept_path):
    """The GPU's mean accepted length over Philox offsets equals the
    probability flow of a fixed three-level tree (the same tree as the
    oracle's pin), and every run equals the oracle."""
    from test_oracle_accept import _expected_accept_len
    log("[accept] probability flow of a fixed tree")
    rng = np.random.default_rng(13)
    V = 6
    parents = np.array([-1, 0, 0, 0, 0, 1, 1, 5, 2], dtype=np.int32)
    tokens = np.array([0, 1, 3, 2, 0, 2, 0, 5, 4], dtype=np.int32)
    T = len(parents)
    tgt = rng.standard_normal((T, V)) * 1.5
    drf = tgt + rng.standard_normal((T, V)) * 1.5
    tgt, drf = tgt.astype(np.float32), drf.astype(np.float32)
    want = _expected_accept_len([sp_softmax(r) for r in tgt.astype(np.float64)],
                                [sp_softmax(r) for r in drf.astype(np.float64)], parents, tokens)
    B, K = 256, 16
    spec = small_spec("flow", dtype="f32", B=B, V=V, tree=("chain", T - 1))
    inp = synth.make_inputs(spec.with_(q_heads=1, kv_heads=1, prefix_lens=(1,) * B), with_kv=False)
    par, tok = np.tile(parents, (B, 1)), np.tile(tokens, (B, 1))
    tg, dr = np.tile(tgt, (B, 1, 1)), np.tile(drf, (B, 1, 1))
    ver = make_verifier(spec, T)
    lens, diverged = [], 0
    for off in range(K):
        got = run_accept(ver, inp, 1.0, SEED, off, target=tg, draft=dr, parents=par, tokens=tok)
        if off < 4:
            ref = oacc.spec_accept(tg.astype(np.float64), dr.astype(np.float64), par, tok, 1.0, SEED, off)
            diverged += compare_accept(got, ref, f"flow offset {off}", par, tok, V)
        lens.append(got["accept_len"])
    lens = np.concatenate(lens).astype(np.float64)
    se = lens.std(ddof=1) / np.sqrt(len(lens))
    log(f"    mean accepted {lens.mean():.4f} vs flow {want:.4f} (se {se:.4f})")
    assert abs(lens.mean() - want) < 4.5 * se
    assert diverged <= excused_bound(4 * B)
    ver.close()


def _filtered_tokens(spec, inp, rng, k, p, temp):
    """Children drawn from their parent's filtered draft distribution."""
    d64 = synth.inputs.as_f64(inp.draft, spec.ldtype)
    tok = inp.tokens.copy()
    for b in range(spec.batch):
        for n, ch in enumerate(oacc.tree_children(inp.parents[b])):
            if not ch:
                continue
            th, _ = oacc.keep_threshold(d64[b, n], temp, k, p)
            w = sp_softmax(np.where(d64[b, n] < th, -np.inf, d64[b, n]) / temp)
            tok[b, ch] = rng.choice(spec.vocab, size=len(ch), p=w)
    return tok


FILTER_CASES = [
    (small_spec("filt_topk_bf16", B=6, V=1000, levels=(4, 6, 10)), 20, 0.0),
    (small_spec("filt_topp_bf16_multi_chunk", B=4, V=20000, levels=(10, 10, 10)), 0, 0.9),
    (small_spec("filt_both_f32_t07", dtype="f32", B=4, V=5003, levels=(6, 6), temperature=0.7), 50, 0.8),
    (small_spec("filt_topp_low_alpha", B=6, V=3000, sigma_d=2.5, levels=(10, 10)), 0, 0.5),
    (small_spec("filt_topk_1_star", dtype="f32", B=4, V=64, tree=("star", 6)), 1, 0.0),
]


@pytest.mark.parametrize("spec,k,p", FILTER_CASES, ids=[c[0].name for c in FILTER_CASES])
def test_filtered_distributions(spec, k, p, accept_path):
    """top-k / top-p filtered target and draft rows (thresholds found by the
    filter kernel), children drawn from the filtered drafts."""
    log(f"[accept] filtered: {spec.name} top_k {k} top_p {p}")
    inp = synth.make_inputs(spec, with_kv=False)
    tok = _filtered_tokens(spec, inp, np.random.default_rng(5), k, p, spec.temperature)
    ver = make_verifier(spec, inp.T)
    diverged = 0
    for off in range(6):
        got = run_accept(ver, inp, spec.temperature, SEED, off, tokens=tok, top_k=k, top_p=p)
        ref = oacc.spec_accept(inp.target64(), inp.draft64(), inp.parents, tok, spec.temperature, SEED, off,
                               top_k=k, top_p=p)
        assert (ref["flags"] & 7).tolist() == [0] * spec.batch
        diverged += compare_accept(got, ref, f"{spec.name} offset {off}", inp.parents, tok, spec.vocab)
    log(f"    near-tie divergences: {diverged}")
    assert diverged <= excused_bound(6 * spec.batch)
    if accept_path == "node_parallel":
        assert ver.last_accept_paths() == ev.ACCEPT_PATH_NODE_PARALLEL
    ver.close()


def test_filtered_distributions_at_the_8b_shape_and_three_kernel_path():
    """The 8B workload (61 rows over 128256 bf16 logits, many tied values)
    with nucleus and top-k filters, and one sequence too large for the fused
    kernel (three-kernel path)."""
    for spec, k, p, offs in ((synth.config_spec(2), 0, 0.95, 3), (synth.config_spec(2), 40, 0.0, 2),
                             (small_spec("filt_general", B=1, V=520000, levels=(10,) * 6, sigma_d=1.2), 40, 0.9, 2)):
        log(f"[accept] filtered: {spec.name} V {spec.vocab} top_k {k} top_p {p}")
        inp = synth.make_inputs(spec, with_kv=False)
        tok = _filtered_tokens(spec, inp, np.random.default_rng(6), k, p, spec.temperature)
        ver = make_verifier(spec, inp.T)
        t64, d64 = inp.target64(), inp.draft64()
        diverged = 0
        for off in range(offs):
            got = run_accept(ver, inp, spec.temperature, SEED, off, tokens=tok, top_k=k, top_p=p)
            ref = oacc.spec_accept(t64, d64, inp.parents, tok, spec.temperature, SEED, off, top_k=k, top_p=p)
            diverged += compare_accept(got, ref, f"{spec.name} offset {off}", inp.parents, tok, spec.vocab)
        assert diverged <= excused_bound(offs * spec.batch)
        ver.close()


def test_filter_edge_rows(accept_path):
    """Rows the threshold search must resolve by its special cases: all
    logits equal (one value), two tied plateaus, a range of 2e37 (coarse first
    bins), -inf entries beyond top-k, a bf16-like row of few distinct values,
    and a cluster of 8190 distinct values 1e-7 wide in a row 1e30 wide (four
    refinement levels do not separate them: exact bisection)."""
    V, T = 8192, 5
    rng = np.random.default_rng(12)
    base = (rng.standard_normal((T, V)) * 2).astype(np.float32)
    rows = [np.zeros((T, V), np.float32),
            np.tile(np.where(np.arange(V) % 3 == 0, 1.0, 0.5).astype(np.float32), (T, 1))]
    wide = base.copy()
    wide[:, ::7] = -1.0e37
    wide[:, 1] = 1.0e37
    rows.append(wide)
    minf = base.copy()
    minf[:, V // 2:] = -np.inf
    rows.append(minf)
    rows.append((np.round(base * 2) / 2).astype(np.float32))
    cluster = -rng.uniform(0.0, 1e-7, size=(T, V)).astype(np.float32)
    cluster[:, 0] = 0.0
    cluster[:, 1] = -1.0e30
    rows.append(cluster)
    tgt = np.stack(rows)
    drf = tgt + np.float32(0.0)
    B = tgt.shape[0]
    spec = small_spec("filt_edges", dtype="f32", B=B, V=V, tree=("chain", T - 1))
    inp = synth.make_inputs(spec.with_(q_heads=1, kv_heads=1, prefix_lens=(1,) * B), with_kv=False)
    par = np.tile(np.arange(-1, T - 1, dtype=np.int32), (B, 1))
    ver = make_verifier(spec, T)
    for k, p in ((7, 0.0), (0, 0.6), (3000, 0.9), (1, 0.3)):
        log(f"[accept] filter edge rows: top_k {k} top_p {p}")
        tok = np.zeros((B, T), np.int32)
        for b in range(B):
            th, _ = oacc.keep_threshold(drf[b, 0].astype(np.float64), 1.0, k, p)
            kept = np.nonzero(drf[b, 0] >= th)[0]
            tok[b, 1:] = rng.choice(kept, size=T - 1)
        diverged = 0
        for off in range(3):
            got = run_accept(ver, inp, 1.0, SEED, off, target=tgt, draft=drf, parents=par, tokens=tok, top_k=k, top_p=p)
            ref = oacc.spec_accept(tgt.astype(np.float64), drf.astype(np.float64), par, tok, 1.0, SEED, off,
                                   top_k=k, top_p=p)
            assert (ref["flags"] & 7).tolist() == [0] * B
            diverged += compare_accept(got, ref, f"edges k {k} p {p} offset {off}", par, tok, V)
        assert diverged <= 1
        if accept_path == "node_parallel":
            assert ver.last_accept_paths() == ev.ACCEPT_PATH_NODE_PARALLEL
    ver.close()


def test_filters_with_siblings_without_replacement():
    spec = small_spec("filt_wr", B=4, V=2000, levels=(8, 8), sigma_d=1.5)
    log(f"[accept] filtered, without replacement: {spec.name}")
    inp = synth.make_inputs(spec, with_kv=False)
    rng = np.random.default_rng(8)
    d64 = inp.draft64()
    tok = inp.tokens.copy()
    k, p = 30, 0.9
    for b in range(spec.batch):
        for n, ch in enumerate(oacc.tree_children(inp.parents[b])):
            if ch:
                th, _ = oacc.keep_threshold(d64[b, n], 1.0, k, p)
                w = sp_softmax(np.where(d64[b, n] < th, -np.inf, d64[b, n]))
                tok[b, ch] = rng.choice(spec.vocab, size=len(ch), replace=len(ch) > int((w > 0).sum()), p=w)
    ver = make_verifier(spec, inp.T)
    diverged = 0
    for off in range(4):
        got = run_accept(ver, inp, 1.0, SEED, off, tokens=tok, top_k=k, top_p=p, without_replacement=True)
        ref = oacc.spec_accept(inp.target64(), d64, inp.parents, tok, 1.0, SEED, off, without_replacement=True,
                               top_k=k, top_p=p)
        diverged += compare_accept(got, ref, f"filtered wr offset {off}", inp.parents, tok, spec.vocab)
    assert diverged <= excused_bound(4 * spec.batch)
    ver.close()
