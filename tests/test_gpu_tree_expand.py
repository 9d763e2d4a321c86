"""GPU parity of the dynamic draft-tree expansion step: the HIP kernels,
called through the C ABI, against the oracle.

The kept (parent, token) pairs must match exactly up to the first ranking
decision the oracle counts as a near tie (values less than 1e-6 apart); the
values must match to 1e-5 (they are returned as float32).  Inputs are
seeded: draft logits drawn like the workloads' (normal logits, plus the
Zipf bias of the 8B workload at its vocabulary), random frontier values,
inactive and unusable rows."""
import numpy as np
import pytest

from gpu_util import dev, log
from oracle import tree_expand as ote

pytestmark = pytest.mark.gpu


def _logits(rng, B, F, V, zipf=False, scale=3.0):
    x = rng.standard_normal((B, F, V)) * scale
    if zipf:
        x += -1.1 * np.log1p(np.arange(V))
    return x.astype(np.float32)


def _to_dtype(x, dtype):
    if dtype == "bf16":   # round to bf16 (nearest even) and keep the fp32 value the kernel will see
        bits = x.view(np.uint32).astype(np.uint64)
        bits = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16).astype(np.uint16)
        return bits, (bits.astype(np.uint32) << 16).view(np.float32)
    return x, x


def _run(ver, x_dev_bits, scores, tau, k, M, dtype):
    import torch
    if dtype == "bf16":
        tx = torch.from_numpy(np.ascontiguousarray(x_dev_bits).view(np.int16)).view(torch.bfloat16).cuda()
    else:
        tx = dev(x_dev_bits)
    out = ver.tree_expand(tx, dev(scores.astype(np.float32)), tau, k, M)
    torch.cuda.synchronize()
    return {key: t.cpu().numpy() for key, t in out.items()}


def _verifier(B, F, V, dtype):
    import eagle_draft_tree_attention_amd as ev
    return ev.Verifier(B, 8, 8, 128, max(F, 1), V, kv_dtype="bf16", logits_dtype=dtype)


def _compare(name, got, want, M):
    B = want["parent"].shape[0]
    for b in range(B):
        # compare the ranking up to the first near tie the oracle reports
        vals = want["value"][b]
        upto = M
        if want["near_ties"][b] > 0:   # positions i and i + 1 of a close pair may swap
            fin = vals[np.isfinite(vals)]
            gaps = np.flatnonzero(fin[:-1] - fin[1:] < ote.NEAR)
            upto = int(gaps[0]) if len(gaps) else M - 1   # else the tie is at the kept/dropped boundary
        assert got["parent"][b][:upto].tolist() == want["parent"][b][:upto].tolist(), (name, b)
        assert got["token"][b][:upto].tolist() == want["token"][b][:upto].tolist(), (name, b)
        fin = np.isfinite(want["value"][b][:upto])
        assert np.array_equal(np.isfinite(got["value"][b][:upto]), fin), (name, b)
        np.testing.assert_allclose(got["value"][b][:upto][fin], want["value"][b][:upto][fin], rtol=0, atol=1e-5)
        assert int(got["flags"][b]) == int(want["flags"][b]), (name, b)
    log(f"  {name}: ok (near ties {want['near_ties'].tolist()})")


CASES = [
    # name, B, F, V, k, M, tau, dtype
    ("f32_three_chunks", 2, 5, 20000, 4, 10, 1.0, "f32"),
    ("bf16_three_chunks_t07", 2, 5, 20000, 4, 10, 0.7, "bf16"),
    ("bf16_k16_keep64_f64", 1, 64, 3000, 16, 64, 1.0, "bf16"),
    ("f32_small_vocab", 3, 4, 7, 16, 20, 1.3, "f32"),
    ("bf16_one_root", 4, 1, 32000, 8, 8, 1.0, "bf16"),
    # a 16-row frontier at V = 128256 has more chunk records per sequence than
    # the one-launch path stages (two launches then)
    ("bf16_wide_frontier_128k", 2, 16, 128256, 4, 16, 1.0, "bf16"),
]


@pytest.mark.parametrize("name,B,F,V,k,M,tau,dtype", CASES, ids=[c[0] for c in CASES])
def test_random_frontiers(name, B, F, V, k, M, tau, dtype):
    rng = np.random.default_rng(sum(map(ord, name)))
    log(f"[tree_expand] {name}")
    x = _logits(rng, B, F, V)
    bits, xk = _to_dtype(x, dtype)
    scores = (-np.abs(rng.standard_normal((B, F))) * 2).astype(np.float32)
    ver = _verifier(B, F, V, dtype)
    got = _run(ver, bits, scores, tau, k, M, dtype)
    want = ote.expand(xk, scores.astype(np.float64), tau, k, M)
    _compare(name, got, want, M)
    ver.close()


def test_inactive_unusable_and_padding():
    rng = np.random.default_rng(11)
    B, F, V, k, M = 2, 6, 9000, 3, 20
    x = _logits(rng, B, F, V)
    scores = (-np.abs(rng.standard_normal((B, F)))).astype(np.float32)
    scores[0, 1] = -np.inf          # inactive
    scores[0, 4] = np.nan           # inactive too
    x[0, 2, 8191] = np.nan          # unusable active row: skipped and flagged
    x[1, 3, :] = -np.inf            # all -inf: unusable
    x[1, 5, 100] = np.inf           # +inf: unusable
    ver = _verifier(B, F, V, "f32")
    got = _run(ver, x, scores, 1.0, k, M, "f32")
    want = ote.expand(x, scores.astype(np.float64), 1.0, k, M)
    assert want["flags"].tolist() == [ote.FLAG_NONFINITE, ote.FLAG_NONFINITE]
    assert (want["parent"][0] == -1).sum() == M - 3 * 3     # three usable active rows of 3 candidates
    _compare("edges", got, want, M)
    assert got["parent"][0][9:].tolist() == [-1] * (M - 9)
    ver.close()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_workload_shape_three_depths(dtype):
    """Three expansion steps at the 8B workload's vocabulary (128256, Zipf
    bias), root k = 8, then 8 kept nodes expanded with k = 4: each side feeds
    its own kept values forward as the next frontier's values."""
    rng = np.random.default_rng(12)
    B, V = 1, 128256
    frontier_gpu = np.zeros((B, 1), dtype=np.float32)
    frontier_ora = np.zeros((B, 1))
    ver = _verifier(B, 8, V, dtype)
    for depth, (k, M) in enumerate([(8, 8), (4, 8), (4, 8)]):
        F = frontier_gpu.shape[1]
        x = _logits(rng, B, F, V, zipf=True, scale=2.0)
        bits, xk = _to_dtype(x, dtype)
        got = _run(ver, bits, frontier_gpu, 1.0, k, M, dtype)
        want = ote.expand(xk, frontier_ora, 1.0, k, M)
        assert want["near_ties"].tolist() == [0], "the seed was chosen without near ties"
        _compare(f"depth {depth}", got, want, M)
        frontier_gpu = got["value"].astype(np.float32)
        frontier_ora = want["value"]
    ver.close()


@pytest.mark.parametrize("seed", [31, 32])
def test_rerank_of_chained_oracle_steps(seed):
    """Steps produced by the oracle (values as float32), reranked on both sides."""
    import torch
    rng = np.random.default_rng(seed)
    B, V = 3, 700
    steps = [(4, 6), (3, 8), (3, 8), (2, 8)]
    Mx = 8
    fr = np.zeros((B, 1))
    P = np.full((len(steps), B, Mx), -1, dtype=np.int32)
    T = np.full((len(steps), B, Mx), -1, dtype=np.int32)
    Vv = np.full((len(steps), B, Mx), -np.inf, dtype=np.float32)
    for d, (k, M) in enumerate(steps):
        x = _logits(rng, B, fr.shape[1], V, scale=2.0)
        out = ote.expand(x, fr, 1.0, k, M)
        P[d, :, :M], T[d, :, :M], Vv[d, :, :M] = out["parent"], out["token"], out["value"].astype(np.float32)
        fr = out["value"]
    roots = np.array([5, 6, 7], dtype=np.int32)
    ver = _verifier(B, 61, V, "f32")   # room for 60 nodes
    for N in (5, 20, 60):
        want = ote.rerank(P, T, Vv, roots, N)
        got = ver.tree_rerank(dev(P), dev(T), dev(Vv), dev(roots), N)
        torch.cuda.synchronize()
        for key in ("parents", "tokens", "rows"):
            assert np.array_equal(got[key].cpu().numpy(), want[key]), (N, key)
    log(f"  rerank seed {seed}: rows {want['rows'].tolist()}")
    ver.close()


def test_short_rerank_output_feeds_verification():
    """A rerank with fewer candidates than rows: its output goes straight into
    spec_accept and tree_attention on the device; the padding rows (parent 0,
    token -1) are accepted as padding and both calls match the oracle."""
    import torch
    from gpu_util import (ATTN_SENTINEL, ATTN_TOL, compare_accept, host_accept, row_error,
                          sentinel_accept_outputs)
    from oracle import accept as oacc
    from oracle import attention as oatt
    rng = np.random.default_rng(41)
    B, V, N = 3, 700, 60
    steps = [(4, 6), (3, 8), (3, 8), (2, 8)]
    fr = np.zeros((B, 1))
    P = np.full((len(steps), B, 8), -1, dtype=np.int32)
    T = np.full((len(steps), B, 8), -1, dtype=np.int32)
    Vv = np.full((len(steps), B, 8), -np.inf, dtype=np.float32)
    for d, (k, M) in enumerate(steps):
        out = ote.expand(_logits(rng, B, fr.shape[1], V, scale=2.0), fr, 1.0, k, M)
        P[d, :, :M], T[d, :, :M], Vv[d, :, :M] = out["parent"], out["token"], out["value"].astype(np.float32)
        fr = out["value"]
    roots = np.array([5, 6, 7], dtype=np.int32)
    ver = _verifier(B, N + 1, V, "f32")
    tree = ver.tree_rerank(dev(P), dev(T), dev(Vv), dev(roots), N)
    par_h, tok_h = tree["parents"].cpu().numpy(), tree["tokens"].cpu().numpy()
    rows = tree["rows"].cpu().numpy()
    assert (rows < N + 1).all() and (par_h[:, rows[0]:] == 0).all() and (tok_h[:, rows[0]:] == -1).all()
    tgt = (rng.standard_normal((B, N + 1, V)) * 2).astype(np.float32)
    drf = (tgt + rng.standard_normal((B, N + 1, V)) * 0.7).astype(np.float32)
    for temp in (1.0, 0.0):
        for off in range(3):
            got = ver.spec_accept(dev(tgt), dev(drf), tree["parents"], tree["tokens"], temp, 0x5EED0000, off,
                                  outputs=sentinel_accept_outputs(B, N + 1))
            torch.cuda.synchronize()
            got = host_accept(got)
            ref = oacc.spec_accept(tgt.astype(np.float64), None if temp == 0 else drf.astype(np.float64),
                                   par_h, tok_h, temp, 0x5EED0000, off)
            assert (ref["flags"] & 7).tolist() == [0] * B and (got["flags"] & 7).tolist() == [0] * B
            assert compare_accept(got, ref, f"rerank tree temperature {temp} offset {off}", par_h, tok_h, V) <= 1
    # tree attention over the same padded trees (bf16, 8 heads, prefix 100)
    Hq = Hkv = 8
    D, L, Tr = 128, 100, N + 1
    q_bits, q32 = _to_dtype(rng.standard_normal((B, Tr, Hq, D)).astype(np.float32), "bf16")
    k_bits, k32 = _to_dtype(rng.standard_normal((B * (L + Tr), Hkv, D)).astype(np.float32), "bf16")
    v_bits, v32 = _to_dtype(rng.standard_normal((B * (L + Tr), Hkv, D)).astype(np.float32), "bf16")
    indptr = np.arange(B + 1, dtype=np.int64) * (L + Tr)
    out = torch.full((B, Tr, Hq, D), float(ATTN_SENTINEL), dtype=torch.float32, device="cuda")
    out, flags = ver.tree_attention(dev(q_bits, "bf16"), dev(k_bits, "bf16"), dev(v_bits, "bf16"), dev(indptr),
                                    [L] * B, tree["parents"], out=out)
    torch.cuda.synchronize()
    assert flags.cpu().numpy().tolist() == [0] * B
    got = out.cpu().numpy().astype(np.float64)
    assert not (got == ATTN_SENTINEL).any()
    scale = 1.0 / np.sqrt(D)
    for b in range(B):
        kb = k32[b * (L + Tr):(b + 1) * (L + Tr)].astype(np.float64)
        vb = v32[b * (L + Tr):(b + 1) * (L + Tr)].astype(np.float64)
        for i in range(int(rows[b])):
            for h in range(Hq):
                ref = oatt.node_head_output(q32[b, i, h].astype(np.float64), kb[:, h], vb[:, h], L, par_h[b], i,
                                            scale)
                assert row_error(got[b, i, h], ref) < ATTN_TOL["bf16"], (b, i, h)
    log(f"  rerank tree rows {rows.tolist()} verified")
    ver.close()
