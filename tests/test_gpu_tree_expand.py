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
