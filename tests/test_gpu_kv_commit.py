"""GPU parity of the KV commit: the HIP kernel, called through the C ABI,
against the oracle, byte for byte (it only moves rows).

Inputs are seeded: random K/V bit patterns (every 16-bit or 32-bit pattern
is moved as is), random trees and paths, sequences of different prefix
lengths packed back to back.  Accepted paths come from random root paths or
from the oracle's own acceptance walk on synthetic logits, never from the
GPU."""
import zlib

import numpy as np
import pytest

from gpu_util import dev, log
from oracle import accept as oacc
from oracle import kv_commit as okc

pytestmark = pytest.mark.gpu


def _tree(rng, T):
    return np.asarray([-1] + [int(rng.integers(0, i)) for i in range(1, T)], dtype=np.int32)


def _root_path(par, node):
    p = []
    while node > 0:
        p.append(node)
        node = int(par[node])
    return p[::-1]


def _case(rng, lens, T, Hkv, D, dtype, gap=0):
    B = len(lens)
    indptr = np.zeros(B + 1, dtype=np.int64)
    indptr[1:] = np.cumsum(np.asarray(lens, dtype=np.int64) + T + gap)
    rows = int(indptr[-1])
    if dtype == "bf16":
        k = rng.integers(0, 1 << 16, size=(rows, Hkv, D), dtype=np.uint16)
        v = rng.integers(0, 1 << 16, size=(rows, Hkv, D), dtype=np.uint16)
    else:
        k = rng.integers(0, 1 << 32, size=(rows, Hkv, D), dtype=np.uint32)
        v = rng.integers(0, 1 << 32, size=(rows, Hkv, D), dtype=np.uint32)
    return k, v, indptr


def _nodes(paths, T):
    out = np.full((len(paths), T), -1, dtype=np.int32)
    for b, p in enumerate(paths):
        out[b, :len(p)] = p
    return out


def _gpu_commit(ver, k, v, indptr, lens, accept_len, nodes, dtype, calls=1):
    import torch
    tk = dev(k.view(np.int16) if dtype == "bf16" else k.view(np.int32))
    tv = dev(v.view(np.int16) if dtype == "bf16" else v.view(np.int32))
    for _ in range(calls):
        new_lens, flags = ver.kv_commit(tk, tv, dev(indptr), lens, dev(np.asarray(accept_len, dtype=np.int32)),
                                        dev(nodes))
    torch.cuda.synchronize()
    kk = tk.cpu().numpy().view(k.dtype)
    vv = tv.cpu().numpy().view(v.dtype)
    return kk, vv, new_lens.cpu().numpy(), flags.cpu().numpy().astype(np.uint32)


def _verifier(B, Hkv, D, T, dtype):
    import eagle_draft_tree_attention_amd as ev
    return ev.Verifier(B, Hkv, Hkv, D, T, 1000, kv_dtype=dtype, logits_dtype="f32")


def _check(name, got, want):
    kk, vv, nl, fl = got
    k2, v2, nl2, fl2 = want
    log(f"  {name}: new_lens {nl.tolist()[:8]} flags {fl.tolist()[:8]}")
    assert nl.tolist() == nl2.tolist(), name
    assert fl.tolist() == fl2.tolist(), name
    assert np.array_equal(kk, k2), name
    assert np.array_equal(vv, v2), name


CASES = [
    # name, lens, T, Hkv, D, dtype
    ("bf16_d128_three_seqs", (37, 0, 130), 21, 8, 128, "bf16"),
    ("f32_d64_two_seqs", (5, 64), 16, 2, 64, "f32"),
    ("bf16_d64_max_tree", (300,), 64, 4, 64, "bf16"),
    ("f32_d128_one_node", (9, 3, 17, 1), 1, 1, 128, "f32"),
    # an odd head count keeps whole rows in one workgroup: a move of
    # 2 x 129 x 128 x 4 bytes spans several copy chunks
    ("f32_d128_129_heads", (41, 7), 24, 129, 128, "f32"),
]


@pytest.mark.parametrize("name,lens,T,Hkv,D,dtype", CASES, ids=[c[0] for c in CASES])
def test_random_root_paths(name, lens, T, Hkv, D, dtype):
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    log(f"[kv_commit] {name}")
    k, v, indptr = _case(rng, lens, T, Hkv, D, dtype)
    paths = []
    for _ in lens:
        par = _tree(rng, T)
        paths.append(_root_path(par, int(rng.integers(0, T))))
    alen = [len(p) for p in paths]
    nodes = _nodes(paths, T)
    ver = _verifier(len(lens), Hkv, D, T, dtype)
    got = _gpu_commit(ver, k, v, indptr, list(lens), alen, nodes, dtype)
    _check(name, got, okc.kv_commit(k, v, indptr, lens, np.asarray(alen), nodes, T))
    ver.close()


def test_overlap_chain_and_edge_conventions():
    rng = np.random.default_rng(7)
    T, Hkv, D = 8, 2, 128
    lens = [4, 6, 0, 11, 3, 2]
    k, v, indptr = _case(rng, lens, T, Hkv, D, "bf16", gap=3)
    paths = [[2, 3, 5, 7],      # overlapping sources and destinations
             [1, 2, 3, 4, 5, 6, 7],   # a chain: nothing moves
             [],                 # poisoned (accept_len -1): the root only
             [3, 3],             # not increasing: flagged, nothing moves
             [4, 8],             # node index outside the tree: flagged
             [6]]
    alen = [4, 7, -1, 2, 2, 1]
    nodes = _nodes(paths, T)
    ver = _verifier(len(lens), Hkv, D, T, "bf16")
    got = _gpu_commit(ver, k, v, indptr, lens, alen, nodes, "bf16")
    want = okc.kv_commit(k, v, indptr, lens, np.asarray(alen), nodes, T)
    assert want[3].tolist() == [0, 0, 0, okc.FLAG_BAD_TREE, okc.FLAG_BAD_TREE, 0]
    _check("edges", got, want)
    ver.close()


def test_bad_kv_range_is_flagged_and_moves_nothing():
    rng = np.random.default_rng(8)
    T, Hkv, D = 6, 2, 64
    lens = [5, 7]
    k, v, indptr = _case(rng, lens, T, Hkv, D, "f32")
    bad = indptr.copy()
    bad[1] -= 1
    nodes = _nodes([[2, 4], [1, 5]], T)
    ver = _verifier(2, Hkv, D, T, "f32")
    got = _gpu_commit(ver, k, v, bad, lens, [2, 2], nodes, "f32")
    want = okc.kv_commit(k, v, bad, lens, np.asarray([2, 2]), nodes, T)
    assert want[3].tolist() == [okc.FLAG_BAD_KV_RANGE, 0]
    _check("bad range", got, want)
    ver.close()


def test_two_calls_in_a_row_act_on_the_committed_cache():
    rng = np.random.default_rng(9)
    T, Hkv, D = 12, 4, 128
    lens = [20, 33]
    k, v, indptr = _case(rng, lens, T, Hkv, D, "bf16")
    nodes = _nodes([[1, 4, 9], [2, 6]], T)
    ver = _verifier(2, Hkv, D, T, "bf16")
    got = _gpu_commit(ver, k, v, indptr, lens, [3, 2], nodes, "bf16", calls=2)
    once = okc.kv_commit(k, v, indptr, lens, np.asarray([3, 2]), nodes, T)
    twice = okc.kv_commit(once[0], once[1], indptr, lens, np.asarray([3, 2]), nodes, T)
    _check("two calls", got, twice)
    ver.close()


@pytest.mark.parametrize("layers,B,Hkv", [(3, 2, 2), (8, 40, 8)], ids=["3x2_heads2", "8x40_heads8"])
def test_every_layer_in_one_launch(layers, B, Hkv):
    # the second shape has 320 (layer, sequence) pairs: each workgroup moves
    # a group of 4 of the 8 heads
    rng = np.random.default_rng(10 + B)
    T, D = 9, 64
    lens = [6, 14] if B == 2 else [int(x) for x in rng.integers(0, 30, size=B)]
    per = [_case(rng, lens, T, Hkv, D, "bf16") for _ in range(layers)]
    indptr = per[0][2]
    k = np.stack([p[0] for p in per])
    v = np.stack([p[1] for p in per])
    if B == 2:
        paths = [[2, 5, 8], [3, 4]]
    else:
        paths = [_root_path(_tree(rng, T), int(rng.integers(0, T))) for _ in range(B)]
    nodes = _nodes(paths, T)
    alen = [len(p) for p in paths]
    log(f"[kv_commit] layers {layers} B {B} Hkv {Hkv}")
    ver = _verifier(B, Hkv, D, T, "bf16")
    got = _gpu_commit(ver, k, v, indptr, lens, alen, nodes, "bf16")
    want_k, want_v = [], []
    for layer in range(layers):
        r = okc.kv_commit(k[layer], v[layer], indptr, lens, np.asarray(alen), nodes, T)
        want_k.append(r[0])
        want_v.append(r[1])
        nl, fl = r[2], r[3]
    _check("layers", got, (np.stack(want_k), np.stack(want_v), nl, fl))
    ver.close()


@pytest.mark.parametrize("cfg", [0, 2, 5])
def test_after_the_oracle_walk_at_workload_shape(cfg):
    """The path the oracle's acceptance walk takes on the workload's synthetic
    logits, committed into a cache of the workload's shape (for the 8K
    configuration: 8 KV heads, D 128, prefix 8192, 61 tree rows)."""
    import synth
    spec = synth.config_spec(cfg)
    inp = synth.make_inputs(spec, with_kv=False)
    T = inp.T
    res = oacc.spec_accept(inp.target64(), inp.draft64(), inp.parents, inp.tokens, spec.temperature,
                           0x5EED0002, 3)
    alen = np.asarray(res["accept_len"], dtype=np.int32)
    nodes = np.asarray(res["accepted_nodes"], dtype=np.int32)
    log(f"[kv_commit] {spec.name}: oracle walk accept_len {alen.tolist()} path {nodes[0][:max(alen[0], 0)].tolist()}")
    rng = np.random.default_rng(100 + cfg)
    k, v, indptr = _case(rng, list(spec.prefix_lens), T, spec.kv_heads, spec.head_dim, spec.dtype)
    ver = _verifier(spec.batch, spec.kv_heads, spec.head_dim, T, spec.dtype)
    got = _gpu_commit(ver, k, v, indptr, list(spec.prefix_lens), alen, nodes, spec.dtype)
    _check(spec.name, got, okc.kv_commit(k, v, indptr, spec.prefix_lens, alen, nodes, T))
    ver.close()
