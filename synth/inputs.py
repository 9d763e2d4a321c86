"""Seeded synthetic workloads shaped like the verification step of EAGLE.

The shapes follow the configurations the method is evaluated on (one target
layer, prefix KV cache plus a draft tree appended after it, target and draft
next-token logits per tree node).  Values are drawn in float64 with NumPy's
PCG64 and then rounded once to the workload dtype; every consumer reads those
rounded values, so the HIP path and the oracle see identical bits.

Nothing in this module computes attention or the acceptance rule.  The only
distribution arithmetic here is the drafter's own token draw (children of a
node are sampled from that node's draft distribution, as a non-greedy EAGLE
drafter samples k children), which is input preparation, outside the verified
path.

Layouts (row-major, innermost last):
  q        [B, T, Hq, D]
  k, v     [sum_b (L_b + T), Hkv, D]; sequence b occupies rows
           kv_indptr[b] .. kv_indptr[b+1]-1, prefix rows first, then the T
           tree-node rows in node order
  parents  [B, T] int32, parents[b,0] = -1, parents[b,i] < i
  tokens   [B, T] int32, tokens[b,0] is the already-committed root token
  target, draft [B, T, V]  row n = next-token logits after node n
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Sequence, Tuple

import numpy as np

# stream tags for independent PCG64 streams
_TAG_TREE, _TAG_Q, _TAG_K, _TAG_V, _TAG_TGT, _TAG_DRF, _TAG_TOK = range(7)


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng([int(x) for x in key])


# ----------------------------------------------------------------------------
# dtype rounding
# ----------------------------------------------------------------------------
def to_bf16_bits(x) -> np.ndarray:
    """float64 -> bfloat16 bit patterns: round to float32, then
    round-to-nearest-even onto the upper 16 bits."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    # infinities and NaN keep their class
    special = (u & np.uint32(0x7F800000)) == np.uint32(0x7F800000)
    if special.any():
        r = np.where(special, (u >> np.uint32(16)) | np.where(
            (u & np.uint32(0xFFFF)) != 0, np.uint32(0x40), np.uint32(0)), r)
    return r.astype(np.uint16)


def bf16_bits_to_f64(b) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint16))
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _round(x64: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return to_bf16_bits(x64)
    if dtype == "f32":
        return np.asarray(x64, dtype=np.float32)
    raise ValueError(dtype)


def as_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of stored values (bf16 bits or float32)."""
    if dtype == "bf16":
        return bf16_bits_to_f64(arr)
    return np.asarray(arr, dtype=np.float64)


# ----------------------------------------------------------------------------
# workload description
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class WorkloadSpec:
    name: str
    dtype: str                      # "f32" or "bf16" (q, k, v and logits)
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    prefix_lens: Tuple[int, ...]    # L_b per sequence
    tree: Tuple                     # tree recipe, see make_tree
    vocab: int
    sigma_t: float                  # target logits ~ N(0, sigma_t^2)
    sigma_d: float                  # draft = target + N(0, sigma_d^2)
    zipf: float = 0.0               # target bias[v] = -zipf * ln(1 + v)
    temperature: float = 1.0        # 0 => greedy trees (top-k children)
    seed: int = 1000
    logits_dtype: Optional[str] = None   # defaults to dtype

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads

    @property
    def ldtype(self) -> str:
        return self.logits_dtype or self.dtype

    def with_(self, **kw) -> "WorkloadSpec":
        return replace(self, **kw)


def _levels(sizes, rule):
    return ("levels", tuple(int(s) for s in sizes), rule)


# The five workloads the method is characterised on (one layer each):
#  0 tiny fp32 sanity case, 1 LLaMA-7B-shaped, 2 LLaMA-3.1-8B-shaped with GQA
#  and an 8K prefix, 3 long-context agent shape (128K prefix, near-chain tree),
#  4 70B-shaped batch of four ragged prefixes, 5 a serving batch of 32
#  sequences with ragged prefixes.
CONFIGS = {
    0: WorkloadSpec("tiny_fp32", "f32", 1, 4, 4, 64, (128,),
                    _levels((4, 4, 2), "uniform"), 1024, 3.0, 1.0, seed=1000),
    1: WorkloadSpec("llama7b_2k", "bf16", 1, 32, 32, 128, (2048,),
                    _levels((10,) * 6, "rank"), 32000, 3.0, 0.7, seed=1001),
    2: WorkloadSpec("llama31_8b_8k", "bf16", 1, 32, 8, 128, (8192,),
                    _levels((10,) * 6, "rank"), 128256, 3.0, 0.5, zipf=1.1,
                    seed=1002),
    3: WorkloadSpec("agent_8b_128k", "bf16", 1, 32, 8, 128, (131072,),
                    ("c3",), 128256, 4.0, 1.0, seed=1003),
    4: WorkloadSpec("llama70b_b4", "bf16", 4, 64, 8, 128, (1024, 2048, 3072, 4096),
                    _levels((10,) * 6, "rank"), 32000, 3.0, 0.7, seed=1004),
    # serving batch: 32 sequences of an 8B-shaped model, prefixes log-uniform
    # in [512, 4096] (drawn once from PCG64 seed 1005), 60-node trees
    5: WorkloadSpec("serving_b32", "bf16", 32, 32, 8, 128,
                    tuple(int(x) for x in np.rint(np.exp(np.random.default_rng(1005).uniform(
                        np.log(512.0), np.log(4096.0), 32)))),
                    _levels((10,) * 6, "rank"), 32000, 3.0, 0.7, seed=1005),
}


def config_spec(i: int, temperature: Optional[float] = None) -> WorkloadSpec:
    s = CONFIGS[i]
    if temperature is not None:
        s = s.with_(temperature=float(temperature))
    return s


# ----------------------------------------------------------------------------
# draft-tree topology
# ----------------------------------------------------------------------------
def make_tree(recipe: Tuple, rng: np.random.Generator) -> np.ndarray:
    """Return parents[T] (BFS order, siblings contiguous, parents[i] < i).

    recipes:
      ("levels", sizes, "uniform"|"rank")  level l has sizes[l-1] nodes; each
          picks its parent on level l-1 uniformly or with probability
          proportional to 1/(rank+1) (rank = position on that level, so the
          first, most probable draft branches grow deeper and wider)
      ("chain", n)       root -> 1 -> 2 -> ... -> n
      ("star", k)        root with k leaf children
      ("c3",)            root -> {1, 2}, then 1 -> 3 -> 4 -> ... -> 8
      ("explicit", parents)
    """
    kind = recipe[0]
    if kind == "explicit":
        return np.asarray(recipe[1], dtype=np.int32)
    if kind == "chain":
        n = int(recipe[1])
        return np.arange(-1, n, dtype=np.int32)
    if kind == "star":
        k = int(recipe[1])
        return np.array([-1] + [0] * k, dtype=np.int32)
    if kind == "c3":
        return np.array([-1, 0, 0, 1, 3, 4, 5, 6, 7], dtype=np.int32)
    if kind == "levels":
        sizes, rule = recipe[1], recipe[2]
        parents = [-1]
        prev = [0]
        for lvl, n in enumerate(sizes):
            if lvl == 0:
                par = np.zeros(n, dtype=np.int64)
            else:
                m = len(prev)
                if rule == "uniform":
                    w = np.ones(m)
                elif rule == "rank":
                    w = 1.0 / (np.arange(m) + 1.0)
                else:
                    raise ValueError(rule)
                idx = rng.choice(m, size=n, p=w / w.sum())
                par = np.sort(np.asarray(prev)[idx])
            base = len(parents)
            parents.extend(int(p) for p in par)
            prev = list(range(base, base + n))
        return np.asarray(parents, dtype=np.int32)
    raise ValueError(recipe)


def tree_rows(spec: WorkloadSpec) -> int:
    return int(len(make_tree(spec.tree, _rng(spec.seed, _TAG_TREE, 0))))


# ----------------------------------------------------------------------------
# the inputs bundle
# ----------------------------------------------------------------------------
@dataclass
class Inputs:
    spec: WorkloadSpec
    T: int
    q: np.ndarray            # [B,T,Hq,D]  bf16 bits (uint16) or float32
    k: Optional[np.ndarray]  # [rows,Hkv,D]
    v: Optional[np.ndarray]
    kv_indptr: np.ndarray    # int64 [B+1]
    prefix_lens: np.ndarray  # int32 [B]
    parents: np.ndarray      # int32 [B,T]
    tokens: np.ndarray       # int32 [B,T]
    target: Optional[np.ndarray]  # [B,T,V]
    draft: Optional[np.ndarray]
    extra: dict = field(default_factory=dict)

    # exact float64 views --------------------------------------------------
    def q64(self):
        return as_f64(self.q, self.spec.dtype)

    def k64(self):
        return as_f64(self.k, self.spec.dtype)

    def v64(self):
        return as_f64(self.v, self.spec.dtype)

    def target64(self):
        return as_f64(self.target, self.spec.ldtype)

    def draft64(self):
        return as_f64(self.draft, self.spec.ldtype)


def kv_head_block(spec: WorkloadSpec, T: int, b: int, h: int):
    """K and V rows of sequence b, KV head h as stored values: [L_b+T, D] each."""
    n = spec.prefix_lens[b] + T
    k = _round(_rng(spec.seed, _TAG_K, b, h).standard_normal((n, spec.head_dim)), spec.dtype)
    v = _round(_rng(spec.seed, _TAG_V, b, h).standard_normal((n, spec.head_dim)), spec.dtype)
    return k, v


def _logits(spec: WorkloadSpec, T: int, b: int):
    V = spec.vocab
    t64 = _rng(spec.seed, _TAG_TGT, b).standard_normal((T, V)) * spec.sigma_t
    if spec.zipf:
        t64 += -spec.zipf * np.log1p(np.arange(V, dtype=np.float64))[None, :]
    d64 = t64 + _rng(spec.seed, _TAG_DRF, b).standard_normal((T, V)) * spec.sigma_d
    return _round(t64, spec.ldtype), _round(d64, spec.ldtype)


def _draw_tokens(spec: WorkloadSpec, parents: np.ndarray, draft_row_f64, rng):
    """Children tokens as a drafter would emit them.

    temperature > 0: each child is an independent draw from the parent's
    draft distribution softmax(draft/temperature) (non-greedy EAGLE drafting).
    temperature == 0: the children of a node are its top-k draft tokens in
    descending draft score (ties: lower id first).
    """
    T = len(parents)
    tok = np.zeros(T, dtype=np.int32)
    tok[0] = int(rng.integers(0, spec.vocab))
    for n in range(T):
        kids = [c for c in range(1, T) if parents[c] == n]
        if not kids:
            continue
        row = draft_row_f64(n)
        if spec.temperature > 0:
            z = row / spec.temperature
            z = z - z.max()
            w = np.exp(z)
            w /= w.sum()
            draws = rng.choice(spec.vocab, size=len(kids), p=w)
        else:
            draws = np.argsort(-row, kind="stable")[: len(kids)]
        for c, t in zip(kids, draws):
            tok[c] = int(t)
    return tok


def make_inputs(spec: WorkloadSpec, *, with_kv: bool = True,
                with_logits: bool = True) -> Inputs:
    """Build every input of one verification step for `spec`."""
    B, Hq, Hkv, D = spec.batch, spec.q_heads, spec.kv_heads, spec.head_dim
    assert len(spec.prefix_lens) == B and Hq % Hkv == 0
    trees = [make_tree(spec.tree, _rng(spec.seed, _TAG_TREE, b)) for b in range(B)]
    T = len(trees[0])
    assert all(len(t) == T for t in trees), "all sequences share the tree row count"
    parents = np.stack(trees).astype(np.int32)

    q = np.stack([_round(_rng(spec.seed, _TAG_Q, b).standard_normal((T, Hq, D)), spec.dtype)
                  for b in range(B)])
    lens = np.asarray(spec.prefix_lens, dtype=np.int32)
    indptr = np.zeros(B + 1, dtype=np.int64)
    indptr[1:] = np.cumsum(lens.astype(np.int64) + T)

    k = v = None
    if with_kv:
        kd = np.uint16 if spec.dtype == "bf16" else np.float32
        k = np.empty((int(indptr[-1]), Hkv, D), dtype=kd)
        v = np.empty_like(k)
        for b in range(B):
            for h in range(Hkv):
                kb, vb = kv_head_block(spec, T, b, h)
                k[indptr[b]:indptr[b + 1], h, :] = kb
                v[indptr[b]:indptr[b + 1], h, :] = vb

    tgt_all, drf_all, toks = [], [], []
    for b in range(B):
        tgt, drf = _logits(spec, T, b)
        drf64 = as_f64(drf, spec.ldtype)
        toks.append(_draw_tokens(spec, parents[b], lambda n: drf64[n],
                                 _rng(spec.seed, _TAG_TOK, b)))
        if with_logits:
            tgt_all.append(tgt)
            drf_all.append(drf)
    tokens = np.stack(toks).astype(np.int32)
    target = np.stack(tgt_all) if with_logits else None
    draft = np.stack(drf_all) if with_logits else None
    return Inputs(spec, T, q, k, v, indptr, lens, parents, tokens, target, draft)
