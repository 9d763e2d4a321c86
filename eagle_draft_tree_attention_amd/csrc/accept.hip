// Multi-round speculative sampling over a draft tree, gfx950 (MI355X).
//
// Rule (EAGLE notes page, core mechanism §5 and the multi-round speculative
// sampling term; lesson page, Leviathan rule, residual distribution and bonus
// token): q = softmax(target/t), p = softmax(draft/t).  From the root, the
// children of the current node are tried in ascending index; child c with
// token x is accepted if r < q_res(x) / p(x); on rejection
// q_res <- norm(max(0, q_res - p)) and the next child is tried; when every
// child is rejected the emitted token is drawn from q_res; a node without
// children emits a bonus token drawn from q.  Greedy mode (t == 0) accepts
// the first child whose token is the target argmax, else emits the argmax.
//
// GPU formulation.  Every node's outcome depends only on its own two rows,
// its children's tokens and its own uniforms, so all nodes are decided in
// parallel and the walk is pointer chasing.  The cumulative residual after i
// rejections is kept in closed form, q_res = max(0, q - C_i p) / s_i with
// C_1 = 0, s_1 = 1, C_{i+1} = C_i + s_i, s_{i+1} = sum_v max(0, q - C_{i+1} p),
// so no residual vector is ever stored and the accept test is division free:
// r * s_i * p(x) < max(0, q(x) - C_i p(x)).
//
// Kernels (one pass over HBM for the statistics, later passes touch only
// the few rows that need them):
//   sa_stats  vocab-parallel: per (node, row, 8192-token chunk) max, sum of
//             exp((x - max)/t) (fp64 accumulation) and NaN/+inf detection,
//             or the chunk argmax in greedy mode.  The last workgroup to
//             finish a node (device-scope atomic counter, no waiting) combines
//             the chunks and takes the node's first decision.
//   sa_pass   for nodes that rejected their first child and have more:
//             vocab-parallel residual mass s = sum max(0, q - C p); the last
//             workgroup of the node continues the sibling loop (further
//             rounds, rare, run in that workgroup).
//   sa_final  per sequence: walk the decided nodes from the root, then the
//             inverse-CDF sample of the terminal distribution (chunk masses
//             in parallel, the last workgroup scans the crossing chunk) and
//             the outputs.
// Uniforms: Philox4x32-10 (Salmon et al., SC'11), one per (sequence, node,
// slot); slot = child ordinal for tests, 0xffffffff for the terminal sample.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ev_internal.h"

namespace ev {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr float kNegInf = -__builtin_inff();
constexpr int kThreads = 256;
constexpr int kPerThread = kVocabChunk / kThreads;   // 32 logits per thread per chunk
constexpr double kNearTie = 1e-6;
constexpr uint32_t kSampleSlot = 0xFFFFFFFFu;

// ------------------------------------------------------------------ Philox
__device__ uint32_t philox4x32_10_x0(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                     uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    if (round) {
      k0 += 0x9E3779B9u;   // golden-ratio Weyl increment
      k1 += 0xBB67AE85u;   // sqrt(3) - 1
    }
    const uint64_t prod0 = static_cast<uint64_t>(0xD2511F53u) * c0;
    const uint64_t prod1 = static_cast<uint64_t>(0xCD9E8D57u) * c2;
    const uint32_t y0 = static_cast<uint32_t>(prod1 >> 32) ^ c1 ^ k0;
    const uint32_t y2 = static_cast<uint32_t>(prod0 >> 32) ^ c3 ^ k1;
    c1 = static_cast<uint32_t>(prod1);
    c3 = static_cast<uint32_t>(prod0);
    c0 = y0;
    c2 = y2;
  }
  return c0;
}

__device__ double decision_uniform(const AcceptKernelArgs& a, int b, int node, uint32_t slot) {
  const uint32_t x0 = philox4x32_10_x0(slot, static_cast<uint32_t>(node) | (static_cast<uint32_t>(b) << 8), a.off_lo,
                                       a.off_hi, a.seed_lo, a.seed_hi);
  return static_cast<double>(x0 >> 8) * (1.0 / 16777216.0);
}

// ---------------------------------------------------------- element access
template <typename TL>
__device__ __forceinline__ float logit(const TL* row, int v);
template <>
__device__ __forceinline__ float logit<float>(const float* row, int v) { return row[v]; }
template <>
__device__ __forceinline__ float logit<uint16_t>(const uint16_t* row, int v) {
  return __uint_as_float(static_cast<uint32_t>(row[v]) << 16);
}

// Load this thread's share of a chunk [v0, v1) into x[]; slots past v1 get -inf.
// Element of slot j: vector path v0 + (tid + 256*(j/G))*G + j%G, scalar path v0 + tid + 256*j.
template <typename TL>
__device__ __forceinline__ void load_chunk(const TL* row, int v0, int v1, bool vec, float (&x)[kPerThread],
                                           int (&idx)[kPerThread]) {
  const int tid = threadIdx.x;
  constexpr int G = 16 / sizeof(TL);
  if (vec && ((v1 - v0) % G) == 0) {
#pragma unroll
    for (int j = 0; j < kPerThread / G; ++j) {
      const int base = v0 + (tid + kThreads * j) * G;
      u32x4_t w = u32x4_t{0, 0, 0, 0};
      if (base < v1) w = *reinterpret_cast<const u32x4_t*>(row + base);
#pragma unroll
      for (int e = 0; e < G; ++e) {
        float val;
        if constexpr (sizeof(TL) == 2)
          val = __uint_as_float(((w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu) << 16);
        else
          val = __uint_as_float(w[e]);
        x[j * G + e] = (base < v1) ? val : kNegInf;
        idx[j * G + e] = base + e;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int v = v0 + tid + kThreads * j;
      x[j] = (v < v1) ? logit<TL>(row, v) : kNegInf;
      idx[j] = v;
    }
  }
}

// ------------------------------------------------------ block reductions
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T v, Op op) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = op(v, __shfl_xor(v, o));
  return v;
}

template <typename T, typename Op>
__device__ T block_reduce(T v, Op op, T* scratch /* >= 4 */) {
  v = wave_reduce(v, op);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch[w] = v;
  __syncthreads();
  T r = scratch[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) r = op(r, scratch[i]);
  return r;
}

struct MaxOp {
  __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct AddD {
  __device__ double operator()(double a, double b) const { return a + b; }
};
struct OrU {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a | b; }
};
struct MinI {
  __device__ int operator()(int a, int b) const { return a < b ? a : b; }
};

// ------------------------------------------------------ tree bookkeeping
struct TreeInfo {
  int32_t par[kMaxTree];
  int32_t ok;
};

// Load the parent array of sequence b into LDS and validate it (all threads).
__device__ void load_tree(const AcceptKernelArgs& a, int b, TreeInfo& ti) {
  const int tid = threadIdx.x;
  const int T = a.T;
  if (tid < 64) {
    int p = 0;
    bool good = true;
    if (tid < T) {
      p = a.parents[b * T + tid];
      good = (tid == 0) ? (p == -1) : (p >= 0 && p < tid);
    }
    ti.par[tid] = p;
    const bool all_good = !__any(!good);
    if (tid == 0) ti.ok = all_good ? 1 : 0;
  }
  __syncthreads();
}

__device__ __forceinline__ bool has_children(const TreeInfo& ti, int T, int n) {
  for (int c = n + 1; c < T; ++c)
    if (ti.par[c] == n) return true;
  return false;
}

// k-th child (ascending) of n, or -1
__device__ __forceinline__ int kth_child(const TreeInfo& ti, int T, int n, int k) {
  for (int c = n + 1; c < T; ++c)
    if (ti.par[c] == n && k-- == 0) return c;
  return -1;
}

__device__ __forceinline__ int num_children(const TreeInfo& ti, int T, int n) {
  int k = 0;
  for (int c = n + 1; c < T; ++c) k += (ti.par[c] == n);
  return k;
}

// Arrival at a per-item counter: returns true in the workgroup that arrived
// last (after making every other workgroup's writes visible) and resets the
// counter for the next call.  Must be called by all threads.
__device__ bool arrive_last(uint32_t* counter, uint32_t expected, int32_t* lds_flag) {
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    const uint32_t old = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = (old == expected - 1);
    if (last) {
      __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __threadfence();
    }
    *lds_flag = last ? 1 : 0;
  }
  __syncthreads();
  return *lds_flag != 0;
}

// Test child ordinal i of node n under residual (C, s).  Returns +1 accepted,
// 0 rejected, -1 token out of range (sequence is poisoned later).
template <typename TL>
__device__ int decide_child(const AcceptKernelArgs& a, int b, int n, int child, int ordinal, double C, double s,
                            const NodeState& st, uint32_t& flags, int32_t& near) {
  const int tok = a.tokens[b * a.T + child];
  if (tok < 0 || tok >= a.V) return -1;
  const int64_t row = static_cast<int64_t>(b * a.T + n) * a.V;
  const double xt = logit<TL>(reinterpret_cast<const TL*>(a.target) + row, tok);
  const double yt = logit<TL>(reinterpret_cast<const TL*>(a.draft) + row, tok);
  const double qt = exp((xt - static_cast<double>(st.mq)) * a.inv_tau) / st.zq;
  const double pt = exp((yt - static_cast<double>(st.mp)) * a.inv_tau) / st.zp;
  const double r = decision_uniform(a, b, n, static_cast<uint32_t>(ordinal));
  if (pt == 0.0) {
    flags |= EAGLE_FLAG_P_ZERO;
    return (qt - C * pt) > 0.0 ? 1 : 0;
  }
  const double num = fmax(0.0, qt - C * pt);
  if (fabs(r - num / (s * pt)) < kNearTie) ++near;
  return (r * s * pt < num) ? 1 : 0;
}

// Residual mass sum_v max(0, q_v - C p_v) of node n over [v0, v1), fp64,
// reduced over the block (all threads call; result valid in every thread).
template <typename TL>
__device__ double residual_mass(const AcceptKernelArgs& a, int b, int n, const NodeState& st, double C, int v0,
                                int v1, double* dscratch) {
  const int64_t row = static_cast<int64_t>(b * a.T + n) * a.V;
  const TL* tr = reinterpret_cast<const TL*>(a.target) + row;
  const TL* dr = reinterpret_cast<const TL*>(a.draft) + row;
  const double izq = 1.0 / st.zq, izp = 1.0 / st.zp;
  double acc = 0.0;
  for (int v = v0 + threadIdx.x; v < v1; v += kThreads) {
    const double qv = static_cast<double>(exp2f((logit<TL>(tr, v) - st.mq) * a.c2)) * izq;
    const double pv = static_cast<double>(exp2f((logit<TL>(dr, v) - st.mp) * a.c2)) * izp;
    acc += fmax(0.0, qv - C * pv);
  }
  return block_reduce(acc, AddD{}, dscratch);
}

// Continue the sibling loop of node n from child ordinal i with known (C, s).
// Runs in one workgroup; further residual masses are computed here.
template <typename TL>
__device__ void continue_siblings(const AcceptKernelArgs& a, int b, int n, const TreeInfo& ti, NodeState& st,
                                  int i, double C, double s, double* dscratch, int32_t* iscratch) {
  const int k = num_children(ti, a.T, n);
  for (;;) {
    if (!(s > 0.0)) {          // residual mass vanished: fall back to q
      st.flags |= EAGLE_FLAG_DEGENERATE_RESIDUAL;
      C = 0.0;
      s = 1.0;
    }
    const int child = kth_child(ti, a.T, n, i);
    if (threadIdx.x == 0) {
      uint32_t fl = st.flags;
      int32_t nr = st.near;
      const int res = decide_child<TL>(a, b, n, child, i, C, s, st, fl, nr);
      st.flags = fl;
      st.near = nr;
      iscratch[0] = res;
    }
    __syncthreads();
    const int res = iscratch[0];
    __syncthreads();
    if (res != 0) {
      st.kind = (res > 0) ? kNodeAccepted : kNodeRejected;
      st.outcome = (res > 0) ? child : -1;
      break;
    }
    C += s;
    ++i;
    if (i >= k) {
      st.kind = kNodeRejected;
      st.outcome = -1;
      break;
    }
    s = residual_mass<TL>(a, b, n, st, C, 0, a.V, dscratch);
  }
  st.C = C;
  st.s = s;
  st.next_child = i;
}

// -------------------------------------------------------------- sa_stats
template <typename TL>
__global__ __launch_bounds__(kThreads) void sa_stats(const AcceptKernelArgs a) {
  __shared__ TreeInfo ti;
  __shared__ float fscr[4];
  __shared__ double dscr[4];
  __shared__ uint32_t uscr[4];
  __shared__ int32_t iscr[4];
  __shared__ int32_t last_flag;
  __shared__ NodeState st_lds;

  const int NC = a.NC, T = a.T;
  int item = blockIdx.x;
  const int c = item % NC;
  item /= NC;
  const int row = item % 2;
  item /= 2;
  const int n = item % T;
  const int b = item / T;
  const bool greedy = a.tau == 0.f;
  if (greedy && row == 1) return;

  load_tree(a, b, ti);
  if (!ti.ok) return;
  const bool kids = has_children(ti, T, n);
  if (row == 1 && !kids) return;
  const uint32_t expected = static_cast<uint32_t>(NC) * ((!greedy && kids) ? 2u : 1u);

  const TL* rp = reinterpret_cast<const TL*>(row ? a.draft : a.target) + static_cast<int64_t>(b * T + n) * a.V;
  const int v0 = c * kVocabChunk, v1 = min(a.V, v0 + kVocabChunk);
  float x[kPerThread];
  int idx[kPerThread];
  load_chunk<TL>(rp, v0, v1, a.vec_ok != 0, x, idx);

  float m = kNegInf;
  uint32_t bad = 0;
  int am = 0x7FFFFFFF;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const float v = x[j];
    if (v != v || v == __builtin_inff()) bad = 1;   // NaN or +inf
    if (v > m) m = v;
  }
  m = block_reduce(m, MaxOp{}, fscr);
  bad = block_reduce(bad, OrU{}, uscr);
  ChunkStat cs;
  cs.m = m;
  cs.bad = bad;
  cs.pad = 0;
  cs.z = 0.0;
  cs.argmax = -1;
  if (greedy) {
#pragma unroll
    for (int j = 0; j < kPerThread; ++j)
      if (x[j] == m && idx[j] < am && idx[j] < v1) am = idx[j];
    cs.argmax = block_reduce(am, MinI{}, iscr);
  } else if (m != kNegInf && !bad) {
    double z = 0.0;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) z += static_cast<double>(exp2f((x[j] - m) * a.c2));
    cs.z = block_reduce(z, AddD{}, dscr);
  }
  if (threadIdx.x == 0) a.stats[(static_cast<int64_t>(b * T + n) * 2 + row) * NC + c] = cs;

  if (!arrive_last(&a.cnt_stats[b * T + n], expected, &last_flag)) return;

  // ---- last arrival for node n: combine chunks, first decision
  if (threadIdx.x == 0) {
    NodeState st = {};
    st.outcome = -1;
    st.argmax = -1;
    uint32_t nonfinite = 0;
    for (int r = 0; r < ((!greedy && kids) ? 2 : 1); ++r) {
      const ChunkStat* cp = a.stats + (static_cast<int64_t>(b * T + n) * 2 + r) * NC;
      float M = kNegInf;
      uint32_t rb = 0;
      int arg = -1;
      for (int q = 0; q < NC; ++q) {
        rb |= cp[q].bad;
        if (cp[q].m > M) {
          M = cp[q].m;
          arg = cp[q].argmax;
        }
      }
      double Z = 0.0;
      if (!greedy && M != kNegInf && !rb)
        for (int q = 0; q < NC; ++q)
          if (cp[q].m != kNegInf) Z += cp[q].z * exp2((static_cast<double>(cp[q].m) - M) * static_cast<double>(a.c2));
      if (rb || M == kNegInf) nonfinite = 1;
      if (r == 0) {
        st.mq = M;
        st.zq = Z;
        st.argmax = arg;
      } else {
        st.mp = M;
        st.zp = Z;
      }
    }
    st.flags = nonfinite ? EAGLE_FLAG_NONFINITE : 0u;
    st.C = 0.0;
    st.s = 1.0;
    if (!kids) {
      st.kind = kNodeLeaf;
    } else if (nonfinite) {
      st.kind = kNodeRejected;
    } else if (greedy) {
      st.kind = kNodeRejected;
      for (int ch = n + 1; ch < T; ++ch) {
        if (ti.par[ch] == n && a.tokens[b * T + ch] == st.argmax) {
          st.kind = kNodeAccepted;
          st.outcome = ch;
          break;
        }
      }
    } else {
      const int child = kth_child(ti, T, n, 0);
      uint32_t fl = st.flags;
      int32_t nr = 0;
      const int res = decide_child<TL>(a, b, n, child, 0, 0.0, 1.0, st, fl, nr);
      st.flags = fl;
      st.near = nr;
      if (res > 0) {
        st.kind = kNodeAccepted;
        st.outcome = child;
      } else if (res < 0) {
        st.kind = kNodeRejected;
      } else {
        st.C = 1.0;   // C_2 = C_1 + s_1
        if (num_children(ti, T, n) > 1) {
          st.kind = kNodeNeedsPass;
          st.next_child = 1;
        } else {
          st.kind = kNodeRejected;
          st.next_child = 1;
        }
      }
    }
    a.nodes[b * T + n] = st;
  }
}

// --------------------------------------------------------------- sa_pass
template <typename TL>
__global__ __launch_bounds__(kThreads) void sa_pass(const AcceptKernelArgs a) {
  __shared__ TreeInfo ti;
  __shared__ double dscr[4];
  __shared__ int32_t iscr[4];
  __shared__ int32_t last_flag;
  const int NC = a.NC, T = a.T;
  const int c = blockIdx.x % NC;
  const int n = (blockIdx.x / NC) % T;
  const int b = blockIdx.x / (NC * T);
  NodeState st = a.nodes[b * T + n];
  if (st.kind != kNodeNeedsPass) return;
  const int v0 = c * kVocabChunk, v1 = min(a.V, v0 + kVocabChunk);
  const double part = residual_mass<TL>(a, b, n, st, st.C, v0, v1, dscr);
  if (threadIdx.x == 0) a.fpart[static_cast<int64_t>(b * T + n) * NC + c] = part;
  if (!arrive_last(&a.cnt_pass[b * T + n], static_cast<uint32_t>(NC), &last_flag)) return;
  load_tree(a, b, ti);
  double s = 0.0;
  for (int q = 0; q < NC; ++q) s += a.fpart[static_cast<int64_t>(b * T + n) * NC + q];
  continue_siblings<TL>(a, b, n, ti, st, st.next_child, st.C, s, dscr, iscr);
  if (threadIdx.x == 0) a.nodes[b * T + n] = st;
}

// -------------------------------------------------------------- sa_final
// Terminal weight of token v: q_v (leaf) or max(0, q_v - C p_v).
template <typename TL>
__device__ __forceinline__ double terminal_weight(const TL* tr, const TL* dr, int v, const NodeState& st, double C,
                                                  bool leaf, float c2, double izq, double izp) {
  const double qv = static_cast<double>(exp2f((logit<TL>(tr, v) - st.mq) * c2)) * izq;
  if (leaf || C == 0.0) return qv;
  const double pv = static_cast<double>(exp2f((logit<TL>(dr, v) - st.mp) * c2)) * izp;
  return fmax(0.0, qv - C * pv);
}

template <typename TL>
__global__ __launch_bounds__(kThreads) void sa_final(const AcceptKernelArgs a) {
  __shared__ TreeInfo ti;
  __shared__ double dscr[4];
  __shared__ int32_t iscr[4];
  __shared__ uint32_t uscr[4];
  __shared__ int32_t last_flag;
  __shared__ int32_t path_lds[kMaxTree];
  __shared__ int32_t plen_lds, term_lds;
  __shared__ uint32_t seqflags_lds;
  __shared__ int32_t near_lds;
  __shared__ int32_t found_lds;
  __shared__ double scan_lds[kThreads];

  const bool greedy = a.tau == 0.f;
  const int NC = greedy ? 1 : a.NC, T = a.T;
  const int c = blockIdx.x % NC;
  const int b = blockIdx.x / NC;
  const int tid = threadIdx.x;

  load_tree(a, b, ti);
  // ---- sequence validity (tree, tokens, usable rows)
  uint32_t bad = ti.ok ? 0u : EAGLE_FLAG_BAD_TREE;
  if (!bad) {
    uint32_t tb = 0, nf = 0;
    if (tid < T) {
      if (tid >= 1) {
        const int tok = a.tokens[b * T + tid];
        if (tok < 0 || tok >= a.V) tb = EAGLE_FLAG_BAD_TOKEN;
      }
      nf = a.nodes[b * T + tid].flags & EAGLE_FLAG_NONFINITE;
    }
    bad = block_reduce(tb | nf, OrU{}, uscr);
  }
  if (bad) {
    if (c == 0) {
      if (tid == 0) {
        a.accept_len[b] = -1;
        a.flags[b] = bad;
        a.near_ties[b] = 0;
      }
      for (int j = tid; j < T; j += kThreads) {
        a.accepted_nodes[b * T + j] = -1;
        a.out_tokens[b * T + j] = -1;
      }
    }
    return;
  }
  // ---- walk
  if (tid == 0) {
    int cur = 0, len = 0, near = 0;
    uint32_t fl = 0;
    for (int steps = 0; steps < T; ++steps) {
      const NodeState& s = a.nodes[b * T + cur];
      fl |= s.flags;
      near += s.near;
      if (s.kind != kNodeAccepted || s.outcome <= cur || s.outcome >= T) break;
      path_lds[len++] = s.outcome;
      cur = s.outcome;
    }
    plen_lds = len;
    term_lds = cur;
    seqflags_lds = fl;
    near_lds = near;
  }
  __syncthreads();
  const int len = plen_lds, term = term_lds;

  auto write_outputs = [&](int final_tok, uint32_t extra_flags, int extra_near) {
    if (tid == 0) {
      a.accept_len[b] = len;
      a.flags[b] = seqflags_lds | extra_flags;
      a.near_ties[b] = near_lds + extra_near;
    }
    for (int j = tid; j < T; j += kThreads) {
      a.accepted_nodes[b * T + j] = (j < len) ? path_lds[j] : -1;
      a.out_tokens[b * T + j] = (j < len) ? a.tokens[b * T + path_lds[j]] : (j == len ? final_tok : -1);
    }
  };

  const NodeState st = a.nodes[b * T + term];
  if (greedy) {
    write_outputs(st.argmax, 0u, 0);
    return;
  }

  // ---- terminal distribution: chunk masses
  const bool leaf = (st.kind == kNodeLeaf);
  double C = leaf ? 0.0 : st.C;
  const int64_t rowoff = static_cast<int64_t>(b * T + term) * a.V;
  const TL* tr = reinterpret_cast<const TL*>(a.target) + rowoff;
  const TL* dr = reinterpret_cast<const TL*>(a.draft) + rowoff;
  const double izq = 1.0 / st.zq, izp = leaf ? 0.0 : 1.0 / st.zp;
  {
    const int v0 = c * kVocabChunk, v1 = min(a.V, v0 + kVocabChunk);
    double acc = 0.0;
    for (int v = v0 + tid; v < v1; v += kThreads) acc += terminal_weight<TL>(tr, dr, v, st, C, leaf, a.c2, izq, izp);
    acc = block_reduce(acc, AddD{}, dscr);
    if (tid == 0) a.spart[static_cast<int64_t>(b) * NC + c] = acc;
  }
  if (!arrive_last(&a.cnt_final[b], static_cast<uint32_t>(NC), &last_flag)) return;

  double* sp = a.spart + static_cast<int64_t>(b) * NC;
  double S = 0.0;
  for (int q = 0; q < NC; ++q) S += sp[q];
  uint32_t extra = 0;
  if (!(S > 0.0)) {          // residual mass vanished: sample q instead
    extra |= EAGLE_FLAG_DEGENERATE_RESIDUAL;
    C = 0.0;
    for (int q = 0; q < NC; ++q) {
      const int v0 = q * kVocabChunk, v1 = min(a.V, v0 + kVocabChunk);
      double acc = 0.0;
      for (int v = v0 + tid; v < v1; v += kThreads) acc += terminal_weight<TL>(tr, dr, v, st, C, leaf, a.c2, izq, izp);
      acc = block_reduce(acc, AddD{}, dscr);
      __syncthreads();
      if (tid == 0) sp[q] = acc;
      __syncthreads();
    }
    S = 0.0;
    for (int q = 0; q < NC; ++q) S += sp[q];
  }
  const double u = decision_uniform(a, b, term, kSampleSlot);
  const double thr = u * S;
  int cs = NC - 1;
  double run = 0.0;
  for (int q = 0; q < NC; ++q) {
    if (run + sp[q] > thr) {
      cs = q;
      break;
    }
    if (q < NC - 1) run += sp[q];
  }
  // scan chunk cs: thread t owns kPerThread consecutive tokens
  const int v0 = cs * kVocabChunk, v1 = min(a.V, v0 + kVocabChunk);
  double w[kPerThread];
  double tsum = 0.0;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const int v = v0 + tid * kPerThread + j;
    w[j] = (v < v1) ? terminal_weight<TL>(tr, dr, v, st, C, leaf, a.c2, izq, izp) : 0.0;
    tsum += w[j];
  }
  scan_lds[tid] = tsum;
  if (tid == 0) found_lds = 0x7FFFFFFF;
  __syncthreads();
  if (tid == 0) {   // exclusive prefix over thread totals, in token order
    double acc = run;
    for (int t = 0; t < kThreads; ++t) {
      const double x = scan_lds[t];
      scan_lds[t] = acc;
      acc += x;
    }
  }
  __syncthreads();
  double cum = scan_lds[tid];
  int hit = 0x7FFFFFFF;
  double hit_hi = 0.0, hit_lo = 0.0;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const double before = cum;
    cum += w[j];
    if (hit == 0x7FFFFFFF && cum > thr) {
      hit = v0 + tid * kPerThread + j;
      hit_hi = cum;
      hit_lo = before;
    }
  }
  atomicMin(&found_lds, hit);
  __syncthreads();
  int tok = found_lds;
  int near = 0;
  if (tok != 0x7FFFFFFF) {
    if (hit == tok) {
      near = ((hit_hi - thr) < kNearTie * S || (thr - hit_lo) < kNearTie * S) ? 1 : 0;
      iscr[0] = near;
    }
    __syncthreads();
    near = iscr[0];
  } else {
    // rounding left no crossing: last token of the chunk with positive weight
    int lastpos = -1;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j)
      if (w[j] > 0.0) lastpos = v0 + tid * kPerThread + j;
    __syncthreads();
    if (tid == 0) iscr[1] = -1;
    __syncthreads();
    atomicMax(&iscr[1], lastpos);
    __syncthreads();
    tok = iscr[1];
  }
  write_outputs(tok, extra, near);
}

template <typename TL>
hipError_t launch_t(const AcceptKernelArgs& a, hipStream_t st) {
  const dim3 block(kThreads);
  hipLaunchKernelGGL((sa_stats<TL>), dim3(static_cast<unsigned>(a.B * a.T * 2 * a.NC)), block, 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.tau > 0.f) {
    hipLaunchKernelGGL((sa_pass<TL>), dim3(static_cast<unsigned>(a.B * a.T * a.NC)), block, 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((sa_final<TL>), dim3(static_cast<unsigned>(a.B * a.NC)), block, 0, st, a);
  } else {
    hipLaunchKernelGGL((sa_final<TL>), dim3(static_cast<unsigned>(a.B)), block, 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace

int launch_spec_accept(const AcceptKernelArgs& args, int logits_bf16, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const hipError_t e = logits_bf16 ? launch_t<uint16_t>(args, st) : launch_t<float>(args, st);
  return static_cast<int>(e);
}

}  // namespace ev
