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

#include <type_traits>

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

// ============================================================ fused path
// One launch, B*T*NC workgroups, all co-resident (the host only takes this
// path when the occupancy query says the grid fits).  The NC workgroups of a
// node keep their slice of the node's target and draft exponentials in
// registers from the statistics pass to the end, and coordinate through
// device-scope arrival words (tagged with the call epoch and phase, so they
// never need resetting) and publication words:
//   stats  -> last arrival combines, decides the first child, publishes
//   rounds -> while the node needs another residual mass: partial sums from
//             registers, last arrival takes the next decision, publishes
//   walk   -> a node that ends without an accepted child checks, once its
//             ancestors are decided, whether the walk reaches it
//   sample -> the terminal node's workgroups add up their chunk masses, the
//             last arrival finds the chunk holding u*S, and that workgroup
//             scans its registers in token order and writes the outputs.
// Every wait is bounded by spin_limit; a wait that expires flags the
// sequence EAGLE_FLAG_INTERNAL instead of hanging.

constexpr uint64_t kPubDone = 255;
constexpr int kFusedMaxChunks = 64;   // V <= 64 * 8192 on the fused path

// Cross-workgroup traffic of the fused path.  The L2 caches of the XCDs are
// not coherent with each other, and agent-scope release/acquire would write
// back / invalidate a whole L2 per operation.  Instead every word that one
// workgroup writes for another goes through system-scope relaxed atomics,
// which bypass the non-coherent caches, and ordering comes from waiting for
// the stores to complete (a workgroup-scope release) before signalling.
__device__ __forceinline__ uint64_t ld_u64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ double ld_f64(const double* p) {
  return __builtin_bit_cast(double, ld_u64(reinterpret_cast<const uint64_t*>(p)));
}
__device__ __forceinline__ void st_u64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ void st_f64(double* p, double v) { st_u64(reinterpret_cast<uint64_t*>(p), __builtin_bit_cast(uint64_t, v)); }
// this thread's earlier stores have completed (been acknowledged by the
// coherent memory side) before anything that follows is issued
__device__ __forceinline__ void stores_done() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// later loads are not moved above the poll that allowed them
__device__ __forceinline__ void loads_after() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ void load_state(const NodeState* src, NodeState* dst) {
  const uint64_t* s = reinterpret_cast<const uint64_t*>(src);
  uint64_t* d = reinterpret_cast<uint64_t*>(dst);
#pragma unroll
  for (int i = 0; i < static_cast<int>(sizeof(NodeState) / 8); ++i) d[i] = ld_u64(s + i);
}
__device__ void store_state(NodeState* dst, const NodeState& src) {
  const uint64_t* s = reinterpret_cast<const uint64_t*>(&src);
  uint64_t* d = reinterpret_cast<uint64_t*>(dst);
#pragma unroll
  for (int i = 0; i < static_cast<int>(sizeof(NodeState) / 8); ++i) st_u64(d + i, s[i]);
}

__device__ __forceinline__ void publish(uint64_t* w, uint64_t v) {
  stores_done();
  __hip_atomic_store(w, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

__device__ __forceinline__ uint64_t poll(const uint64_t* w) {
  return __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Every thread t < count waits until w[t] >= target (relaxed polls, one
// acquire when done); block-wide verdict in *ok (all threads call).
__device__ bool wait_all(const uint64_t* w, int count, uint64_t target, uint32_t limit, int32_t* ok) {
  if (threadIdx.x == 0) *ok = 1;
  __syncthreads();
  if (static_cast<int>(threadIdx.x) < count) {
    uint32_t it = 0;
    while (poll(w + threadIdx.x) < target) {
      if (++it > limit) {
        *ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    loads_after();
  }
  __syncthreads();
  return *ok != 0;
}

struct FusedShared {
  TreeInfo ti;
  NodeState st;
  double dscr[4];
  float fscr[4];
  uint32_t uscr[4];
  int32_t iscr[4];
  int32_t flag;
  int32_t ok;
  int32_t onpath;
  uint32_t seqflags;
  int32_t seqnear;
  int32_t found;
  double scan[kThreads / 64];
  double sample[4];
  double mass[2 * kFusedMaxChunks];
};


// One row chunk staged in LDS in token order (index = token - v0); tokens
// past the chunk hold -inf.  Thread t owns the slots j = 0..31 at index
// ((j / G) * 256 + t) * G + j % G, G = 16 / sizeof(TL), so a thread reads
// 16-byte groups and consecutive lanes read consecutive groups.
template <typename TL>
struct ChunkView {
  const TL* lds;
  static constexpr int G = 16 / static_cast<int>(sizeof(TL));
  __device__ __forceinline__ static int index(int j) { return ((j / G) * kThreads + static_cast<int>(threadIdx.x)) * G + (j % G); }
  __device__ __forceinline__ float get(int j) const {
    if constexpr (sizeof(TL) == 2)
      return __uint_as_float(static_cast<uint32_t>(lds[index(j)]) << 16);
    else
      return lds[index(j)];
  }
};

template <typename TL>
__device__ void stage_chunk(const TL* row, int v0, int v1, bool vecpath, TL* lds) {
  const int tid = threadIdx.x;
  constexpr int G = 16 / sizeof(TL);
  if (vecpath) {
#pragma unroll
    for (int jj = 0; jj < kPerThread / G; ++jj) {
      const int i0 = (jj * kThreads + tid) * G;
      u32x4_t w;
      if (v0 + i0 < v1) {
        w = *reinterpret_cast<const u32x4_t*>(row + v0 + i0);
      } else {
        const uint32_t ni = sizeof(TL) == 2 ? 0xFF80FF80u : 0xFF800000u;
        w = u32x4_t{ni, ni, ni, ni};
      }
      *reinterpret_cast<u32x4_t*>(lds + i0) = w;
    }
  } else {
    for (int i = tid; i < kVocabChunk; i += kThreads) {
      const float x = (v0 + i < v1) ? logit<TL>(row, v0 + i) : kNegInf;
      if constexpr (sizeof(TL) == 2)
        lds[i] = static_cast<TL>(__float_as_uint(x) >> 16);
      else
        lds[i] = x;
    }
  }
}

// Chunk statistics of one row: block max m, NaN/+inf flag, chunk argmax
// (greedy mode) or sum of exp((x - m)/tau) (fp64).
template <typename TL>
__device__ void chunk_stats(const ChunkView<TL>& r, int v0, int v1, const AcceptKernelArgs& a, bool greedy,
                            float& m, uint32_t& bad, int& am, double& z, FusedShared& sh) {
  float lm = kNegInf;
  uint32_t lb = 0;
#pragma unroll 4
  for (int j = 0; j < kPerThread; ++j) {
    const float v = r.get(j);
    if (v != v || v == __builtin_inff()) lb = 1;
    lm = fmaxf(lm, v);
  }
  m = block_reduce(lm, MaxOp{}, sh.fscr);
  bad = block_reduce(lb, OrU{}, sh.uscr);
  am = -1;
  z = 0.0;
  if (greedy) {
    int la = 0x7FFFFFFF;
#pragma unroll 4
    for (int j = 0; j < kPerThread; ++j) {
      const int t = v0 + ChunkView<TL>::index(j);
      if (r.get(j) == m && t < v1 && t < la) la = t;
    }
    am = block_reduce(la, MinI{}, sh.iscr);
    return;
  }
  double lz = 0.0;
  if (m != kNegInf && !bad) {
#pragma unroll 4
    for (int j = 0; j < kPerThread; ++j) lz += static_cast<double>(exp2f((r.get(j) - m) * a.c2));
  }
  z = block_reduce(lz, AddD{}, sh.dscr);
}

__device__ void write_poison(const AcceptKernelArgs& a, int b, uint32_t flags) {
  const int T = a.T;
  if (threadIdx.x == 0) {
    a.accept_len[b] = -1;
    a.flags[b] = flags;
    a.near_ties[b] = 0;
  }
  for (int j = threadIdx.x; j < T; j += kThreads) {
    a.accepted_nodes[b * T + j] = -1;
    a.out_tokens[b * T + j] = -1;
  }
}

// Root path of node n (root first) in ti.par order; returns its length.
__device__ int root_path(const TreeInfo& ti, int n, int* path) {
  int len = 0;
  for (int x = n; x >= 0; x = ti.par[x]) ++len;
  int i = len;
  for (int x = n; x >= 0; x = ti.par[x]) path[--i] = x;
  return len;
}

// Arrive at a phase counter shared by `group` workgroups and wait until all
// of them have arrived (thread 0).  The counter only grows: each phase adds
// `group`.  This workgroup's results were stored before the arrival.
__device__ bool phase_barrier(uint64_t* w, uint32_t group, uint32_t limit) {
  stores_done();
  const uint64_t old = __hip_atomic_fetch_add(w, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  const uint64_t target = (old / group + 1) * group;
  uint32_t it = 0;
  while (poll(w) < target) {
    if (++it > limit) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  loads_after();
  return true;
}

template <typename TL>
__global__ __launch_bounds__(kThreads, 4) void sa_fused(const AcceptKernelArgs a) {
  __shared__ FusedShared sh;
  __shared__ int32_t path_lds[kMaxTree];
  __shared__ __attribute__((aligned(16))) TL lq[kVocabChunk];
  __shared__ __attribute__((aligned(16))) TL lp[kVocabChunk];
  const int NC = a.NC, T = a.T, V = a.V, tid = threadIdx.x;
  const int c = blockIdx.x % NC;
  const int n = (blockIdx.x / NC) % T;
  const int b = blockIdx.x / (NC * T);
  const bool greedy = a.tau == 0.f;
  const uint64_t base = a.epoch << 8;
  uint64_t* npub = a.node_pub + static_cast<int64_t>(b) * T;
  uint64_t* narr = a.node_arrive + static_cast<int64_t>(b) * T;
  const uint32_t limit = a.spin_limit;
  const bool lead = (c == 0);   // publishes the node's state for the other nodes' groups

  auto fail_internal = [&]() {
    if (tid == 0) atomicOr(&a.flags[b], EAGLE_FLAG_INTERNAL);
  };

  // ---- sequence validity, the same verdict in every workgroup of b
  load_tree(a, b, sh.ti);
  if (tid < 64) {
    bool tb = false;
    if (tid >= 1 && tid < T) {
      const int tok = a.tokens[b * T + tid];
      tb = tok < 0 || tok >= V;
    }
    const bool any_tb = __any(tb);
    if (tid == 0) sh.uscr[0] = any_tb ? EAGLE_FLAG_BAD_TOKEN : 0u;
  }
  __syncthreads();
  if (!sh.ti.ok) {
    if (n == 0 && c == 0) write_poison(a, b, EAGLE_FLAG_BAD_TREE);
    return;
  }
  // a token outside the vocabulary poisons the sequence too, but the row
  // checks still run so that every unusable input is reported
  const uint32_t tokbad = sh.uscr[0];
  __syncthreads();
  const bool kids = has_children(sh.ti, T, n);
  const bool two = kids && !greedy;
  const int v0 = c * kVocabChunk, v1 = min(V, v0 + kVocabChunk);
  constexpr int G = 16 / sizeof(TL);
  const bool vecpath = a.vec_ok != 0 && ((v1 - v0) % G) == 0;

  // ---- statistics pass: the chunk goes to LDS once and stays there
  const int64_t rowoff = static_cast<int64_t>(b * T + n) * V;
  stage_chunk<TL>(reinterpret_cast<const TL*>(a.target) + rowoff, v0, v1, vecpath, lq);
  if (two) stage_chunk<TL>(reinterpret_cast<const TL*>(a.draft) + rowoff, v0, v1, vecpath, lp);
  __syncthreads();
  const ChunkView<TL> rq{lq}, rp{lp};
  float mq_c, mp_c = kNegInf;
  uint32_t badq, badp = 0;
  int amq, amp;
  double zq_c, zp_c = 0.0;
  chunk_stats<TL>(rq, v0, v1, a, greedy, mq_c, badq, amq, zq_c, sh);
  if (two) chunk_stats<TL>(rp, v0, v1, a, false, mp_c, badp, amp, zp_c, sh);
  ChunkStat* cs = a.stats + (static_cast<int64_t>(b * T + n) * 2) * NC;
  if (tid == 0) {
    auto put = [](ChunkStat* d, float m, uint32_t bad, int am, double z) {
      uint64_t* w = reinterpret_cast<uint64_t*>(d);
      st_u64(w, static_cast<uint64_t>(__float_as_uint(m)) | (static_cast<uint64_t>(bad) << 32));
      st_u64(w + 1, static_cast<uint64_t>(static_cast<uint32_t>(am)));
      st_f64(&d->z, z);
    };
    put(cs + c, mq_c, badq, amq, zq_c);
    if (two) put(cs + NC + c, mp_c, badp, -1, zp_c);
    sh.ok = phase_barrier(narr + n, static_cast<uint32_t>(NC), limit) ? 1 : 0;
  }
  __syncthreads();
  if (!sh.ok) return fail_internal();

  // ---- every workgroup of the node combines the chunks (same arithmetic in
  // the same order everywhere, so all of them hold the same node state)
  if (tid < 64) {
    for (int r = 0; r < (two ? 2 : 1); ++r) {
      const ChunkStat* rs = cs + r * NC;
      float M = kNegInf;
      uint32_t rb = 0;
      for (int q = tid; q < NC; q += 64) {
        const uint64_t w0 = ld_u64(reinterpret_cast<const uint64_t*>(rs + q));
        M = fmaxf(M, __builtin_bit_cast(float, static_cast<uint32_t>(w0)));
        rb |= static_cast<uint32_t>(w0 >> 32);
      }
      M = wave_reduce(M, MaxOp{});
      rb = wave_reduce(rb, OrU{});
      double Z = 0.0;
      int arg = 0x7FFFFFFF;
      for (int q = tid; q < NC; q += 64) {
        const uint64_t w0 = ld_u64(reinterpret_cast<const uint64_t*>(rs + q));
        const float mq = __builtin_bit_cast(float, static_cast<uint32_t>(w0));
        if (greedy) {
          const int aq = static_cast<int>(static_cast<uint32_t>(ld_u64(reinterpret_cast<const uint64_t*>(rs + q) + 1)));
          if (mq == M && aq < arg) arg = aq;
        } else if (mq != kNegInf) {
          Z += ld_f64(&rs[q].z) * exp2((static_cast<double>(mq) - M) * static_cast<double>(a.c2));
        }
      }
      Z = wave_reduce(Z, AddD{});
      arg = wave_reduce(arg, MinI{});
      if (tid == 0) {
        if (r == 0) {
          sh.st.mq = M;
          sh.st.zq = Z;
          sh.st.argmax = arg;
          sh.st.flags = (rb || M == kNegInf) ? EAGLE_FLAG_NONFINITE : 0u;
        } else {
          sh.st.mp = M;
          sh.st.zp = Z;
          if (rb || M == kNegInf) sh.st.flags |= EAGLE_FLAG_NONFINITE;
        }
      }
    }
  }
  __syncthreads();
  // ---- first decision (thread 0, identical in every workgroup of the node)
  if (tid == 0) {
    NodeState st = sh.st;
    if (!two) {
      st.mp = 0.f;
      st.zp = 1.0;
    }
    st.C = 0.0;
    st.s = 1.0;
    st.outcome = -1;
    st.next_child = 0;
    st.near = 0;
    if (!kids) {
      st.kind = kNodeLeaf;
    } else if (st.flags & EAGLE_FLAG_NONFINITE) {
      st.kind = kNodeRejected;
    } else if (greedy) {
      st.kind = kNodeRejected;
      for (int ch = n + 1; ch < T; ++ch)
        if (sh.ti.par[ch] == n && a.tokens[b * T + ch] == st.argmax) {
          st.kind = kNodeAccepted;
          st.outcome = ch;
          break;
        }
    } else {
      const int child = kth_child(sh.ti, T, n, 0);
      uint32_t fl = st.flags;
      int32_t nr = 0;
      const int res = decide_child<TL>(a, b, n, child, 0, 0.0, 1.0, st, fl, nr);
      st.flags = fl;
      st.near = nr;
      if (res > 0) {
        st.kind = kNodeAccepted;
        st.outcome = child;
      } else {
        st.C = 1.0;
        st.next_child = 1;
        st.kind = (res == 0 && num_children(sh.ti, T, n) > 1) ? kNodeNeedsPass : kNodeRejected;
      }
    }
    sh.st = st;
    if (lead) {
      store_state(&a.nodes[b * T + n], st);
      publish(npub + n, base + (st.kind == kNodeNeedsPass ? 1u : kPubDone));
    }
  }
  __syncthreads();

  // ---- residual-mass rounds from LDS; partials double-buffered by round
  const bool q_live = mq_c != kNegInf, p_live = two && mp_c != kNegInf;
  const double fq = q_live ? exp2((static_cast<double>(mq_c) - sh.st.mq) * static_cast<double>(a.c2)) / sh.st.zq : 0.0;
  const double fp = p_live ? exp2((static_cast<double>(mp_c) - sh.st.mp) * static_cast<double>(a.c2)) / sh.st.zp : 0.0;
  // normalised probabilities of slot j (fp64)
  auto qv = [&](int j) -> double {
    return q_live ? static_cast<double>(exp2f((rq.get(j) - mq_c) * a.c2)) * fq : 0.0;
  };
  auto pv = [&](int j) -> double {
    return p_live ? static_cast<double>(exp2f((rp.get(j) - mp_c) * a.c2)) * fp : 0.0;
  };
  int round = 0;
  while (sh.st.kind == kNodeNeedsPass) {
    const double C = sh.st.C;
    double part = 0.0;
#pragma unroll 4
    for (int j = 0; j < kPerThread; ++j) part += fmax(0.0, qv(j) - C * pv(j));
    part = block_reduce(part, AddD{}, sh.dscr);
    double* fbuf = a.fpart + (static_cast<int64_t>(round & 1) * a.B * T + b * T + n) * NC;
    if (tid == 0) {
      st_f64(fbuf + c, part);
      sh.ok = phase_barrier(narr + n, static_cast<uint32_t>(NC), limit) ? 1 : 0;
    }
    __syncthreads();
    if (!sh.ok) return fail_internal();
    double s = 0.0;
    if (tid < 64) {
      for (int q = tid; q < NC; q += 64) s += ld_f64(fbuf + q);
      s = wave_reduce(s, AddD{});
    }
    if (tid == 0) {
      NodeState st = sh.st;
      const int k = num_children(sh.ti, T, n);
      int i = st.next_child;
      double Cn = st.C;
      if (!(s > 0.0)) {
        st.flags |= EAGLE_FLAG_DEGENERATE_RESIDUAL;
        Cn = 0.0;
        s = 1.0;
      }
      const int child = kth_child(sh.ti, T, n, i);
      uint32_t fl = st.flags;
      int32_t nr = st.near;
      const int res = decide_child<TL>(a, b, n, child, i, Cn, s, st, fl, nr);
      st.flags = fl;
      st.near = nr;
      if (res > 0) {
        st.kind = kNodeAccepted;
        st.outcome = child;
      } else {
        Cn += s;
        ++i;
        st.kind = (res == 0 && i < k) ? kNodeNeedsPass : kNodeRejected;
      }
      st.C = Cn;
      st.s = s;
      st.next_child = i;
      sh.st = st;
      if (lead && st.kind != kNodeNeedsPass) {
        store_state(&a.nodes[b * T + n], st);
        publish(npub + n, base + kPubDone);
      }
    }
    __syncthreads();
    ++round;
  }

  // ---- is this node where the walk ends?
  const bool poison_writer = (n == 0 && c == 0);
  if (sh.st.kind == kNodeAccepted && !poison_writer) return;
  // every node's statistics must be known (an unusable row poisons the sequence)
  if (tid == 0) sh.seqflags = tokbad;
  wait_all(npub, T, base + 1, limit, &sh.ok);
  if (sh.ok && tid < T) {
    const uint32_t f = static_cast<uint32_t>(ld_u64(reinterpret_cast<const uint64_t*>(&a.nodes[b * T + tid].flags)));
    if (f & EAGLE_FLAG_NONFINITE) atomicOr(&sh.seqflags, EAGLE_FLAG_NONFINITE);
  }
  __syncthreads();
  if (!sh.ok) return fail_internal();
  if (sh.seqflags) {
    if (poison_writer) write_poison(a, b, sh.seqflags);
    return;
  }
  if (sh.st.kind == kNodeAccepted) return;
  // on the walk iff every ancestor accepted the next node of this root path
  if (tid == 0) {
    sh.iscr[0] = root_path(sh.ti, n, path_lds);
    sh.onpath = 1;
    sh.ok = 1;
  }
  __syncthreads();
  const int plen = sh.iscr[0];
  if (tid < plen - 1) {
    const int anc = path_lds[tid];
    uint32_t it = 0;
    while (poll(npub + anc) < base + kPubDone) {
      if (++it > limit) {
        sh.ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    loads_after();
    if (sh.ok) {
      const uint64_t w = ld_u64(reinterpret_cast<const uint64_t*>(&a.nodes[b * T + anc].kind));
      const int kind = static_cast<int>(static_cast<uint32_t>(w));
      const int outc = static_cast<int>(static_cast<uint32_t>(w >> 32));
      if (kind != kNodeAccepted || outc != path_lds[tid + 1]) sh.onpath = 0;
    }
  }
  __syncthreads();
  if (!sh.ok) return fail_internal();
  if (!sh.onpath) return;
  const int len = plen - 1;   // accepted draft nodes

  // flags and near ties along the path (ancestors from memory, this node from LDS)
  if (tid == 0) {
    sh.seqflags = sh.st.flags;
    sh.seqnear = sh.st.near;
  }
  __syncthreads();
  if (tid < plen - 1) {
    const uint64_t w = ld_u64(reinterpret_cast<const uint64_t*>(&a.nodes[b * T + path_lds[tid]].flags));
    atomicOr(&sh.seqflags, static_cast<uint32_t>(w));
    atomicAdd(&sh.seqnear, static_cast<int32_t>(static_cast<uint32_t>(w >> 32)));
  }
  __syncthreads();

  auto write_outputs = [&](int final_tok, uint32_t extra_flags, int extra_near) {
    if (tid == 0) {
      a.accept_len[b] = len;
      a.flags[b] = sh.seqflags | extra_flags;
      a.near_ties[b] = sh.seqnear + extra_near;
    }
    for (int j = tid; j < T; j += kThreads) {
      a.accepted_nodes[b * T + j] = (j < len) ? path_lds[j + 1] : -1;
      a.out_tokens[b * T + j] = (j < len) ? a.tokens[b * T + path_lds[j + 1]] : (j == len ? final_tok : -1);
    }
  };

  if (greedy) {
    if (c == 0) write_outputs(sh.st.argmax, 0u, 0);
    return;
  }

  // ---- terminal sample: chunk masses of the residual (and of q, used if the
  // residual mass turns out to be zero)
  const bool leaf = (sh.st.kind == kNodeLeaf);
  const double Ct = leaf ? 0.0 : sh.st.C;
  double mres = 0.0, mqs = 0.0;
#pragma unroll 4
  for (int j = 0; j < kPerThread; ++j) {
    const double q = qv(j);
    mqs += q;
    mres += leaf ? q : fmax(0.0, q - Ct * pv(j));
  }
  mres = block_reduce(mres, AddD{}, sh.dscr);
  mqs = block_reduce(mqs, AddD{}, sh.dscr);
  if (tid == 0) {
    st_f64(&a.spart[(static_cast<int64_t>(b) * NC + c) * 2], mres);
    st_f64(&a.spart[(static_cast<int64_t>(b) * NC + c) * 2 + 1], mqs);
    sh.ok = phase_barrier(a.seq_arrive + b, static_cast<uint32_t>(NC), limit) ? 1 : 0;
  }
  __syncthreads();
  if (!sh.ok) return fail_internal();
  // every terminal workgroup: the chunk holding u * S (chunk order, same
  // arithmetic everywhere)
  for (int q = tid; q < NC; q += kThreads) {
    sh.mass[2 * q] = ld_f64(&a.spart[(static_cast<int64_t>(b) * NC + q) * 2]);
    sh.mass[2 * q + 1] = ld_f64(&a.spart[(static_cast<int64_t>(b) * NC + q) * 2 + 1]);
  }
  __syncthreads();
  if (tid == 0) {
    double sr = 0.0;
    for (int q = 0; q < NC; ++q) sr += sh.mass[2 * q];
    const bool degen = !(sr > 0.0);
    const int col = degen ? 1 : 0;
    double S = 0.0;
    for (int q = 0; q < NC; ++q) S += sh.mass[2 * q + col];
    const double u = decision_uniform(a, b, n, kSampleSlot);
    const double thr = u * S;
    int cstar = -1;
    double run = 0.0;
    for (int q = 0; q < NC; ++q) {
      if (run + sh.mass[2 * q + col] > thr) {
        cstar = q;
        break;
      }
      run += sh.mass[2 * q + col];
    }
    if (cstar < 0) {     // rounding: the last chunk with positive mass
      run = 0.0;
      for (int q = 0; q < NC; ++q)
        if (sh.mass[2 * q + col] > 0.0) cstar = q;
      for (int q = 0; q < cstar; ++q) run += sh.mass[2 * q + col];
    }
    sh.sample[0] = run;
    sh.sample[1] = S;
    sh.sample[2] = thr;
    sh.iscr[3] = cstar | (degen ? 0x40000000 : 0);
  }
  __syncthreads();
  const int cstar = sh.iscr[3] & 0x3FFFFFFF;
  const bool degen = (sh.iscr[3] & 0x40000000) != 0;
  if (c != cstar) return;
  const double S = sh.sample[1], thr = sh.sample[2];
  double run = sh.sample[0];

  // ---- scan this chunk's weights in token order, from registers
  auto weight = [&](int j) -> double {
    const double q = qv(j);
    return (leaf || degen) ? q : fmax(0.0, q - Ct * pv(j));
  };
  if (tid == 0) sh.found = 0x7FFFFFFF;
  int hit = 0x7FFFFFFF;
  double hit_hi = 0.0, hit_lo = 0.0;
  // token order = (group jj, thread, element e), G tokens per group
  {
    constexpr int GG = ChunkView<TL>::G;
    for (int jj = 0; jj < kPerThread / GG; ++jj) {
      double gs = 0.0;
#pragma unroll
      for (int e = 0; e < GG; ++e) gs += weight(jj * GG + e);
      double incl = gs;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const double y = __shfl_up(incl, o);
        if ((tid & 63) >= o) incl += y;
      }
      __syncthreads();
      if ((tid & 63) == 63) sh.scan[tid >> 6] = incl;
      __syncthreads();
      double wave_off = 0.0, total = 0.0;
#pragma unroll
      for (int wv = 0; wv < kThreads / 64; ++wv) {
        if (wv < (tid >> 6)) wave_off += sh.scan[wv];
        total += sh.scan[wv];
      }
      double cum = run + wave_off + incl - gs;
#pragma unroll
      for (int e = 0; e < GG; ++e) {
        const double before = cum;
        cum += weight(jj * GG + e);
        if (hit == 0x7FFFFFFF && cum > thr) {
          hit = v0 + ChunkView<TL>::index(jj * GG + e);
          hit_hi = cum;
          hit_lo = before;
        }
      }
      run += total;
    }
  }
  atomicMin(&sh.found, hit);
  __syncthreads();
  int tok = sh.found;
  int near = 0;
  if (tok != 0x7FFFFFFF) {
    if (hit == tok) sh.iscr[1] = ((hit_hi - thr) < kNearTie * S || (thr - hit_lo) < kNearTie * S) ? 1 : 0;
    __syncthreads();
    near = sh.iscr[1];
  } else {
    // rounding left no crossing: the last token of the chunk with positive weight
    int lastpos = -1;
#pragma unroll 4
    for (int j = 0; j < kPerThread; ++j) {
      const int t = v0 + ChunkView<TL>::index(j);
      if (t < v1 && weight(j) > 0.0 && t > lastpos) lastpos = t;
    }
    if (tid == 0) sh.iscr[2] = -1;
    __syncthreads();
    atomicMax(&sh.iscr[2], lastpos);
    __syncthreads();
    tok = sh.iscr[2];
  }
  write_outputs(tok, degen ? EAGLE_FLAG_DEGENERATE_RESIDUAL : 0u, near);
}

template <typename TL>
hipError_t launch_t(const AcceptKernelArgs& a, hipStream_t st) {
  const dim3 block(kThreads);
  if (a.fused) {
    hipLaunchKernelGGL((sa_fused<TL>), dim3(static_cast<unsigned>(a.B * a.T * a.NC)), block, 0, st, a);
    return hipGetLastError();
  }
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

int fused_accept_capacity(int logits_bf16, int num_cus) {
  int per_cu = 0;
  (void)kFusedMaxChunks;
  const hipError_t e = logits_bf16
      ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(&sa_fused<uint16_t>), kThreads, 0)
      : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(&sa_fused<float>), kThreads, 0);
  if (e != hipSuccess || per_cu <= 0) return 0;
  return per_cu * num_cus;
}

int launch_spec_accept(const AcceptKernelArgs& args, int logits_bf16, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const hipError_t e = logits_bf16 ? launch_t<uint16_t>(args, st) : launch_t<float>(args, st);
  return static_cast<int>(e);
}

}  // namespace ev
