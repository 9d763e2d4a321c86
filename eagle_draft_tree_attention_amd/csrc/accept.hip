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

#include "ev_device.h"
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
  const uint32_t x0 = philox4x32_10_x0(slot, static_cast<uint32_t>(node) | (static_cast<uint32_t>(a.b0 + b) << 8), a.off_lo,
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

// Filtered distributions (top-k / top-p): logits below their row's
// keep-threshold count as -inf.  NaN and +inf pass unchanged, so that an
// unusable row is still reported.
__device__ __forceinline__ float thr_of(const AcceptKernelArgs& a, int b, int n, int r) {
  return a.thr ? a.thr[(static_cast<int64_t>(b) * a.T + n) * 2 + r] : kNegInf;
}
__device__ __forceinline__ float cut(float x, float th) { return x < th ? kNegInf : x; }
// near ties of the filter boundaries of node n's rows (the draft row only
// when the node tests children)
__device__ __forceinline__ int32_t filter_near(const AcceptKernelArgs& a, int b, int n, bool draft_used) {
  if (!a.thr) return 0;
  const int64_t i = (static_cast<int64_t>(b) * a.T + n) * 2;
  return a.thr_near[i] + (draft_used ? a.thr_near[i + 1] : 0);
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
// Lane-to-lane moves for reductions: DPP row rotations (16-lane rows) move
// a 32- or 64-bit value between the lanes of a row without going through
// LDS, and readlane takes a row's value into a scalar register.
template <int CTRL, typename T>
__device__ __forceinline__ T dpp_move(T v) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit values");
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
  } else {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(u)), CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(u >> 32)), CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(T, static_cast<uint64_t>(static_cast<uint32_t>(lo)) | (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32));
  }
}
template <typename T>
__device__ __forceinline__ T read_lane(T v, int l) {
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
  } else {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(u)), l));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(u >> 32)), l));
    return __builtin_bit_cast(T, static_cast<uint64_t>(lo) | (static_cast<uint64_t>(hi) << 32));
  }
}

// Moves whose source may lie outside the row (or the enabled rows): such
// lanes receive 0, the identity of the sums below.
template <int CTRL, int ROWS, typename T>
__device__ __forceinline__ T dpp_shift(T v) {
  static_assert(sizeof(T) == 8, "64-bit values");
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(u)), CTRL, ROWS, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(u >> 32)), CTRL, ROWS, 0xF, false);
  return __builtin_bit_cast(T, static_cast<uint64_t>(static_cast<uint32_t>(lo)) | (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32));
}
// Inclusive prefix sum over the 64 lanes of a wave (every lane active):
// log-step sums inside each 16-lane row, then the row totals are carried
// forward by row broadcasts.
__device__ __forceinline__ double wave_scan_add(double v) {
  v += dpp_shift<0x111, 0xF>(v);   // row_shr:1
  v += dpp_shift<0x112, 0xF>(v);   // row_shr:2
  v += dpp_shift<0x114, 0xF>(v);   // row_shr:4
  v += dpp_shift<0x118, 0xF>(v);   // row_shr:8
  v += dpp_shift<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
  v += dpp_shift<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
  return v;
}
// the value of the previous lane (0 in lane 0)
__device__ __forceinline__ double wave_prev(double v) { return dpp_shift<0x138, 0xF>(v); }   // wave_shr:1

// Reduction over the 64 lanes of a wave (every lane active); the result is
// the same in every lane and is combined in one fixed order.
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T v, Op op) {
  v = op(v, dpp_move<0x128>(v));   // row_ror:8
  v = op(v, dpp_move<0x124>(v));   // row_ror:4
  v = op(v, dpp_move<0x122>(v));   // row_ror:2
  v = op(v, dpp_move<0x121>(v));   // row_ror:1 -> every lane holds its row's result
  return op(op(read_lane(v, 0), read_lane(v, 16)), op(read_lane(v, 32), read_lane(v, 48)));
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
  int32_t nreal;   // rows before the padding suffix (token -1): the tree proper
};

// Padding rows (token -1 at a row >= 1) let trees of different sizes share a
// batch; they must form a suffix of the rows.  Returns the number of rows
// before it, or -1 when the padding rows are not a suffix.  Called by a whole
// wave with `pad` set for the padding rows among lanes 0 .. T-1.
__device__ __forceinline__ int real_rows(bool pad, int T) {
  const uint64_t pm = __ballot(pad);
  if (pm == 0ull) return T;
  const int nreal = __builtin_ctzll(pm);   // <= 63 here
  const uint64_t rows = T >= 64 ? ~0ull : ((1ull << T) - 1ull);
  return pm == (rows & ~((1ull << nreal) - 1ull)) ? nreal : -1;
}

// Load the parent array of sequence b into LDS and validate it (all threads).
__device__ void load_tree(const AcceptKernelArgs& a, int b, TreeInfo& ti) {
  const int tid = threadIdx.x;
  const int T = a.T;
  if (tid < 64) {
    int p = 0;
    bool good = true, pad = false;
    if (tid < T) {
      p = a.parents[b * T + tid];
      good = (tid == 0) ? (p == -1) : (p >= 0 && p < tid);
      pad = tid >= 1 && a.tokens[b * T + tid] == -1;
    }
    ti.par[tid] = p;
    const int nreal = real_rows(pad, T);
    const bool all_good = !__any(!good) && nreal >= 1;
    if (tid == 0) {
      ti.ok = all_good ? 1 : 0;
      ti.nreal = nreal;
    }
  }
  __syncthreads();
}

// children are rows of the tree proper (padding rows are never children)
__device__ __forceinline__ bool has_children(const TreeInfo& ti, int T, int n) {
  for (int c = n + 1; c < min(T, ti.nreal); ++c)
    if (ti.par[c] == n) return true;
  return false;
}

// k-th child (ascending) of n, or -1
__device__ __forceinline__ int kth_child(const TreeInfo& ti, int T, int n, int k) {
  for (int c = n + 1; c < min(T, ti.nreal); ++c)
    if (ti.par[c] == n && k-- == 0) return c;
  return -1;
}

__device__ __forceinline__ int num_children(const TreeInfo& ti, int T, int n) {
  int k = 0;
  for (int c = n + 1; c < min(T, ti.nreal); ++c) k += (ti.par[c] == n);
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

// Accept test of one child under residual (C, s): q(t), p(t) at its token
// and the test's uniform r.  Returns +1 accepted, 0 rejected, -1 token out of
// range (the sequence is poisoned later).
__device__ int decide_pre(double qt, double pt, double r, int tok, int V, double C, double s, uint32_t& flags,
                          int32_t& near) {
  if (tok < 0 || tok >= V) return -1;
  if (pt == 0.0) {
    flags |= EAGLE_FLAG_P_ZERO;
    return (qt - C * pt) > 0.0 ? 1 : 0;
  }
  const double num = fmax(0.0, qt - C * pt);
  if (fabs(r - num / (s * pt)) < kNearTie) ++near;
  return (r * s * pt < num) ? 1 : 0;
}

// The same test from the raw logits xt / yt of the node's target / draft rows
// at the child's token (child ordinal i draws slot i).
__device__ int decide_values(const AcceptKernelArgs& a, int b, int n, int ordinal, int tok, double xt, double yt,
                             double C, double s, const NodeState& st, uint32_t& flags, int32_t& near) {
  if (tok < 0 || tok >= a.V) return -1;
  const double qt = exp((xt - static_cast<double>(st.mq)) * a.inv_tau) / st.zq;
  const double pt = exp((yt - static_cast<double>(st.mp)) * a.inv_tau) / st.zp;
  const double r = decision_uniform(a, b, n, static_cast<uint32_t>(ordinal));
  return decide_pre(qt, pt, r, tok, a.V, C, s, flags, near);
}

template <typename TL>
__device__ int decide_child(const AcceptKernelArgs& a, int b, int n, int child, int ordinal, double C, double s,
                            const NodeState& st, uint32_t& flags, int32_t& near) {
  const int tok = a.tokens[b * a.T + child];
  if (tok < 0 || tok >= a.V) return -1;
  const int64_t row = static_cast<int64_t>(b * a.T + n) * a.V;
  const double xt = cut(logit<TL>(reinterpret_cast<const TL*>(a.target) + row, tok), thr_of(a, b, n, 0));
  const double yt = cut(logit<TL>(reinterpret_cast<const TL*>(a.draft) + row, tok), thr_of(a, b, n, 1));
  return decide_values(a, b, n, ordinal, tok, xt, yt, C, s, st, flags, near);
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
  const float thq = thr_of(a, b, n, 0), thp = thr_of(a, b, n, 1);
  double acc = 0.0;
  for (int v = v0 + threadIdx.x; v < v1; v += kThreads) {
    const double qv = static_cast<double>(exp2f((cut(logit<TL>(tr, v), thq) - st.mq) * a.c2)) * izq;
    const double pv = static_cast<double>(exp2f((cut(logit<TL>(dr, v), thp) - st.mp) * a.c2)) * izp;
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

// q(t), p(t) of a child's token at node n, from the raw logits (the same
// arithmetic as decide_values)
template <typename TL>
__device__ void child_qp(const AcceptKernelArgs& a, int b, int n, int tok, const NodeState& st, double& qt,
                         double& pt) {
  const int64_t row = static_cast<int64_t>(b * a.T + n) * a.V;
  const double xt = cut(logit<TL>(reinterpret_cast<const TL*>(a.target) + row, tok), thr_of(a, b, n, 0));
  const double yt = cut(logit<TL>(reinterpret_cast<const TL*>(a.draft) + row, tok), thr_of(a, b, n, 1));
  qt = exp((xt - static_cast<double>(st.mq)) * a.inv_tau) / st.zq;
  pt = exp((yt - static_cast<double>(st.mp)) * a.inv_tau) / st.zp;
}

// Siblings drawn without replacement, on the three-kernel path: sibling i is
// tested against the draft without the earlier siblings' tokens,
// renormalised by the mass Z left; rejecting it moves the untried tokens'
// residual to C + s / Z, and its own token keeps the weight max(0, q(t) -
// C p(t)) at that new C for good (the later siblings' draft puts no mass on
// it).  A round's mass is the full-vocabulary sum at C with the tried
// tokens' terms replaced by their kept weights.
struct WrLds {
  int32_t tok[kMaxTree];
  double qt[kMaxTree], pt[kMaxTree], kept[kMaxTree];
  double zrem, C;
  int32_t i, stop;
};

template <typename TL>
__device__ void continue_siblings_wr(const AcceptKernelArgs& a, int b, int n, const TreeInfo& ti, NodeState& st,
                                     double s_full, double* dscratch, WrLds& w) {
  const int tid = threadIdx.x;
  const int k = num_children(ti, a.T, n);
  double* const kw = a.wr_kept + static_cast<int64_t>(b * a.T + n) * kMaxTree;
  if (tid < k) {
    const int tok = a.tokens[b * a.T + kth_child(ti, a.T, n, tid)];
    double qt = 0.0, pt = 0.0;
    if (tok >= 0 && tok < a.V) child_qp<TL>(a, b, n, tok, st, qt, pt);
    w.tok[tid] = tok;
    w.qt[tid] = qt;
    w.pt[tid] = pt;
    w.kept[tid] = tid < st.next_child ? kw[tid] : -1.0;
  }
  if (tid == 0) {
    w.zrem = kw[kMaxTree - 1];
    w.C = st.C;
    w.i = st.next_child;
  }
  __syncthreads();
  for (;;) {
    if (tid == 0) {
      int i = w.i;
      double C = w.C;
      double s = s_full;
      for (int j = 0; j < i; ++j)
        if (w.kept[j] >= 0.0) s += w.kept[j] - fmax(0.0, w.qt[j] - C * w.pt[j]);
      if (!(s > 0.0)) {   // residual mass vanished: start over from q, tried tokens included
        st.flags |= EAGLE_FLAG_DEGENERATE_RESIDUAL;
        C = 0.0;
        s = 1.0;
        for (int j = 0; j < i; ++j)
          if (w.kept[j] >= 0.0) w.kept[j] = w.qt[j];
      }
      int rep = -1;
      for (int j = 0; j < i && rep < 0; ++j)
        if (w.tok[j] == w.tok[i]) rep = j;
      uint32_t fl = st.flags;
      int32_t nr = st.near;
      int res;
      if (w.tok[i] < 0 || w.tok[i] >= a.V) {
        res = -1;
      } else if (rep >= 0 || !(w.zrem > 0.0)) {   // p_i(t) = 0: accept iff the residual keeps mass there
        fl |= EAGLE_FLAG_P_ZERO;
        res = (rep >= 0 ? w.kept[rep] : fmax(0.0, w.qt[i] - C * w.pt[i])) > 0.0 ? 1 : 0;
      } else {
        const double r = decision_uniform(a, b, n, static_cast<uint32_t>(i));
        res = decide_pre(w.qt[i], w.pt[i] / w.zrem, r, w.tok[i], a.V, C * w.zrem, s, fl, nr);
      }
      st.flags = fl;
      st.near = nr;
      int stop = 1;
      if (res > 0) {
        st.kind = kNodeAccepted;
        st.outcome = kth_child(ti, a.T, n, i);
      } else if (res < 0) {
        st.kind = kNodeRejected;
        st.outcome = -1;
      } else {
        const double Cn = w.zrem > 0.0 ? C + s / w.zrem : C;
        w.kept[i] = rep >= 0 ? -1.0 : fmax(0.0, w.qt[i] - Cn * w.pt[i]);
        if (rep < 0) w.zrem -= w.pt[i];
        C = Cn;
        ++i;
        if (i >= k) {
          st.kind = kNodeRejected;
          st.outcome = -1;
        } else {
          stop = 0;
        }
      }
      st.C = C;
      st.s = s;
      st.next_child = i;
      w.C = C;
      w.i = i;
      w.stop = stop;
    }
    __syncthreads();
    const int stop = w.stop;
    const double C = w.C;
    __syncthreads();
    if (stop) break;
    s_full = residual_mass<TL>(a, b, n, st, C, 0, a.V, dscratch);
  }
  // the kept weights and the draft mass left (the terminal sample reads them)
  if (tid < k) kw[tid] = w.kept[tid];
  if (tid == 0) kw[kMaxTree - 1] = w.zrem;
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
  if (!ti.ok || n >= ti.nreal) return;   // padding rows are not read
  const bool kids = has_children(ti, T, n);
  if (row == 1 && !kids) return;
  const uint32_t expected = static_cast<uint32_t>(NC) * ((!greedy && kids) ? 2u : 1u);

  const TL* rp = reinterpret_cast<const TL*>(row ? a.draft : a.target) + static_cast<int64_t>(b * T + n) * a.V;
  const int v0 = c * kVocabChunk, v1 = min(a.V, v0 + kVocabChunk);
  float x[kPerThread];
  int idx[kPerThread];
  load_chunk<TL>(rp, v0, v1, a.vec_ok != 0, x, idx);
  if (a.thr) {
    const float th = thr_of(a, b, n, row);
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) x[j] = cut(x[j], th);
  }

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
    st.near = greedy ? 0 : filter_near(a, b, n, kids);
    if (!kids) {
      st.kind = kNodeLeaf;
    } else if (nonfinite) {
      st.kind = kNodeRejected;
    } else if (greedy) {
      st.kind = kNodeRejected;
      for (int ch = n + 1; ch < ti.nreal; ++ch) {
        if (ti.par[ch] == n && a.tokens[b * T + ch] == st.argmax) {
          st.kind = kNodeAccepted;
          st.outcome = ch;
          break;
        }
      }
    } else {
      const int child = kth_child(ti, T, n, 0);
      uint32_t fl = st.flags;
      int32_t nr = st.near;
      const int res = decide_child<TL>(a, b, n, child, 0, 0.0, 1.0, st, fl, nr);
      st.flags = fl;
      st.near = nr;
      if (res > 0) {
        st.kind = kNodeAccepted;
        st.outcome = child;
      } else if (res < 0) {
        st.kind = kNodeRejected;
      } else {
        if (a.wr) {   // without replacement: the first sibling's token keeps max(0, q - p); Z = 1 - p(t)
          double qt, pt;
          child_qp<TL>(a, b, n, a.tokens[b * T + child], st, qt, pt);
          double* const kw = a.wr_kept + static_cast<int64_t>(b * T + n) * kMaxTree;
          kw[0] = fmax(0.0, qt - pt);
          kw[kMaxTree - 1] = 1.0 - pt;
        }
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
  __shared__ WrLds wr_lds;
  const int NC = a.NC, T = a.T;
  const int c = blockIdx.x % NC;
  const int n = (blockIdx.x / NC) % T;
  const int b = blockIdx.x / (NC * T);
  NodeState st = a.nodes[b * T + n];
  if (st.kind != kNodeNeedsPass) return;
  load_tree(a, b, ti);
  if (n >= ti.nreal) return;   // a padding row's state is left over from an earlier call
  const int v0 = c * kVocabChunk, v1 = min(a.V, v0 + kVocabChunk);
  const double part = residual_mass<TL>(a, b, n, st, st.C, v0, v1, dscr);
  if (threadIdx.x == 0) a.fpart[static_cast<int64_t>(b * T + n) * NC + c] = part;
  if (!arrive_last(&a.cnt_pass[b * T + n], static_cast<uint32_t>(NC), &last_flag)) return;
  double s = 0.0;
  for (int q = 0; q < NC; ++q) s += a.fpart[static_cast<int64_t>(b * T + n) * NC + q];
  if (a.wr) continue_siblings_wr<TL>(a, b, n, ti, st, s, dscr, wr_lds);
  else continue_siblings<TL>(a, b, n, ti, st, st.next_child, st.C, s, dscr, iscr);
  if (threadIdx.x == 0) a.nodes[b * T + n] = st;
}

// -------------------------------------------------------------- sa_final
// Terminal weight of token v: q_v (leaf) or max(0, q_v - C p_v).
template <typename TL>
__device__ __forceinline__ double terminal_weight(const TL* tr, const TL* dr, int v, const NodeState& st, double C,
                                                  bool leaf, float c2, double izq, double izp, float thq, float thp) {
  const double qv = static_cast<double>(exp2f((cut(logit<TL>(tr, v), thq) - st.mq) * c2)) * izq;
  if (leaf || C == 0.0) return qv;
  const double pv = static_cast<double>(exp2f((cut(logit<TL>(dr, v), thp) - st.mp) * c2)) * izp;
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
  __shared__ int32_t wtok[kMaxTree];     // without replacement: the tried siblings' tokens
  __shared__ double wkept[kMaxTree];     // ... and the weights they keep (-1: a repeated token)

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
    if (tid < ti.nreal) {
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
  const float thq = thr_of(a, b, term, 0), thp = thr_of(a, b, term, 1);
  // siblings drawn without replacement: a tried token's weight is the one it
  // kept after its rejection, not the closed form max(0, q - C p)
  const bool wr_term = a.wr && !leaf;
  const int ntried = wr_term ? min(st.next_child, num_children(ti, T, term)) : 0;
  if (tid < ntried) {
    wtok[tid] = a.tokens[b * T + kth_child(ti, T, term, tid)];
    wkept[tid] = a.wr_kept[static_cast<int64_t>(b * T + term) * kMaxTree + tid];
  }
  __syncthreads();
  auto kept_weight = [&](int v, double wv) {
    for (int j = 0; j < ntried; ++j)
      if (wkept[j] >= 0.0 && wtok[j] == v) return wkept[j];
    return wv;
  };
  {
    const int v0 = c * kVocabChunk, v1 = min(a.V, v0 + kVocabChunk);
    double acc = 0.0;
    for (int v = v0 + tid; v < v1; v += kThreads) acc += terminal_weight<TL>(tr, dr, v, st, C, leaf, a.c2, izq, izp, thq, thp);
    acc = block_reduce(acc, AddD{}, dscr);
    if (tid == 0) {
      if (C != 0.0)
        for (int j = 0; j < ntried; ++j)
          if (wkept[j] >= 0.0 && wtok[j] >= v0 && wtok[j] < v1)
            acc += wkept[j] - terminal_weight<TL>(tr, dr, wtok[j], st, C, leaf, a.c2, izq, izp, thq, thp);
      a.spart[static_cast<int64_t>(b) * NC + c] = acc;
    }
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
      for (int v = v0 + tid; v < v1; v += kThreads) acc += terminal_weight<TL>(tr, dr, v, st, C, leaf, a.c2, izq, izp, thq, thp);
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
    w[j] = (v < v1) ? terminal_weight<TL>(tr, dr, v, st, C, leaf, a.c2, izq, izp, thq, thp) : 0.0;
    if (ntried && C != 0.0 && v < v1) w[j] = kept_weight(v, w[j]);
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
// node stage their slice of the node's target and draft rows in LDS once and
// work from there to the end:
//   stats  -> chunk statistics published as self-tagged words; every
//             workgroup of the node polls them, combines them (same arithmetic
//             in the same order, so all of them hold the same node state) and
//             takes the first decision itself
//   rounds -> while the node needs another residual mass, each workgroup adds
//             (1 << 57) + its partial mass in 2^-49 fixed point to the round's
//             word with one atomic: the word carries the arrival count and an
//             exact, order-independent sum, so one poll ends the round with
//             the same s in every workgroup
//   walk   -> a node that ends without an accepted child prepares its
//             terminal chunk masses, then checks from the nodes' publication
//             words whether the walk reaches it
//   sample -> the workgroup of the chunk holding u*S scans its LDS slice in
//             token order and writes the outputs.
// Every wait is bounded by spin_limit; a wait that expires flags the
// sequence EAGLE_FLAG_INTERNAL instead of hanging.

// Publication word of a node, relative to the call's base (epoch << 20):
//   2 + u          first decision taken, another residual round follows
//                  (u = 1: one of the node's rows is unusable, non-finite)
//   2^19 + 2^12 near + 2^9 f + 2^6 kind + o
//                  final state: near-tie count, flags f (bit 0 non-finite,
//                  bit 1 P_ZERO, bit 2 degenerate residual), kind and the
//                  accepted child o (0 otherwise)
// A poll of the word alone tells the walk and the outputs everything they
// need from another node, so no node state goes through memory.
constexpr uint64_t kPubFirst = 2;
constexpr uint64_t kPubDone = 1ull << 19;
__device__ __forceinline__ uint64_t pub_word(const NodeState& st) {
  const uint64_t u = (st.flags & EAGLE_FLAG_NONFINITE) ? 1u : 0u;
  if (st.kind == kNodeNeedsPass) return kPubFirst + u;
  const uint64_t f = u | ((st.flags & EAGLE_FLAG_P_ZERO) ? 2u : 0u) | ((st.flags & EAGLE_FLAG_DEGENERATE_RESIDUAL) ? 4u : 0u);
  const uint64_t nr = static_cast<uint64_t>(min(max(st.near, 0), 127));
  const uint64_t o = st.kind == kNodeAccepted ? static_cast<uint64_t>(st.outcome & 63) : 0u;
  return kPubDone + (nr << 12) + (f << 9) + (static_cast<uint64_t>(st.kind & 3) << 6) + o;
}
__device__ __forceinline__ uint32_t pub_flags(uint64_t code) {
  const uint32_t f = static_cast<uint32_t>(code >> 9) & 7u;
  return ((f & 1u) ? EAGLE_FLAG_NONFINITE : 0u) | ((f & 2u) ? EAGLE_FLAG_P_ZERO : 0u) |
         ((f & 4u) ? EAGLE_FLAG_DEGENERATE_RESIDUAL : 0u);
}
// unusable-row bit of a published word (first or final)
__device__ __forceinline__ bool pub_unusable(uint64_t code) {
  return code >= kPubDone ? ((code >> 9) & 1u) : ((code - kPubFirst) & 1u);
}
constexpr int kFusedMaxChunks = 64;   // V <= 64 * 8192 on the fused path
// Round words: bits 57..63 count arrivals (<= 64 chunks), bits 0..56 hold the
// sum of the chunks' partial masses in units of 2^-49.  A partial is a mass
// of a probability distribution (at most 1 up to rounding; clamped to 2), so
// 64 of them stay below 2^56.
constexpr int kCountShift = 57;
constexpr uint64_t kSumMask = (1ull << kCountShift) - 1;
constexpr double kFixScale = 0x1p49;
constexpr double kFixUnit = 0x1p-49;

// Cross-workgroup words of the fused path use the system-scope helpers of
// ev_device.h (ld_u64, st_u64, stores_done, loads_after, poll, publish).


// A child of the node: its token, the node's two logits at that token and,
// once the node's normalisers are known, q(t), p(t) and the test's uniform.
struct Cand {
  double qt, pt, r;
  float xq, yp;
  int32_t tok, child;
};

struct FusedShared {
  TreeInfo ti;
  NodeState st;
  Cand cand[kMaxTree];   // by child ordinal
  int32_t nkids;
  double dscr[8];
  float fscr[8];
  int32_t iscr[4];
  int32_t ok;
  int32_t onpath;
  uint32_t seqflags;
  int32_t seqnear;
  double gscan[kPerThread / 4][kThreads / 64];   // per group column (at most 8) and wave
  int32_t wfirst[kThreads / 64];
  uint32_t pflags[kMaxTree];   // flags and near-tie counts of the root path's nodes,
  int32_t pnear[kMaxTree];     // decoded from their publication words
  double cmass[kFusedMaxChunks];   // q mass of each chunk (from the chunk statistics)
  double fscale[2];   // 2^((m_c - M) c2) / Z of this chunk's target (0) and draft (1) row
  double sample[4];
  // siblings drawn without replacement: the residual weight each tried
  // child's token keeps once later siblings no longer see it (-1: the token
  // repeats an earlier sibling's), and the draft mass not yet tried
  double wfz[kMaxTree];
  double zrem;
  int32_t tok[kMaxTree];   // the sequence's draft tokens by node (the outputs read them from here)
};

// Siblings drawn without replacement (thread 0): sibling i is tested against
// p_i = p without the earlier siblings' tokens, renormalised by the mass Z
// left.  With the untried tokens' residual max(0, q - C p) / s as before,
// rejecting sibling i gives C <- C + s / Z for the untried tokens, while a
// tried token keeps the weight max(0, q(t) - C p(t)) it had just after its own
// rejection (p_j no longer reaches it).  So the residual mass of round i is
// the full-vocabulary sum at C minus the tried tokens' terms at C plus their
// kept weights.
__device__ __forceinline__ double wr_mass(const FusedShared& sh, int tried, double C, double full) {
  double s = full;
  for (int j = 0; j < tried; ++j) {
    const double w = sh.wfz[j];
    if (w < 0.0) continue;   // a repeated token: counted once
    s += w - fmax(0.0, sh.cand[j].qt - C * sh.cand[j].pt);
  }
  return s;
}
// earlier sibling ordinal with the same token as sibling i, or -1
__device__ __forceinline__ int wr_repeat(const FusedShared& sh, int i) {
  for (int j = 0; j < i; ++j)
    if (sh.cand[j].tok == sh.cand[i].tok) return j;
  return -1;
}
// test of sibling i under (C, s) without replacement; returns 1 accept, 0 reject
__device__ __forceinline__ int wr_decide(const FusedShared& sh, int i, int V, double C, double s, uint32_t& fl,
                                         int32_t& nr) {
  const Cand& cd = sh.cand[i];
  const int rep = wr_repeat(sh, i);
  if (rep >= 0 || !(sh.zrem > 0.0)) {   // p_i(t) = 0: accept iff the residual keeps mass there
    fl |= EAGLE_FLAG_P_ZERO;
    return (rep >= 0 ? sh.wfz[rep] : fmax(0.0, cd.qt - C * cd.pt)) > 0.0 ? 1 : 0;
  }
  return decide_pre(cd.qt, cd.pt / sh.zrem, cd.r, cd.tok, V, C * sh.zrem, s, fl, nr);
}
// after rejecting sibling i at (C, s): the next C, and the kept weight of its token
__device__ __forceinline__ double wr_reject(FusedShared& sh, int i, double C, double s) {
  const int rep = wr_repeat(sh, i);
  const double Cn = sh.zrem > 0.0 ? C + s / sh.zrem : C;
  const Cand& cd = sh.cand[i];
  sh.wfz[i] = rep >= 0 ? -1.0 : fmax(0.0, cd.qt - Cn * cd.pt);
  if (rep < 0) sh.zrem -= cd.pt;
  return Cn;
}

// Two reductions over the block sharing one pair of barriers (all threads call).
template <typename T, typename Op>
__device__ void block_reduce2(T& x, T& y, Op op, T* scratch /* >= 8 */) {
  x = wave_reduce(x, op);
  y = wave_reduce(y, op);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    scratch[w] = x;
    scratch[4 + w] = y;
  }
  __syncthreads();
  x = op(op(scratch[0], scratch[1]), op(scratch[2], scratch[3]));
  y = op(op(scratch[4], scratch[5]), op(scratch[6], scratch[7]));
}

// 16 bytes of logits <-> G values in token order.
template <typename TL>
struct Pack;
template <>
struct Pack<uint16_t> {
  static constexpr int G = 8;
  __device__ __forceinline__ static void unpack(const u32x4_t w, float (&f)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  __device__ __forceinline__ static uint32_t neg_inf_word() { return 0xFF80FF80u; }
  __device__ __forceinline__ static uint32_t bits(uint16_t x) { return x; }
};
template <>
struct Pack<float> {
  static constexpr int G = 4;
  __device__ __forceinline__ static void unpack(const u32x4_t w, float (&f)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
  }
  __device__ __forceinline__ static uint32_t neg_inf_word() { return 0xFF800000u; }
  __device__ __forceinline__ static uint32_t bits(float x) { return __float_as_uint(x); }
};

// One logit of a chunk staged in LDS, as fp32.
template <typename TL>
__device__ __forceinline__ float lds_logit(const TL* l, int i) {
  if constexpr (sizeof(TL) == 2)
    return __uint_as_float(static_cast<uint32_t>(l[i]) << 16);
  else
    return l[i];
}

// A row chunk lives in LDS in token order (index = token - v0; tokens past
// the vocabulary hold -inf).  In the "strided" view thread t owns the
// 16-byte groups jj * 256 + t (jj < NV), so a warp reads consecutive groups.
template <typename TL>
__device__ __forceinline__ int group_index(int jj) {
  return (jj * kThreads + static_cast<int>(threadIdx.x)) * Pack<TL>::G;
}

// Load this thread's strided groups of [v0, v1) from a row.
template <typename TL, int NV>
__device__ __forceinline__ void load_groups(const TL* row, int v0, int v1, bool vecpath, u32x4_t (&w)[NV]) {
  constexpr int G = Pack<TL>::G;
#pragma unroll
  for (int jj = 0; jj < NV; ++jj) {
    const int i0 = group_index<TL>(jj);
    const uint32_t ni = Pack<TL>::neg_inf_word();
    if (vecpath) {
      w[jj] = (v0 + i0 < v1) ? *reinterpret_cast<const u32x4_t*>(row + v0 + i0) : u32x4_t{ni, ni, ni, ni};
    } else {
      uint32_t e32[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < G; ++e) {
        const uint32_t x = (v0 + i0 + e < v1) ? Pack<TL>::bits(row[v0 + i0 + e]) : (ni & (sizeof(TL) == 2 ? 0xFFFFu : ~0u));
        if constexpr (sizeof(TL) == 2)
          e32[e >> 1] |= x << (16 * (e & 1));
        else
          e32[e] = x;
      }
      w[jj] = u32x4_t{e32[0], e32[1], e32[2], e32[3]};
    }
  }
}

// The chunk [v0, v1) as 16-byte groups when every row and chunk boundary is
// a whole group: each request is made unconditionally (a group past v1
// re-reads the chunk's last group), so the loads of a wave form one
// straight run and a later wait can name how many of them may still be in
// flight.  mask_groups then replaces the groups past v1 by -inf.
template <typename TL, int NV>
__device__ __forceinline__ void request_groups(const TL* row, int v0, int v1, u32x4_t (&w)[NV]) {
  constexpr int G = Pack<TL>::G;
#pragma unroll
  for (int jj = 0; jj < NV; ++jj)
    w[jj] = *reinterpret_cast<const u32x4_t*>(row + min(v0 + group_index<TL>(jj), v1 - G));
}
template <typename TL, int NV>
__device__ __forceinline__ void mask_groups(int v0, int v1, u32x4_t (&w)[NV]) {
  const uint32_t ni = Pack<TL>::neg_inf_word();
#pragma unroll
  for (int jj = 0; jj < NV; ++jj)
    if (v0 + group_index<TL>(jj) >= v1) w[jj] = u32x4_t{ni, ni, ni, ni};
}

// Logits below th become -inf (NaN and +inf pass unchanged).
template <typename TL, int NV>
__device__ __forceinline__ void cut_groups(u32x4_t (&w)[NV], float th) {
  const uint32_t ni = Pack<TL>::neg_inf_word();
#pragma unroll
  for (int jj = 0; jj < NV; ++jj) {
    float f[Pack<TL>::G];
    Pack<TL>::unpack(w[jj], f);
    if constexpr (sizeof(TL) == 2) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = f[2 * i] < th ? (ni & 0xFFFFu) : (w[jj][i] & 0xFFFFu);
        const uint32_t hi = f[2 * i + 1] < th ? (ni & 0xFFFF0000u) : (w[jj][i] & 0xFFFF0000u);
        w[jj][i] = lo | hi;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (f[i] < th) w[jj][i] = ni;
    }
  }
}

// Row statistics of this thread's values: the maximum, or +inf when a NaN or
// +inf is present (the row is then unusable).
template <typename TL, int NV>
__device__ __forceinline__ float local_max(const u32x4_t (&w)[NV]) {
  float m = kNegInf;
#pragma unroll
  for (int jj = 0; jj < NV; ++jj) {
    float f[Pack<TL>::G];
    Pack<TL>::unpack(w[jj], f);
#pragma unroll
    for (int e = 0; e < Pack<TL>::G; ++e) m = (f[e] != f[e] || f[e] == __builtin_inff()) ? __builtin_inff() : fmaxf(m, f[e]);
  }
  return m;
}

// exp((x - m) / tau) = 2^((x - m) c2) on the hardware exp2 (results below
// 2^-126 of the row maximum, irrelevant to any sum here, may flush to 0).
// The difference is taken first: x c2 - m c2 as one fma would carry the
// rounding error of m c2, a factor common to a chunk but not across chunks,
// which grows with |m| (and overflows for |m| near the float range).
__device__ __forceinline__ float ex2(float x, float c2, float m) { return __builtin_amdgcn_exp2f((x - m) * c2); }

// The per-thread sums below share one order: the thread's values in its
// token order i = jj G + e, added in pairs (i, i + 1) in fp32 (one rounding,
// at most 2^-24 relative, below the exponentials' own error), each pair
// added in fp64 to accumulator (i / 2) mod 4, the accumulators combined as
// (a0 + a1) + (a2 + a3).  Half the fp64 conversions and additions of a
// per-value fp64 sum.

// sum of exp((x - m) / tau) over this thread's values, fp64
template <typename TL, int NV>
__device__ __forceinline__ double local_expsum(const u32x4_t (&w)[NV], float m, float c2) {
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int jj = 0; jj < NV; ++jj) {
    float f[Pack<TL>::G];
    Pack<TL>::unpack(w[jj], f);
#pragma unroll
    for (int e = 0; e < Pack<TL>::G; e += 2)
      acc[((jj * Pack<TL>::G + e) >> 1) & 3] += static_cast<double>(ex2(f[e], c2, m) + ex2(f[e + 1], c2, m));
  }
  return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// local_expsum that also keeps every exponential (index jj * G + e) for the
// residual rounds; an all -inf chunk (m = -inf) keeps zeros and sums 0.
template <typename TL, int NV>
__device__ __forceinline__ double local_expsum_keep(const u32x4_t (&w)[NV], float m, float c2,
                                                    float (&ex)[NV * Pack<TL>::G]) {
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  const bool live = m != kNegInf;
  const float ms = live ? m : 0.f;
#pragma unroll
  for (int jj = 0; jj < NV; ++jj) {
    float f[Pack<TL>::G];
    Pack<TL>::unpack(w[jj], f);
#pragma unroll
    for (int e = 0; e < Pack<TL>::G; e += 2) {
      const float v0 = ex2(f[e], c2, ms), v1 = ex2(f[e + 1], c2, ms);
      ex[jj * Pack<TL>::G + e] = v0;
      ex[jj * Pack<TL>::G + e + 1] = v1;
      acc[((jj * Pack<TL>::G + e) >> 1) & 3] += static_cast<double>(v0 + v1);
    }
  }
  return live ? (acc[0] + acc[1]) + (acc[2] + acc[3]) : 0.0;
}

// Residual mass sum max(0, q - C p) of this thread's strided slots from the
// exponentials the statistics pass kept (the same values local_masses
// computes from LDS, summed in the same pairs and order).
template <int N>
__device__ __forceinline__ double kept_masses(const float (&eq)[N], const float (&ep)[N], float K, double fq) {
  static_assert(N % 2 == 0, "pairs");
  double ra[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int i = 0; i < N; i += 2)
    ra[(i >> 1) & 3] += static_cast<double>(fmaxf(0.f, __builtin_fmaf(-K, ep[i], eq[i])) +
                                            fmaxf(0.f, __builtin_fmaf(-K, ep[i + 1], eq[i + 1])));
  return ((ra[0] + ra[1]) + (ra[2] + ra[3])) * fq;
}

// Residual mass sum max(0, q - C p) and plain mass sum q of this thread's
// strided slots, from LDS.  With q = fq e_q and p = fp e_p (e = exp2 of the
// scaled logit minus the chunk maximum; mqs / mps are 0 for an all -inf
// chunk, whose exponentials are then 0), max(0, q - C p) = fq max(0, e_q -
// K e_p) with K = C fp / fq: per token two exp2, one fma and one max in
// fp32, token pairs added in fp32, the pairs accumulated in fp64.
template <typename TL, int NV>
__device__ __forceinline__ void local_masses(const TL* lq, const TL* lp, bool use_p, float mqs, float mps, float c2,
                                             double fq, double fp, double C, double& res, double& qsum) {
  double ra[4] = {0.0, 0.0, 0.0, 0.0}, qa[4] = {0.0, 0.0, 0.0, 0.0};
  const float K = (use_p && fq > 0.0) ? static_cast<float>(C * fp / fq) : 0.f;
  u32x4_t wq[NV], wp[NV];
#pragma unroll
  for (int jj = 0; jj < NV; ++jj) {
    wq[jj] = *reinterpret_cast<const u32x4_t*>(lq + group_index<TL>(jj));
    if (use_p) wp[jj] = *reinterpret_cast<const u32x4_t*>(lp + group_index<TL>(jj));
  }
#pragma unroll
  for (int jj = 0; jj < NV; ++jj) {
    float fa[Pack<TL>::G], fb[Pack<TL>::G];
    Pack<TL>::unpack(wq[jj], fa);
    if (use_p) Pack<TL>::unpack(wp[jj], fb);
#pragma unroll
    for (int e = 0; e < Pack<TL>::G; e += 2) {
      const int k = ((jj * Pack<TL>::G + e) >> 1) & 3;
      const float eq0 = ex2(fa[e], c2, mqs), eq1 = ex2(fa[e + 1], c2, mqs);
      qa[k] += static_cast<double>(eq0 + eq1);
      if (use_p)
        ra[k] += static_cast<double>(fmaxf(0.f, __builtin_fmaf(-K, ex2(fb[e], c2, mps), eq0)) +
                                     fmaxf(0.f, __builtin_fmaf(-K, ex2(fb[e + 1], c2, mps), eq1)));
    }
  }
  qsum = ((qa[0] + qa[1]) + (qa[2] + qa[3])) * fq;
  res = use_p ? ((ra[0] + ra[1]) + (ra[2] + ra[3])) * fq : qsum;
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

// VEC: rows and chunks are whole 16-byte groups (then every chunk is read
// with straight-line vector requests)
// WR: siblings drawn without replacement (a separate instantiation, so that
// the common kernel carries none of it)
// LATE: the target chunk is requested once the node's children are known,
// a leaf's after a.leaf_wait sleeps (sampled mode on the common path)
template <typename TL, bool VEC, bool WR, bool LATE = false>
__global__ __launch_bounds__(kThreads, 4) void sa_fused(const AcceptKernelArgs a) {
  constexpr int G = Pack<TL>::G;
  constexpr int NV = kPerThread / G;   // 16-byte groups per thread and row
  __shared__ FusedShared sh;
  __shared__ int32_t path_lds[kMaxTree];
  __shared__ __attribute__((aligned(16))) TL lq[kVocabChunk];
  __shared__ __attribute__((aligned(16))) TL lp[kVocabChunk];
  // One field of each 64-byte line of the argument block, requested together
  // and waited for once: later first uses of the other fields then hit the
  // scalar cache instead of each paying a round trip.
  {
    const void* l0 = a.target;
    const void* l1 = a.near_ties;
    const void* l2 = a.node_pub;
    const int l3 = a.T;
    const float l4 = a.tau;
    asm volatile("" ::"s"(l0), "s"(l1), "s"(l2), "s"(l3), "s"(l4));
  }
  const int NC = a.NC, T = a.T, V = a.V, tid = threadIdx.x;
  const int c = blockIdx.x % NC;
  const int n = (blockIdx.x / NC) % T;
  const int b = blockIdx.x / (NC * T);
  const bool greedy = a.tau == 0.f;
  const uint64_t base = a.epoch << 20;
  const uint32_t limit = a.spin_limit;
  const bool lead = (c == 0);   // publishes the node's state for the other nodes' groups
  stamp(a.stamps, 0);

  // the round words of the previous fused call start this call's successor at zero
  {
    const int64_t total = static_cast<int64_t>(a.zero_b) * a.Tm * kRoundWords;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + tid; i < total;
         i += static_cast<int64_t>(gridDim.x) * kThreads)
      st_u64(a.round_clear + i, 0ull);
  }

  // node j of this sequence publishes its decisions at pubs[j]
  uint64_t* const pubs = a.node_pub + static_cast<int64_t>(b) * a.Tm;   // publication words of the sequence
  uint64_t* const npub = pubs + n;

  auto fail_internal = [&]() {
    if (tid == 0) __hip_atomic_fetch_or(&a.flags[b], static_cast<uint32_t>(EAGLE_FLAG_INTERNAL), __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_SYSTEM);
  };

  // ---- sequence validity (the same verdict in every workgroup of b) and
  // this node's children, in ascending index = child ordinal.  Every wave
  // reads the sequence's parents and tokens one per lane.  Without LATE it
  // requests its share of the target chunk right behind them, so the
  // transfer is under way while the tree is checked (loads of a wave return
  // in order: waiting for the parents leaves the chunk requests in flight);
  // with LATE it requests it once the node's children are known (a leaf
  // later, see below).  The draft chunk follows once the node is known to
  // have children.
  const int lane = tid & 63;
  const int v0 = c * kVocabChunk, v1 = min(V, v0 + kVocabChunk);
  const int64_t rowoff = static_cast<int64_t>(b * T + n) * V;
  const TL* trow = reinterpret_cast<const TL*>(a.target) + rowoff;
  const TL* drow = reinterpret_cast<const TL*>(a.draft) + rowoff;
  const int li = b * T + min(lane, T - 1);   // lanes past the tree re-read its last row
  int par = a.parents[li];
  int tok = a.tokens[li];
  u32x4_t wq[NV], wd[NV];
  if constexpr (!LATE) {
    if constexpr (VEC) request_groups<TL, NV>(trow, v0, v1, wq);
    else load_groups<TL, NV>(trow, v0, v1, false, wq);
  }
  if (lane >= T) par = 0;
  if (lane < 1 || lane >= T) tok = 0;
  const bool good = lane >= T || (lane == 0 ? par == -1 : (par >= 0 && par < lane));
  const int Tr = real_rows(tok == -1, T);   // rows of the tree proper; -1: padding not a suffix
  if (__any(!good) || Tr < 1) {
    if (n == 0 && c == 0) write_poison(a, b, EAGLE_FLAG_BAD_TREE);
    return;
  }
  if (n >= Tr) return;   // a padding row: nothing reads or waits for it
  // The root's first workgroup poisons the sequence's outputs (flag
  // INTERNAL) before its first publication, with stores that go through to
  // memory.  The workgroup that writes the real outputs waits for that
  // publication, so it overwrites them afterwards; if a bounded wait expires
  // and nobody writes them, the caller finds them poisoned and flagged.
  if (n == 0 && c == 0) {
    if (tid == 0) {
      __hip_atomic_store(&a.accept_len[b], -1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      __hip_atomic_store(&a.flags[b], static_cast<uint32_t>(EAGLE_FLAG_INTERNAL), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_SYSTEM);
      __hip_atomic_store(&a.near_ties[b], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    for (int j = tid; j < T; j += kThreads) {
      __hip_atomic_store(&a.accepted_nodes[b * T + j], -1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      __hip_atomic_store(&a.out_tokens[b * T + j], -1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    stores_done();   // complete before the barriers that precede the first publication
  }
  const bool tb = lane >= 1 && lane < Tr && (tok < 0 || tok >= V);
  const bool is_child = lane >= 1 && lane < Tr && par == n;
  const uint64_t kids_mask = __ballot(is_child);
  const int nkids = __popcll(kids_mask);
  // a token outside the vocabulary poisons the sequence too, but the row
  // checks still run so that every unusable input is reported
  const uint32_t tokbad = __any(tb) ? EAGLE_FLAG_BAD_TOKEN : 0u;
  const bool two = nkids > 0 && !greedy;
  // Internal nodes decide (statistics, first decision, residual rounds) on
  // the way to every walk; a leaf's statistics matter only if the walk ends
  // there.  Where the workgroups of a CU compete for the vector ALU, the
  // internal nodes' waves are issued first.
  if (nkids > 0 && a.node_priority) __builtin_amdgcn_s_setprio(2);
  // LATE: a leaf's row gates nothing until the walk ends, while the internal
  // nodes' rows gate the first decisions and the residual rounds.  Under the
  // full-chip burst that stages every chunk, a leaf requests its row
  // a.leaf_wait sleeps of 640 clocks later (the host sizes the wait to the
  // launch's bytes), so that HBM serves the internal nodes first.
  if constexpr (LATE) {
    if (nkids == 0)
      for (int i = 0; i < a.leaf_wait; ++i) __builtin_amdgcn_s_sleep(10);
    if constexpr (VEC) request_groups<TL, NV>(trow, v0, v1, wq);
    else load_groups<TL, NV>(trow, v0, v1, false, wq);
  }
  if (two) {
    if constexpr (VEC) request_groups<TL, NV>(drow, v0, v1, wd);
    else load_groups<TL, NV>(drow, v0, v1, false, wd);
  }
  if (tid < 64) {
    sh.ti.par[lane] = par;
    sh.tok[lane] = tok;
    if (is_child) {
      const int ord = __popcll(kids_mask & ((1ull << lane) - 1ull));
      Cand cd;
      cd.qt = cd.pt = cd.r = 0.0;
      cd.xq = cd.yp = 0.f;
      cd.tok = tok;
      cd.child = lane;
      if (!greedy && !tb) {
        cd.xq = cut(logit<TL>(trow, tok), thr_of(a, b, n, 0));
        cd.yp = cut(logit<TL>(drow, tok), thr_of(a, b, n, 1));
      }
      // the test's uniform depends on nothing the statistics decide: drawn
      // while the rows are still arriving
      if (!greedy) cd.r = decision_uniform(a, b, n, static_cast<uint32_t>(ord));
      sh.cand[ord] = cd;
    }
  }

  // ---- statistics pass: the chunk is loaded once, kept in LDS, and its
  // statistics come straight from the loaded registers
  float mq_c, mp_c = kNegInf;
  int amq = -1;
  double zq_c = 0.0, zp_c = 0.0;
  // the statistics' exponentials of this thread's slots (the draft row's at
  // an internal node only), kept for the residual rounds and the terminal
  // weights; the path for rows that are not whole 16-byte groups, short of
  // registers, recomputes them from LDS each time instead
  constexpr bool kKeep = VEC;
  float xq[kPerThread], xp[kPerThread];
  {
    if constexpr (VEC) {
      mask_groups<TL, NV>(v0, v1, wq);
      if (two) mask_groups<TL, NV>(v0, v1, wd);
    }
    if (a.thr) {   // filtered distributions: logits below the row's threshold become -inf
      cut_groups<TL, NV>(wq, thr_of(a, b, n, 0));
      if (two) cut_groups<TL, NV>(wd, thr_of(a, b, n, 1));
    }
#pragma unroll
    for (int jj = 0; jj < NV; ++jj) {
      *reinterpret_cast<u32x4_t*>(lq + group_index<TL>(jj)) = wq[jj];
      if (two) *reinterpret_cast<u32x4_t*>(lp + group_index<TL>(jj)) = wd[jj];
    }
    stamp(a.stamps, 1);   // the chunk has arrived
    mq_c = local_max<TL, NV>(wq);
    if (two) mp_c = local_max<TL, NV>(wd);
    block_reduce2(mq_c, mp_c, MaxOp{}, sh.fscr);
    if (greedy) {
      int la = 0x7FFFFFFF;
#pragma unroll
      for (int jj = 0; jj < NV; ++jj) {
        float f[G];
        Pack<TL>::unpack(wq[jj], f);
#pragma unroll
        for (int e = 0; e < G; ++e) {
          const int t = v0 + group_index<TL>(jj) + e;
          if (f[e] == mq_c && t < v1 && t < la) la = t;
        }
      }
      amq = block_reduce(la, MinI{}, sh.iscr);
    } else {
      double lzq = 0.0, lzp = 0.0;
      if constexpr (kKeep) {
        if (mq_c != __builtin_inff()) lzq = local_expsum_keep<TL, NV>(wq, mq_c, a.c2, xq);
        if (two && mp_c != __builtin_inff()) lzp = local_expsum_keep<TL, NV>(wd, mp_c, a.c2, xp);
      } else {
        if (mq_c != kNegInf && mq_c != __builtin_inff()) lzq = local_expsum<TL, NV>(wq, mq_c, a.c2);
        if (two && mp_c != kNegInf && mp_c != __builtin_inff()) lzp = local_expsum<TL, NV>(wd, mp_c, a.c2);
      }
      block_reduce2(lzq, lzp, AddD{}, sh.dscr);
      zq_c = lzq;
      zp_c = lzp;
    }
  }
  stamp(a.stamps, 2);   // chunk statistics
  // Chunk statistics go out as four 64-bit words per row, each carrying the
  // call's tag in its high half (m, z low, z high, argmax | bad << 31), and
  // are read back by polling the words themselves: no arrival counter.
  const uint64_t stag = static_cast<uint64_t>(static_cast<uint32_t>(a.epoch)) << 32;
  uint64_t* const cw = reinterpret_cast<uint64_t*>(a.stats) + (static_cast<int64_t>(b * T + n) * 2) * NC * 4;
  if (tid < 8) {   // lanes 0..3 the target row, 4..7 the draft row
    const int r = tid >> 2, k = tid & 3;
    if (r == 0 || two) {
      const float m = r == 0 ? mq_c : mp_c;
      const double z = r == 0 ? zq_c : zp_c;
      const uint64_t zb = __builtin_bit_cast(uint64_t, z);
      const uint32_t bad = (m == __builtin_inff()) ? 1u : 0u;
      const uint32_t lo = k == 0 ? __float_as_uint(m)
                        : k == 1 ? static_cast<uint32_t>(zb)
                        : k == 2 ? static_cast<uint32_t>(zb >> 32)
                                 : ((static_cast<uint32_t>(r == 0 ? amq : 0) & 0x7FFFFFFFu) | (bad << 31));
      st_u64(cw + (r * NC + c) * 4 + k, stag | lo);
    }
  }

  // ---- every workgroup of the node combines the chunks (same arithmetic in
  // the same order everywhere, so all of them hold the same node state):
  // wave 0 the target row, wave 1 the draft row, one chunk per lane
  if (tid == 0) sh.ok = 1;
  __syncthreads();
  if (tid < 128) {
    const int r = tid >> 6, q = tid & 63;
    if (r == 0 || two) {
      float mc = kNegInf;
      uint32_t bc = 0;
      int ac = 0x7FFFFFFF;
      double zc = 0.0;
      uint64_t w[4] = {0, 0, 0, 0};
      bool have = q >= NC;
      for (uint32_t it = 0;; ++it) {
        if (!have) {
#pragma unroll
          for (int k = 0; k < 4; ++k) w[k] = ld_u64(cw + (r * NC + q) * 4 + k);
          have = ((w[0] & w[1] & w[2] & w[3]) >> 32) == (stag >> 32) && ((w[0] | w[1] | w[2] | w[3]) >> 32) == (stag >> 32);
        }
        if (__all(have)) break;
        if (it >= limit) {
          sh.ok = 0;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      if (q < NC) {
        mc = __uint_as_float(static_cast<uint32_t>(w[0]));
        zc = __builtin_bit_cast(double, (w[1] & 0xFFFFFFFFull) | (w[2] << 32));
        bc = static_cast<uint32_t>(w[3]) >> 31;
        ac = static_cast<int>(static_cast<uint32_t>(w[3]) & 0x7FFFFFFFu);
      }
      const float M = wave_reduce(mc, MaxOp{});
      const uint32_t rb = wave_reduce(bc, OrU{});
      const double Z = wave_reduce(
          (!greedy && q < NC && mc != kNegInf) ? zc * exp2((static_cast<double>(mc) - M) * static_cast<double>(a.c2)) : 0.0,
          AddD{});
      const int arg = wave_reduce((greedy && q < NC && mc == M) ? ac : 0x7FFFFFFF, MinI{});
      if (r == 0)   // q mass of chunk q: the terminal distribution of a leaf, per chunk
        sh.cmass[q] = (!greedy && q < NC && mc != kNegInf && Z > 0.0)
                          ? zc * exp2((static_cast<double>(mc) - M) * static_cast<double>(a.c2)) / Z
                          : 0.0;
      // this workgroup's own chunk: the factor from its exponentials to the
      // row's probabilities (the residual rounds and the terminal weights)
      if (q == c)
        sh.fscale[r] = (!greedy && mc != kNegInf && Z > 0.0)
                           ? exp2((static_cast<double>(mc) - M) * static_cast<double>(a.c2)) / Z
                           : 0.0;
      if (q == 0) {
        const uint32_t fl = (rb || M == kNegInf) ? EAGLE_FLAG_NONFINITE : 0u;
        if (r == 0) {
          sh.st.mq = M;
          sh.st.zq = Z;
          sh.st.argmax = arg;
          sh.st.flags = fl;
        } else {
          sh.st.mp = M;
          sh.st.zp = Z;
          sh.iscr[1] = static_cast<int32_t>(fl);
        }
      }
    }
  }
  __syncthreads();
  if (!sh.ok) return fail_internal();
  stamp(a.stamps, 3);   // row statistics combined
  if (tid == 0 && two) sh.st.flags |= static_cast<uint32_t>(sh.iscr[1]);
  __syncthreads();
  if (tid < 64) {
    // q(t), p(t) and the uniform of every child test, in parallel
    if (two && tid < nkids && !(sh.st.flags & EAGLE_FLAG_NONFINITE)) {
      Cand& cd = sh.cand[tid];
      if (cd.tok >= 0 && cd.tok < V) {
        cd.qt = exp((static_cast<double>(cd.xq) - static_cast<double>(sh.st.mq)) * a.inv_tau) / sh.st.zq;
        cd.pt = exp((static_cast<double>(cd.yp) - static_cast<double>(sh.st.mp)) * a.inv_tau) / sh.st.zp;
      }
    }
    // greedy: the first child carrying the target argmax
    if (greedy) {
      const bool match = tid < nkids && sh.cand[tid].tok == sh.st.argmax;
      const uint64_t mm = __ballot(match);
      if (tid == 0) sh.iscr[0] = mm ? sh.cand[__ffsll(static_cast<long long>(mm)) - 1].child : -1;
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
    st.near = greedy ? 0 : filter_near(a, b, n, two);
    if (nkids == 0) {
      st.kind = kNodeLeaf;
    } else if (st.flags & EAGLE_FLAG_NONFINITE) {
      st.kind = kNodeRejected;
    } else if (greedy) {
      st.outcome = sh.iscr[0];
      st.kind = st.outcome >= 0 ? kNodeAccepted : kNodeRejected;
    } else {
      const Cand& cd = sh.cand[0];
      uint32_t fl = st.flags;
      int32_t nr = st.near;
      sh.zrem = 1.0;
      for (int j = 0; j < nkids; ++j) sh.wfz[j] = -1.0;   // no kept weight until the sibling is rejected
      const int res = decide_pre(cd.qt, cd.pt, cd.r, cd.tok, V, 0.0, 1.0, fl, nr);
      st.flags = fl;
      st.near = nr;
      if (res > 0) {
        st.kind = kNodeAccepted;
        st.outcome = cd.child;
      } else {
        st.C = WR ? wr_reject(sh, 0, 0.0, 1.0) : 1.0;
        st.next_child = 1;
        st.kind = (res == 0 && nkids > 1) ? kNodeNeedsPass : kNodeRejected;
      }
    }
    sh.st = st;
    if (lead) publish(npub, base + pub_word(st));
  }
  __syncthreads();

  stamp(a.stamps, 4);   // first decision
  // ---- residual-mass rounds from LDS
  const bool q_live = mq_c != kNegInf, p_live = two && mp_c != kNegInf;
  const float mqs = q_live ? mq_c : 0.f, mps = p_live ? mp_c : 0.f;
  const double fq = q_live ? sh.fscale[0] : 0.0;
  const double fp = p_live ? sh.fscale[1] : 0.0;
  uint64_t* const rwords = a.round_sum + (static_cast<int64_t>(b) * a.Tm + n) * kRoundWords;
  int round = 0;
  while (sh.st.kind == kNodeNeedsPass) {
    double part;
    if constexpr (kKeep) {
      part = kept_masses(xq, xp, fq > 0.0 ? static_cast<float>(sh.st.C * fp / fq) : 0.f, fq);
    } else {
      double unused;
      local_masses<TL, NV>(lq, lp, true, mqs, mps, a.c2, fq, fp, sh.st.C, part, unused);
    }
    part = block_reduce(part, AddD{}, sh.dscr);
    if (tid == 0) {
      const double pc = fmin(fmax(part, 0.0), 2.0);
      const uint64_t add = (1ull << kCountShift) + static_cast<uint64_t>(__double2ull_rn(pc * kFixScale));
      __hip_atomic_fetch_add(rwords + round, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      uint64_t w = poll(rwords + round);
      uint32_t it = 0;
      bool fine = true;
      while ((w >> kCountShift) < static_cast<uint64_t>(NC)) {
        if (++it > limit) {
          fine = false;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
        w = poll(rwords + round);
      }
      sh.ok = fine ? 1 : 0;
      NodeState st = sh.st;
      int i = st.next_child;
      double Cn = st.C;
      double s = static_cast<double>(w & kSumMask) * kFixUnit;
      if (WR) s = wr_mass(sh, i, Cn, s);
      if (!(s > 0.0)) {
        st.flags |= EAGLE_FLAG_DEGENERATE_RESIDUAL;
        Cn = 0.0;
        s = 1.0;
        if (WR)   // the residual starts over from q, tried tokens included
          for (int j = 0; j < i; ++j)
            if (sh.wfz[j] >= 0.0) sh.wfz[j] = sh.cand[j].qt;
      }
      const Cand& cd = sh.cand[i];
      uint32_t fl = st.flags;
      int32_t nr = st.near;
      const int res = WR ? wr_decide(sh, i, V, Cn, s, fl, nr) : decide_pre(cd.qt, cd.pt, cd.r, cd.tok, V, Cn, s, fl, nr);
      st.flags = fl;
      st.near = nr;
      if (res > 0) {
        st.kind = kNodeAccepted;
        st.outcome = cd.child;
      } else {
        Cn = WR ? wr_reject(sh, i, Cn, s) : Cn + s;
        ++i;
        st.kind = (res == 0 && i < nkids) ? kNodeNeedsPass : kNodeRejected;
      }
      st.C = Cn;
      st.s = s;
      st.next_child = i;
      sh.st = st;
      if (fine && lead && st.kind != kNodeNeedsPass) publish(npub, base + pub_word(st));
    }
    __syncthreads();
    if (!sh.ok) return fail_internal();
    if (round < 12) stamp(a.stamps, 5 + round);   // end of residual round
    ++round;
  }
  stamp_value(a.stamps, 30, static_cast<uint64_t>(round));
  stamp_value(a.stamps, 31, static_cast<uint64_t>(n) | (static_cast<uint64_t>(c) << 8) |
                                (static_cast<uint64_t>(sh.st.kind) << 16) | (static_cast<uint64_t>(b) << 24));
  stamp(a.stamps, 17);   // node decided

  // ---- sequence verdict: workgroup 0 of the root waits for every node's
  // first publication and writes the poisoned outputs if any row was
  // unusable (the terminal node reaches the same verdict from the words)
  const bool master = (n == 0 && c == 0);
  if (master) {
    if (tid == 0) {
      sh.seqflags = tokbad;
      sh.ok = 1;
    }
    __syncthreads();
    if (tid < 64) {   // lane j waits for node j's first publication
      bool seen = tid >= Tr;
      for (uint32_t it = 0;; ++it) {
        if (!seen) {
          const uint64_t w = poll(pubs + tid);
          if (w >= base + kPubFirst) {
            seen = true;
            if (pub_unusable(w - base)) atomicOr(&sh.seqflags, EAGLE_FLAG_NONFINITE);
          }
        }
        if (__all(seen)) break;
        if (it >= limit) {
          sh.ok = 0;
          break;
        }
        __builtin_amdgcn_s_sleep(4);
      }
    }
    __syncthreads();
    if (!sh.ok) return fail_internal();
    const uint32_t sf = sh.seqflags;
    if (sf) {
      write_poison(a, b, sf);
      return;
    }
  }
  if (sh.st.kind == kNodeAccepted) return;
  // an unusable row poisons the whole sequence: nothing to sample here
  if (sh.st.flags & EAGLE_FLAG_NONFINITE) return;
  const bool leaf = (sh.st.kind == kNodeLeaf);

  // ---- the walk ends at this node iff every ancestor accepted the next node
  // of this root path and no node of the sequence has an unusable row.
  // Lane j of wave 0 follows node j's publication word: wpos is node j's
  // position on the root path if it is an ancestor (else -1), wnxt the
  // node after it there.
  if (tid == 0) sh.iscr[0] = root_path(sh.ti, n, path_lds);
  __syncthreads();
  const int plen = sh.iscr[0];
  int wpos = -1, wnxt = -1;
  if (tid < 64) {
    for (int i = 0; i + 1 < plen; ++i)
      if (path_lds[i] == tid) wpos = i;
    wnxt = wpos >= 0 ? path_lds[wpos + 1] : -1;
  }
  // 0: undecided, 1: consistent with the walk ending here, 2: rules it out.
  // A final word of an ancestor also gives its flags and near ties (record).
  auto walk_state = [&](uint64_t w, bool record) __attribute__((always_inline)) -> int {
    if (w < base + kPubFirst) return 0;
    const uint64_t code = w - base;
    if (pub_unusable(code)) return 2;
    if (wpos < 0) return 1;
    if (code < kPubDone) return 0;
    if (record) {
      sh.pflags[tid] = pub_flags(code);
      sh.pnear[tid] = static_cast<int32_t>((code >> 12) & 127u);
    }
    return (static_cast<int>((code >> 6) & 3u) == kNodeAccepted && static_cast<int>(code & 63u) == wnxt) ? 1 : 2;
  };
  // Decisions published by now may already rule this node out: then it
  // skips the terminal preparation.  Its workgroups still publish (empty)
  // chunk masses, which other workgroups of the node (that read the words
  // earlier) may be waiting for; the node cannot be sampled from, so their
  // values do not matter.
  uint64_t* const mw = reinterpret_cast<uint64_t*>(a.spart) + static_cast<int64_t>(b * T + n) * NC * 4;
  if (tid < 64) {
    const int st0 = tid < Tr ? walk_state(poll(pubs + tid), false) : 1;
    const bool out = __any(st0 == 2);
    if (tid == 0) sh.iscr[1] = out ? 1 : 0;
  }
  __syncthreads();
  if (sh.iscr[1]) {
    if (!leaf && !greedy && tid < 4) st_u64(mw + c * 4 + tid, stag);
    return;
  }

  stamp(a.stamps, 18);   // terminal preparation starts
  // ---- terminal distribution of this node, prepared before the walk is
  // known to end here (it overlaps the walk): inverse CDF of the residual
  // max(0, q - C p) (of q at a leaf; of q again if the residual mass is
  // zero).  It works in the strided view: group g = jj * kThreads + t of
  // thread t holds the G consecutive tokens [g G, g G + G) of the chunk, so
  // token order is group order.  Every workgroup of the node publishes its
  // chunk mass and finds the chunk holding u*S; only that workgroup
  // continues once the walk is known to end here.
  const double Ct = leaf ? 0.0 : sh.st.C;
  const float Kt = fq > 0.0 ? static_cast<float>(Ct * fp / fq) : 0.f;
  // weight of the token at LDS slot s, from its two logits (the same value
  // as from the kept exponentials)
  auto weight = [&](bool q_only, int s) __attribute__((always_inline)) -> double {
    const float eq = ex2(lds_logit<TL>(lq, s), a.c2, mqs);
    return fq * static_cast<double>(q_only ? eq : fmaxf(0.f, __builtin_fmaf(-Kt, ex2(lds_logit<TL>(lp, s), a.c2, mps), eq)));
  };
  // weight and q exponential of this thread's slot i = jj * G + e, from the
  // kept exponentials (regs) or from LDS
  auto slot_weight = [&](bool q_only, bool regs, int jj, int e, float& eq) __attribute__((always_inline)) -> double {
    float ep = 0.f;
    if (kKeep && regs) {
      eq = xq[jj * G + e];
      if (!q_only) ep = xp[jj * G + e];
    } else {
      const int s = group_index<TL>(jj) + e;
      eq = ex2(lds_logit<TL>(lq, s), a.c2, mqs);
      if (!q_only) ep = ex2(lds_logit<TL>(lp, s), a.c2, mps);
    }
    return fq * static_cast<double>(q_only ? eq : fmaxf(0.f, __builtin_fmaf(-Kt, ep, eq)));
  };
  // without replacement: a tried token's terminal weight is the one it kept
  const bool wr_tail = WR && !leaf && !greedy;
  auto kept_weight = [&](int token, double wdef) __attribute__((always_inline)) -> double {
    for (int j = 0; j < nkids; ++j)
      if (sh.wfz[j] >= 0.0 && sh.cand[j].tok == token) return sh.wfz[j];
    return wdef;
  };
  // this thread's group weights gw and its q mass tq
  double gw[NV];
  double tq = 0.0;
  auto group_sums = [&](bool q_only, bool regs) __attribute__((always_inline)) {
    double qa = 0.0;
#pragma unroll
    for (int jj = 0; jj < NV; ++jj) {
      double g = 0.0;
#pragma unroll
      for (int e = 0; e < G; ++e) {
        float eq;
        g += slot_weight(q_only, regs, jj, e, eq);
        qa += static_cast<double>(eq);
      }
      gw[jj] = g;
    }
    tq = qa * fq;
    if (wr_tail && !q_only) {   // replace the formula's weight of each tried token in this thread's groups
      for (int j = 0; j < nkids; ++j) {
        const int slot = sh.cand[j].tok - v0;
        if (sh.wfz[j] >= 0.0 && slot >= 0 && slot < kVocabChunk && sh.cand[j].tok < v1 &&
            (slot / G) % kThreads == tid) {
          const double d = sh.wfz[j] - weight(false, slot);
#pragma unroll
          for (int jj = 0; jj < NV; ++jj)
            if (jj == (slot / G) / kThreads) gw[jj] += d;
        }
      }
    }
  };
  // block exclusive scans of the group weights, one per group column: the
  // starting offset goff of each of this thread's groups inside the chunk,
  // and the chunk total
  double goff[NV];
  double chunk_total = 0.0;
  auto scan_offsets = [&]() __attribute__((always_inline)) {
    double excl[NV];
    __syncthreads();
#pragma unroll
    for (int jj = 0; jj < NV; ++jj) {
      const double incl = wave_scan_add(gw[jj]);
      excl[jj] = wave_prev(incl);
      if ((tid & 63) == 63) sh.gscan[jj][tid >> 6] = incl;
    }
    __syncthreads();
    double base = 0.0;
#pragma unroll
    for (int jj = 0; jj < NV; ++jj) {
      double off = base, tot = 0.0;
#pragma unroll
      for (int wv = 0; wv < kThreads / 64; ++wv) {
        if (wv < (tid >> 6)) off += sh.gscan[jj][wv];
        tot += sh.gscan[jj][wv];
      }
      goff[jj] = off + excl[jj];
      base += tot;
    }
    chunk_total = base;
  };
  int cstar = 0;
  bool degen = false;
  if (!greedy) {
    group_sums(leaf, true);   // the last use of the kept exponentials
    scan_offsets();
    // residual and q masses of every chunk: four words per chunk (low and
    // high halves of the two doubles) whose high halves carry the call's
    // tag, read back by polling the words themselves (as the statistics)
    if (!leaf) {
      const double mqsum = block_reduce(tq, AddD{}, sh.dscr);
      if (tid < 4) {
        const uint64_t bits = __builtin_bit_cast(uint64_t, tid < 2 ? chunk_total : mqsum);
        st_u64(mw + c * 4 + tid, stag | ((tid & 1) ? (bits >> 32) : (bits & 0xFFFFFFFFull)));
      }
    }
    // the chunk holding u * S (wave 0, one chunk per lane; same arithmetic
    // in every workgroup of the node)
    if (tid < 64) {
      // leaf: the chunk statistics already hold every chunk's q mass
      double mr = 0.0, mq = 0.0;
      if (leaf) {
        mr = mq = tid < NC ? sh.cmass[tid] : 0.0;
      } else {
        uint64_t w[4] = {0, 0, 0, 0};
        bool have = tid >= NC, fine = true;
        for (uint32_t it = 0;; ++it) {
          if (!have) {
#pragma unroll
            for (int k = 0; k < 4; ++k) w[k] = ld_u64(mw + tid * 4 + k);
            have = ((w[0] & w[1] & w[2] & w[3]) >> 32) == (stag >> 32) && ((w[0] | w[1] | w[2] | w[3]) >> 32) == (stag >> 32);
          }
          if (__all(have)) break;
          if (it >= limit) {
            fine = false;
            break;
          }
          __builtin_amdgcn_s_sleep(2);
        }
        if (tid == 0) sh.ok = fine ? 1 : 0;
        if (tid < NC) {
          mr = __builtin_bit_cast(double, (w[0] & 0xFFFFFFFFull) | (w[1] << 32));
          mq = __builtin_bit_cast(double, (w[2] & 0xFFFFFFFFull) | (w[3] << 32));
        }
      }
      const double sr = wave_reduce(mr, AddD{});
      const bool degen = !(sr > 0.0);
      const double m = degen ? mq : mr;
      const double S = degen ? wave_reduce(mq, AddD{}) : sr;
      const double thr = decision_uniform(a, b, n, kSampleSlot) * S;
      const double incl = wave_scan_add(m);
      const double excl = incl - m;
      const uint64_t cross = __ballot(tid < NC && incl > thr);
      // rounding: no crossing -> the last chunk with positive mass
      const uint64_t pos = __ballot(tid < NC && m > 0.0);
      const int cs_ = cross ? (__ffsll(static_cast<long long>(cross)) - 1) : (pos ? 63 - __clzll(static_cast<long long>(pos)) : 0);
      const double run = __shfl(excl, cs_);
      if (tid == 0) {
        sh.sample[0] = run;
        sh.sample[1] = S;
        sh.sample[2] = thr;
        sh.iscr[3] = cs_ | (degen ? 0x40000000 : 0);
      }
    }
    __syncthreads();
    if (!leaf && !sh.ok) return fail_internal();
    cstar = sh.iscr[3] & 0x3FFFFFFF;
    degen = (sh.iscr[3] & 0x40000000) != 0;
  }
  stamp(a.stamps, 19);   // the chunk holding u*S is known
  // only the workgroup that samples (the chunk holding u*S; chunk 0 in
  // greedy mode) needs to know whether the walk ends here
  if (c != (greedy ? 0 : cstar)) return;

  // ---- is this node where the walk ends?  The wave gives up as soon as one
  // word rules this node out.
  if (tid < 64) {
    int state = tid < Tr ? 0 : 1;
    bool on = false, fine = true;
    for (uint32_t it = 0;; ++it) {
      if (state == 0) state = walk_state(poll(pubs + tid), true);
      if (__any(state == 2)) break;
      if (__all(state == 1)) {
        on = true;
        break;
      }
      if (it >= limit) {
        fine = false;
        break;
      }
      __builtin_amdgcn_s_sleep(8);
    }
    if (tid == 0) {
      sh.onpath = (on && !tokbad) ? 1 : 0;   // a bad token: the root's workgroup wrote the outputs
      sh.ok = fine ? 1 : 0;
    }
  }
  __syncthreads();
  if (!sh.ok) return fail_internal();
  if (!sh.onpath) return;
  stamp(a.stamps, 20);   // the walk ends here
  const int len = plen - 1;   // accepted draft nodes

  // ---- terminal sample (the workgroup of the chunk holding u*S)
  int final_tok = sh.st.argmax;
  uint32_t extra_flags = 0;
  int extra_near = 0;
  if (!greedy) {
    const double S = sh.sample[1], thr = sh.sample[2];
    const bool q_only = leaf || degen;
    if (degen && !leaf) {   // the residual vanished: sample q instead
      group_sums(true, false);
      scan_offsets();
    }
    // the smallest token whose running sum exceeds u*S.  The first group
    // (in token order) whose range reaches u*S is found by a block minimum;
    // wave 0 then scans that group's G tokens one per lane.  A group
    // starting past u*S offers its first token (rounding hid the crossing
    // just before it, which the near-tie test reports).
    {
      int gfirst = 0x7FFFFFFF;
      double gstart = 0.0;
#pragma unroll
      for (int jj = NV - 1; jj >= 0; --jj) {   // the smallest reaching column wins
        const double st = sh.sample[0] + goff[jj];
        if (st > thr || thr - st < gw[jj] * (1.0 + 1e-9)) {
          gfirst = jj * kThreads + tid;
          gstart = st;
        }
      }
      const int wmin = wave_reduce(gfirst, MinI{});
      if ((tid & 63) == 0) sh.wfirst[tid >> 6] = wmin;
      __syncthreads();
      int gstar = 0x7FFFFFFF;
#pragma unroll
      for (int wv = 0; wv < kThreads / 64; ++wv) gstar = min(gstar, sh.wfirst[wv]);
      if (gfirst == gstar && gstar != 0x7FFFFFFF) sh.sample[3] = gstart;
      __syncthreads();
      if (tid < 64) {
        int hit = -1;
        double lo = 0.0, hi = 0.0;
        if (gstar != 0x7FFFFFFF) {
          const double s0 = sh.sample[3];
          const int t0 = gstar * G;
          double w = 0.0;
          if (tid < G) {
            w = weight(q_only, t0 + tid);
            if (wr_tail && !q_only) w = kept_weight(v0 + t0 + tid, w);
          }
          const double incl = wave_scan_add(w);   // lanes past the group carry 0
          const double cum = s0 + incl;
          const uint64_t over = __ballot(tid < G && (s0 > thr || cum > thr));
          if (over) {
            const int f = __ffsll(static_cast<long long>(over)) - 1;
            hit = t0 + f;
            hi = __shfl(cum, f);
            lo = hi - __shfl(w, f);
            if (s0 > thr) lo = hi = s0;
          } else if (gstar + 1 < NV * kThreads) {   // the crossing fell just past this group
            hit = t0 + G;
            lo = hi = __shfl(cum, G - 1);
          }
        }
        if (tid == 0) {
          const bool ok = hit >= 0 && v0 + hit < v1;
          sh.iscr[1] = ok ? hit : -1;
          sh.iscr[2] = ok ? (((hi - thr) < kNearTie * S || (thr - lo) < kNearTie * S) ? 1 : 0) : 0;
        }
      }
    }
    __syncthreads();
    if (sh.iscr[1] >= 0) {
      extra_near = sh.iscr[2];
      final_tok = v0 + sh.iscr[1];
    } else {
      // rounding left no crossing: the last token of the chunk with positive weight
      int last = -1;
#pragma unroll
      for (int jj = 0; jj < NV; ++jj) {
#pragma unroll
        for (int e = 0; e < G; ++e) {
          const int sl = group_index<TL>(jj) + e;
          float eq;
          double we = slot_weight(q_only, false, jj, e, eq);
          if (wr_tail && !q_only) we = kept_weight(v0 + sl, we);
          if (v0 + sl < v1 && we > 0.0) last = max(last, v0 + sl);
        }
      }
      if (tid == 0) sh.iscr[2] = -1;
      __syncthreads();
      atomicMax(&sh.iscr[2], last);
      __syncthreads();
      final_tok = sh.iscr[2];
    }
    extra_flags = degen ? EAGLE_FLAG_DEGENERATE_RESIDUAL : 0u;
  }

  // flags and near ties along the path (ancestors from memory, this node from LDS)
  if (tid == 0) {
    sh.seqflags = sh.st.flags | extra_flags;
    sh.seqnear = sh.st.near + extra_near;
  }
  __syncthreads();
  if (tid < plen - 1) {
    atomicOr(&sh.seqflags, sh.pflags[path_lds[tid]]);
    atomicAdd(&sh.seqnear, sh.pnear[path_lds[tid]]);
  }
  __syncthreads();
  if (tid == 0) {
    a.accept_len[b] = len;
    a.flags[b] = sh.seqflags;
    a.near_ties[b] = sh.seqnear;
  }
  for (int j = tid; j < T; j += kThreads) {
    a.accepted_nodes[b * T + j] = (j < len) ? path_lds[j + 1] : -1;
    a.out_tokens[b * T + j] = (j < len) ? sh.tok[path_lds[j + 1]] : (j == len ? final_tok : -1);
  }
  stamp(a.stamps, 21);   // outputs written
}

// ------------------------------------------------------ node-parallel path
// For V <= kNodeVocab a node's whole target and draft rows fit one
// 512-thread workgroup (64 tokens per thread and row, their exponentials
// kept in registers: two waves per SIMD with 256 registers each), so one
// workgroup decides the node with block-level reductions only: the
// statistics, the tests in order and the residual rounds.  Every node's
// decisions depend only on its own rows, its children's tokens and its own
// uniforms, so the workgroups never wait for each other: no residency
// requirement, and a large batch is one launch.  sa_finish then walks each
// sequence's decisions and draws the one sample the walk needs, at the node
// where it ends, from that node's rows.
constexpr int kNodeThreads = 512;
constexpr int kNodeWaves = kNodeThreads / 64;
constexpr int kNodePer = kNodeVocab / kNodeThreads;   // tokens per thread and row
static_assert(kNodePer == 64, "64 tokens per thread and row");

struct NodeOut {        // one per (sequence, node), in the handle's NodeState slots
  int32_t kind;         // kNodeLeaf / kNodeAccepted / kNodeRejected; -1 for a padding row
  int32_t outcome;      // the accepted child, else -1
  int32_t argmax;       // greedy mode: the target argmax (the emitted token if the walk ends here)
  uint32_t flags;       // P_ZERO / DEGENERATE_RESIDUAL of the node's tests; NONFINITE: an unusable row
  int32_t near_visit;   // near ties counted when the walk reaches the node (filter boundaries, tests)
  float K;              // the sample's weights are max(0, e_q - K e_p), e = 2^((x - m) c2) (K = 0 at a leaf)
  float mq, mp;         // row maxima
};
static_assert(sizeof(NodeOut) <= sizeof(NodeState), "node outputs live in the NodeState slots");

struct NodeShared {
  int32_t kid[kMaxTree];   // children in ascending index
  int32_t ktok[kMaxTree];
  double qt[kMaxTree], pt[kMaxTree], r[kMaxTree];
  int32_t nkids, nreal;
  double dscr[2 * kNodeWaves];
  float fscr[2 * kNodeWaves];
  int32_t iscr[kNodeWaves];
  int32_t res;
};

// reduction over the workgroup (all threads call; the result in every thread)
template <typename T, typename Op>
__device__ T node_reduce(T v, Op op, T* scratch /* >= kNodeWaves */) {
  v = wave_reduce(v, op);
  __syncthreads();   // the previous use of scratch is over
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
  __syncthreads();
  T r = scratch[0];
#pragma unroll
  for (int i = 1; i < kNodeWaves; ++i) r = op(r, scratch[i]);
  return r;
}

// the same for two values at once (scratch >= 2 kNodeWaves)
template <typename T, typename Op>
__device__ void node_reduce2(T& x, T& y, Op op, T* scratch) {
  x = wave_reduce(x, op);
  y = wave_reduce(y, op);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    scratch[threadIdx.x >> 6] = x;
    scratch[kNodeWaves + (threadIdx.x >> 6)] = y;
  }
  __syncthreads();
  x = scratch[0];
  y = scratch[kNodeWaves];
#pragma unroll
  for (int i = 1; i < kNodeWaves; ++i) {
    x = op(x, scratch[i]);
    y = op(y, scratch[kNodeWaves + i]);
  }
}

template <int NV>
__device__ __forceinline__ void words_opaque(u32x4_t (&w)[NV]) {
#pragma unroll
  for (int jj = 0; jj < NV; ++jj) asm volatile("" : "+v"(w[jj]));
}

// This thread's kNodePer logits in the strided group view: word jj holds the
// G consecutive tokens of group g = jj * kNodeThreads + tid, i.e. tokens
// g G .. g G + G - 1 (token order is group order, and the lanes of a wave
// read consecutive 16-byte groups); -inf past the row.  VEC: the row starts
// on a 16-byte boundary and holds whole 16-byte groups.
template <typename TL>
__device__ __forceinline__ int node_token(int jj, int e) {
  return (jj * kNodeThreads + static_cast<int>(threadIdx.x)) * Pack<TL>::G + e;
}
template <typename TL, bool VEC>
__device__ __forceinline__ void node_load(const TL* row, int V, u32x4_t (&w)[kNodePer / Pack<TL>::G]) {
  // aligned rows: every load is issued (from the row's start when past its
  // end) and -inf selected afterwards, with no branch between the loads, so
  // that all of them are in flight at once.  Unaligned rows (rare): words
  // inside the row for every thread load without a select (fewer address
  // registers), the last ones element by element.
  constexpr int G = Pack<TL>::G;
  const uint32_t ni = Pack<TL>::neg_inf_word();
#pragma unroll
  for (int jj = 0; jj < kNodePer / G; ++jj) {
    const int t0 = node_token<TL>(jj, 0);
    if constexpr (VEC) {
      const u32x4_t x = *reinterpret_cast<const u32x4_t*>(row + (t0 < V ? t0 : 0));
#pragma unroll
      for (int i = 0; i < 4; ++i) w[jj][i] = t0 < V ? x[i] : ni;
    } else if ((jj + 1) * kNodeThreads * G <= V) {   // (uniform) inside the row for every thread
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (sizeof(TL) == 2)
          w[jj][i] = static_cast<uint32_t>(row[t0 + 2 * i]) | (static_cast<uint32_t>(row[t0 + 2 * i + 1]) << 16);
        else
          w[jj][i] = __float_as_uint(row[t0 + i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (sizeof(TL) == 2) {
          const int t = t0 + 2 * i;
          const uint32_t lo = static_cast<uint32_t>(row[t < V ? t : 0]);
          const uint32_t hi = static_cast<uint32_t>(row[t + 1 < V ? t + 1 : 0]) << 16;
          w[jj][i] = (t < V ? lo : (ni & 0xFFFFu)) | (t + 1 < V ? hi : (ni & 0xFFFF0000u));
        } else {
          const int t = t0 + i;
          const uint32_t x = __float_as_uint(row[t < V ? t : 0]);
          w[jj][i] = t < V ? x : ni;
        }
      }
    }
  }
}

template <typename TL, bool VEC>
__global__ __launch_bounds__(kNodeThreads) void sa_node(const AcceptKernelArgs a) {
  __shared__ NodeShared sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.T, V = a.V;
  const int b = blockIdx.x / T, n = blockIdx.x - b * T;
  NodeOut* const out = reinterpret_cast<NodeOut*>(a.nodes) + static_cast<int64_t>(b) * T + n;
  const bool greedy = a.tau == 0.f;
  stamp(a.stamps, 0);
  stamp_value(a.stamps, 29, a.stamps ? placement() : 0);

  // the tree (wave 0, lane = row): this node's children in ascending index
  if (wave == 0) {
    const int par = lane < T ? a.parents[b * T + lane] : -1;
    const int tok = lane < T ? a.tokens[b * T + lane] : -1;
    const uint64_t padm = __ballot(lane >= 1 && lane < T && tok == -1);
    const int nreal = padm ? __ffsll(static_cast<long long>(padm)) - 1 : T;
    const bool is_child = lane > n && lane < nreal && par == n;
    const uint64_t km = __ballot(is_child);
    if (is_child) {
      const int ord = __popcll(km & ((1ull << lane) - 1ull));
      sh.kid[ord] = lane;
      sh.ktok[ord] = tok;
    }
    if (lane == 0) {
      sh.nkids = __popcll(km);
      sh.nreal = nreal;
    }
  }
  __syncthreads();
  if (n >= sh.nreal) {   // a padding row: never read, never on a walk
    if (tid == 0) *out = NodeOut{-1, -1, -1, 0u, 0, 0.f, 0.f, 0.f};
    return;
  }
  const int nkids = sh.nkids;
  const bool two = nkids > 0 && !greedy;
  const int64_t rowoff = static_cast<int64_t>(b * T + n) * V;
  const TL* const trow = reinterpret_cast<const TL*>(a.target) + rowoff;
  const TL* const drow = reinterpret_cast<const TL*>(a.draft) + rowoff;

  // both rows requested at once, except fp32 rows (64 registers each): the
  // draft row there once the target row's exponentials exist
  constexpr int G = Pack<TL>::G, NV = kNodePer / G;
  constexpr bool kLateDraft = sizeof(TL) == 4;
  u32x4_t wq[NV], wd[NV];
  node_load<TL, VEC>(trow, V, wq);
  if (two && !kLateDraft) node_load<TL, VEC>(drow, V, wd);
  if (a.thr) cut_groups<TL, NV>(wq, thr_of(a, b, n, 0));   // filtered: logits below the threshold count as -inf

  if (greedy) {   // the target argmax (lowest id), matched against the children's tokens
    const float mq = node_reduce(local_max<TL, NV>(wq), MaxOp{}, sh.fscr);
    stamp(a.stamps, 1);   // rows in, their maxima
    if (mq == __builtin_inff() || mq == kNegInf) {   // an unusable row poisons the sequence (the walk reports it)
      if (tid == 0) *out = NodeOut{kNodeRejected, -1, -1, static_cast<uint32_t>(EAGLE_FLAG_NONFINITE), 0, 0.f, 0.f, 0.f};
      return;
    }
    int la = 0x7FFFFFFF;
#pragma unroll
    for (int jj = NV - 1; jj >= 0; --jj) {
      float f[G];
      Pack<TL>::unpack(wq[jj], f);
#pragma unroll
      for (int e = G - 1; e >= 0; --e)
        if (f[e] == mq) la = node_token<TL>(jj, e);
    }
    const int am = node_reduce(la, MinI{}, sh.iscr);
    if (tid == 0) {
      int acc = -1;
      for (int i = 0; i < nkids; ++i)
        if (sh.ktok[i] == am) {
          acc = sh.kid[i];
          break;
        }
      *out = NodeOut{acc >= 0 ? kNodeAccepted : (nkids ? kNodeRejected : kNodeLeaf), acc, am, 0u, 0, 0.f, mq, 0.f};
    }
    return;
  }

  // each row's exponentials 2^((x - m) c2), kept in registers (token
  // node_token(jj, e) at index jj G + e; sums in fp64), the target row first,
  // so that a row's logits die before the next row's exponentials are made;
  // the exponentials unpack the words again rather than keeping unpacked
  // logits live across the reduction
  float xq[kNodePer], xp[kNodePer];
  const float mq = node_reduce(local_max<TL, NV>(wq), MaxOp{}, sh.fscr);
  stamp(a.stamps, 1);   // target row in, its maximum
  if (nkids == 0) {
    // a leaf: a walk that ends here samples from its target row, whose
    // weights the sampling kernel makes again against this maximum; the
    // row's sum is not needed
    stamp(a.stamps, 3);
    stamp_value(a.stamps, 30, static_cast<uint64_t>(kNodeLeaf));
    if (tid == 0)
      *out = (mq == __builtin_inff() || mq == kNegInf)
                 ? NodeOut{kNodeRejected, -1, -1, static_cast<uint32_t>(EAGLE_FLAG_NONFINITE), 0, 0.f, 0.f, 0.f}
                 : NodeOut{kNodeLeaf, -1, -1, 0u, filter_near(a, b, n, false), 0.f, mq, 0.f};
    return;
  }
  words_opaque<NV>(wq);
  double zq = local_expsum_keep<TL, NV>(wq, mq, a.c2, xq);
  float mp = 0.f;
  double zp = 0.0;
  if (two) {
    if (kLateDraft) node_load<TL, VEC>(drow, V, wd);
    if (a.thr) cut_groups<TL, NV>(wd, thr_of(a, b, n, 1));
    mp = node_reduce(local_max<TL, NV>(wd), MaxOp{}, sh.fscr);
    words_opaque<NV>(wd);
    zp = local_expsum_keep<TL, NV>(wd, mp, a.c2, xp);
  }
  if (mq == __builtin_inff() || mq == kNegInf || (two && (mp == __builtin_inff() || mp == kNegInf))) {
    // an unusable row (the walk reports it)
    if (tid == 0) *out = NodeOut{kNodeRejected, -1, -1, static_cast<uint32_t>(EAGLE_FLAG_NONFINITE), 0, 0.f, 0.f, 0.f};
    return;
  }
  node_reduce2(zq, zp, AddD{}, sh.dscr);
  const double fq = 1.0 / zq, fp = two ? 1.0 / zp : 0.0;
  stamp(a.stamps, 2);   // row statistics

  uint32_t fl = 0;
  int32_t nr = filter_near(a, b, n, nkids > 0);
  int kind = kNodeLeaf, outcome = -1;
  double C = 0.0;
  if (nkids > 0) {
    // q(t), p(t) and the uniform of every test, one child per lane
    if (tid < nkids) {
      const int tok = sh.ktok[tid];
      double qt = 0.0, pt = 0.0;
      if (tok >= 0 && tok < V) {
        qt = exp((static_cast<double>(cut(logit<TL>(trow, tok), thr_of(a, b, n, 0))) - mq) * a.inv_tau) / zq;
        pt = exp((static_cast<double>(cut(logit<TL>(drow, tok), thr_of(a, b, n, 1))) - mp) * a.inv_tau) / zp;
      }
      sh.qt[tid] = qt;
      sh.pt[tid] = pt;
      sh.r[tid] = decision_uniform(a, b, n, static_cast<uint32_t>(tid));
    }
    // children in order under the residual max(0, q - C p) / s
    double s = 1.0;
    kind = kNodeRejected;
    for (int i = 0; i < nkids; ++i) {
      __syncthreads();
      if (tid == 0) sh.res = decide_pre(sh.qt[i], sh.pt[i], sh.r[i], sh.ktok[i], V, C, s, fl, nr);
      __syncthreads();
      const int res = sh.res;
      if (res > 0) {
        kind = kNodeAccepted;
        outcome = sh.kid[i];
        break;
      }
      if (res < 0) break;   // a token outside the vocabulary (the walk reports it)
      C += s;
      // the residual mass after this rejection (after the last one it is
      // the sample's distribution)
      const double part = kept_masses(xq, xp, static_cast<float>(C * fp / fq), fq);
      s = node_reduce(part, AddD{}, sh.dscr);
      if (!(s > 0.0)) {   // nothing left: the residual starts over from q
        fl |= EAGLE_FLAG_DEGENERATE_RESIDUAL;
        C = 0.0;
        s = 1.0;
      }
    }
  }
  stamp(a.stamps, 3);   // tests and residual rounds done
  stamp_value(a.stamps, 30, static_cast<uint64_t>(kind));
  if (tid == 0) {
    const float K = kind == kNodeRejected ? static_cast<float>(C * fp / fq) : 0.f;
    *out = NodeOut{kind, outcome, -1, fl, nr, K, mq, two ? mp : 0.f};
  }
}

// One 512-thread workgroup per sequence: wave 0 validates the tree and walks
// the decided nodes from the root; then (sampled mode) the whole workgroup
// draws the emitted token at the node where the walk ends, from that node's
// rows: the smallest token whose running sum of the weights max(0, e_q -
// K e_p) exceeds u * S (e_q alone at a leaf), the exponentials recomputed
// exactly as the node's workgroup computed them.  In token order: per-group
// sums (a thread's word jj is group jj * kNodeThreads + tid), one block scan
// per group column, the first group reaching u * S by a block minimum, then
// that group's G tokens in order by the thread that holds it.
template <typename TL, bool VEC>
__global__ __launch_bounds__(kNodeThreads) void sa_finish(const AcceptKernelArgs a) {
  __shared__ NodeOut no[kMaxTree];
  __shared__ int32_t path[kMaxTree];
  __shared__ int32_t walk[4];   // length, final node, bad flags, 0
  __shared__ uint32_t wflags;
  __shared__ int32_t wnear;
  __shared__ double cscan[kNodePer / 4][kNodeWaves];   // per group column and wave: weight totals
  __shared__ int32_t iscr[kNodeWaves];
  __shared__ int32_t hit, hitnear;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x, T = a.T, V = a.V;
  const int64_t mslot = static_cast<int64_t>(a.B) * T + b;   // timeline slot
  if (a.stamps && tid == 0) a.stamps[mslot * 32] = __builtin_amdgcn_s_memrealtime();
  if (wave == 0) {
    const int par = lane < T ? a.parents[b * T + lane] : -1;
    const int tok = lane < T ? a.tokens[b * T + lane] : -1;
    const bool tree_bad = __any(lane < T && (lane == 0 ? par != -1 : (par < 0 || par >= lane)));
    const uint64_t padm = __ballot(lane >= 1 && lane < T && tok == -1);
    const int nreal = padm ? __ffsll(static_cast<long long>(padm)) - 1 : T;
    const bool pad_bad = __any(lane >= nreal && lane < T && tok != -1);   // padding must be a suffix
    const bool tok_bad = __any(lane >= 1 && lane < nreal && (tok < 0 || tok >= V));
    if (lane < nreal) no[lane] = reinterpret_cast<const NodeOut*>(a.nodes)[static_cast<int64_t>(b) * T + lane];
    const bool nonfinite = __any(lane < nreal && (no[lane].flags & EAGLE_FLAG_NONFINITE));
    uint32_t bad = 0;
    if (tree_bad || pad_bad) bad = EAGLE_FLAG_BAD_TREE;
    else bad = (tok_bad ? EAGLE_FLAG_BAD_TOKEN : 0u) | (nonfinite ? EAGLE_FLAG_NONFINITE : 0u);
    if (lane == 0) {
      walk[2] = static_cast<int32_t>(bad);
      if (!bad) {
        int cur = 0, len = 0, near = 0;
        uint32_t fl = 0;
        for (;;) {
          const NodeOut o = no[cur];
          fl |= o.flags;
          near += o.near_visit;
          if (o.kind != kNodeAccepted) break;
          path[len++] = o.outcome;
          cur = o.outcome;
        }
        walk[0] = len;
        walk[1] = cur;
        wflags = fl;
        wnear = near;
      }
    }
  }
  __syncthreads();
  const uint32_t bad = static_cast<uint32_t>(walk[2]);
  if (bad) {   // an unusable input: every integer output -1
    if (tid == 0) {
      a.accept_len[b] = -1;
      a.flags[b] = bad;
      a.near_ties[b] = 0;
    }
    for (int j = tid; j < T; j += kNodeThreads) {
      a.accepted_nodes[b * T + j] = -1;
      a.out_tokens[b * T + j] = -1;
    }
    return;
  }
  const int len = walk[0], nt = walk[1];
  const NodeOut o = no[nt];
  int final_tok;
  int near_end = 0;
  if (a.tau == 0.f) {
    final_tok = o.argmax;
  } else {
    constexpr int G = Pack<TL>::G, NV = kNodePer / G;
    const bool leaf = o.kind == kNodeLeaf;
    const int64_t rowoff = static_cast<int64_t>(b * T + nt) * V;
    u32x4_t wq[NV], wd[NV];
    node_load<TL, VEC>(reinterpret_cast<const TL*>(a.target) + rowoff, V, wq);
    if (a.thr) cut_groups<TL, NV>(wq, thr_of(a, b, nt, 0));
    if (leaf) {   // no draft term: logits 0 against the maximum 0 give e_p = 1, and K = 0
#pragma unroll
      for (int jj = 0; jj < NV; ++jj) wd[jj] = u32x4_t{0u, 0u, 0u, 0u};
    } else {
      node_load<TL, VEC>(reinterpret_cast<const TL*>(a.draft) + rowoff, V, wd);
      if (a.thr) cut_groups<TL, NV>(wd, thr_of(a, b, nt, 1));
    }
    const float K = leaf ? 0.f : o.K, mp = leaf ? 0.f : o.mp;
    // the weights of this thread's tokens, summed per group (the
    // exponentials as the node's workgroup made them: ex2 of the same logits
    // against the same maxima)
    auto weight = [&](float xq_, float xp_) __attribute__((always_inline)) {
      return fmaxf(0.f, __builtin_fmaf(-K, ex2(xp_, a.c2, mp), ex2(xq_, a.c2, o.mq)));
    };
    double gw[NV], goff[NV];
    int lastpos = -1;   // this thread's last token with positive weight
#pragma unroll
    for (int jj = 0; jj < NV; ++jj) asm volatile("" : "+v"(wq[jj]), "+v"(wd[jj]));
#pragma unroll
    for (int jj = 0; jj < NV; ++jj) {
      float fq_[G], fp_[G];
      Pack<TL>::unpack(wq[jj], fq_);
      Pack<TL>::unpack(wd[jj], fp_);
      double g = 0.0;
#pragma unroll
      for (int e = 0; e < G; ++e) {
        const float w = weight(fq_[e], fp_[e]);
        g += static_cast<double>(w);
        if (w > 0.f) lastpos = node_token<TL>(jj, e);
      }
      gw[jj] = g;
    }
    __builtin_amdgcn_sched_barrier(0);
    // per-column exclusive offsets of this thread's groups, column totals
#pragma unroll
    for (int jj = 0; jj < NV; ++jj) {
      const double incl = wave_scan_add(gw[jj]);
      goff[jj] = incl - gw[jj];
      if (lane == 63) cscan[jj][wave] = incl;
    }
    __syncthreads();
    double base = 0.0;
#pragma unroll
    for (int jj = 0; jj < NV; ++jj) {
      double off = base, tot = 0.0;
#pragma unroll
      for (int w = 0; w < kNodeWaves; ++w) {
        if (w < wave) off += cscan[jj][w];
        tot += cscan[jj][w];
      }
      goff[jj] += off;
      base += tot;
      __builtin_amdgcn_sched_barrier(0);   // one column's LDS words in flight at a time
    }
    const double S = base;
    const double thr = decision_uniform(a, b, nt, kSampleSlot) * S;
    // the first group (in token order) whose range reaches past u * S
    int gfirst = 0x7FFFFFFF;
#pragma unroll
    for (int jj = NV - 1; jj >= 0; --jj)
      if (goff[jj] + gw[jj] > thr) gfirst = jj * kNodeThreads + tid;
    const int gstar = node_reduce(gfirst, MinI{}, iscr);
    if (gstar != 0x7FFFFFFF && gfirst == gstar) {
      // that group's tokens again, from the rows (the same logits, so the
      // same weights), in token order from the group's offset
      const int js = gstar / kNodeThreads;
      double hi = 0.0;
#pragma unroll
      for (int jj = 0; jj < NV; ++jj)
        if (jj == js) hi = goff[jj];
      const float thq = a.thr ? thr_of(a, b, nt, 0) : kNegInf, thp = a.thr ? thr_of(a, b, nt, 1) : kNegInf;
      const TL* const tr = reinterpret_cast<const TL*>(a.target) + rowoff;
      const TL* const dr = reinterpret_cast<const TL*>(a.draft) + rowoff;
      float lq[G], lp[G];
#pragma unroll
      for (int e = 0; e < G; ++e) {
        const int t = gstar * G + e;
        lq[e] = t < V ? cut(logit<TL>(tr, t), thq) : kNegInf;
        lp[e] = leaf ? 0.f : (t < V ? cut(logit<TL>(dr, t), thp) : kNegInf);
      }
      int v = -1, lastg = -1;
      double lo = hi;
#pragma unroll
      for (int e = 0; e < G; ++e) {
        const double w = weight(lq[e], lp[e]);
        if (w > 0.0) {
          lastg = gstar * G + e;
          if (v < 0) {
            lo = hi;
            hi += w;
            if (hi > thr) v = lastg;
          }
        }
      }
      if (v < 0) {   // rounding hid the crossing inside this group: its last positive weight
        v = lastg;
        lo = hi = thr;
      }
      hit = v;
      hitnear = ((hi - thr) < kNearTie * S || (thr - lo) < kNearTie * S) ? 1 : 0;
    }
    if (gstar == 0x7FFFFFFF) {   // no crossing at all: the last token with positive weight
      const int lm = node_reduce(lastpos, [](int x, int y) { return x > y ? x : y; }, iscr);
      if (tid == 0) {
        hit = lm;
        hitnear = 0;
      }
    }
    __syncthreads();
    final_tok = hit;
    near_end = hitnear;
  }
  if (tid == 0) {
    a.accept_len[b] = len;
    a.flags[b] = wflags;
    a.near_ties[b] = wnear + near_end;
  }
  for (int j = tid; j < T; j += kNodeThreads) {
    a.accepted_nodes[b * T + j] = j < len ? path[j] : -1;
    a.out_tokens[b * T + j] = j < len ? a.tokens[b * T + path[j]] : (j == len ? final_tok : -1);
  }
  if (a.stamps && tid == 0) a.stamps[mslot * 32 + 1] = __builtin_amdgcn_s_memrealtime();
}

// The fused kernel's workgroups wait for each other: launched cooperatively,
// the runtime either makes all of them resident at once or refuses the
// launch (hipErrorCooperativeLaunchTooLarge, nothing enqueued; the caller
// then takes the three-kernel path).
hipError_t launch_fused(const void* fn, dim3 grid, dim3 block, const AcceptKernelArgs& a, hipStream_t st) {
  void* args[] = {const_cast<AcceptKernelArgs*>(&a)};
  if (a.coop) return hipLaunchCooperativeKernel(fn, grid, block, args, 0, st);
  return hipLaunchKernel(fn, grid, block, args, 0, st);
}

template <typename TL>
hipError_t launch_t(const AcceptKernelArgs& a, hipStream_t st) {
  const dim3 block(kThreads);
  if (a.fused == 2) {   // node-parallel path (V <= kNodeVocab, siblings with replacement)
    const dim3 grid(static_cast<unsigned>(a.B * a.T));
    if (a.vec_ok) hipLaunchKernelGGL((sa_node<TL, true>), grid, dim3(kNodeThreads), 0, st, a);
    else hipLaunchKernelGGL((sa_node<TL, false>), grid, dim3(kNodeThreads), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.vec_ok) hipLaunchKernelGGL((sa_finish<TL, true>), dim3(static_cast<unsigned>(a.B)), dim3(kNodeThreads), 0, st, a);
    else hipLaunchKernelGGL((sa_finish<TL, false>), dim3(static_cast<unsigned>(a.B)), dim3(kNodeThreads), 0, st, a);
    return hipGetLastError();
  }
  if (a.fused) {
    const dim3 grid(static_cast<unsigned>(a.B * a.T * a.NC));
    const void* fn = a.wr ? (a.vec_ok ? reinterpret_cast<const void*>(&sa_fused<TL, true, true>)
                                      : reinterpret_cast<const void*>(&sa_fused<TL, false, true>))
                          : (a.vec_ok ? (a.leaf_wait > 0 ? reinterpret_cast<const void*>(&sa_fused<TL, true, false, true>)
                                                         : reinterpret_cast<const void*>(&sa_fused<TL, true, false>))
                                      : reinterpret_cast<const void*>(&sa_fused<TL, false, false>));
    return launch_fused(fn, grid, block, a, st);
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
  // every loader and sibling-rule variant must fit: the smallest occupancy decides
  int per_cu = 1 << 30;
  const void* kernels[5] = {
      logits_bf16 ? reinterpret_cast<const void*>(&sa_fused<uint16_t, true, false, true>) : reinterpret_cast<const void*>(&sa_fused<float, true, false, true>),
      logits_bf16 ? reinterpret_cast<const void*>(&sa_fused<uint16_t, true, false>) : reinterpret_cast<const void*>(&sa_fused<float, true, false>),
      logits_bf16 ? reinterpret_cast<const void*>(&sa_fused<uint16_t, false, false>) : reinterpret_cast<const void*>(&sa_fused<float, false, false>),
      logits_bf16 ? reinterpret_cast<const void*>(&sa_fused<uint16_t, true, true>) : reinterpret_cast<const void*>(&sa_fused<float, true, true>),
      logits_bf16 ? reinterpret_cast<const void*>(&sa_fused<uint16_t, false, true>) : reinterpret_cast<const void*>(&sa_fused<float, false, true>)};
  for (const void* k : kernels) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k, kThreads, 0) != hipSuccess || n <= 0) return 0;
    per_cu = n < per_cu ? n : per_cu;
  }
  return per_cu * num_cus;
}

int launch_spec_accept(const AcceptKernelArgs& args, int logits_bf16, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const hipError_t e = logits_bf16 ? launch_t<uint16_t>(args, st) : launch_t<float>(args, st);
  return static_cast<int>(e);
}

}  // namespace ev
