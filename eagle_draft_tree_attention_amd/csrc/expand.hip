// One expansion step of a dynamic draft tree (EAGLE-2), gfx950 (MI355X).
//
// Rule (EAGLE notes page, the EAGLE-2 section: the draft model's confidence
// tracks the acceptance rate, so the tree grows where the cumulative
// confidence of a path is high; the tree-drafting section: greedy drafting
// takes each node's top-k children by probability).  Frontier node f carries
// the log-probability s_f of its path and the draft logits x_f; with
// p_f = softmax(x_f / t) its candidates are its k most probable tokens
// (largest logit first, ties to the lower id), valued s_f + log p_f(token);
// the M candidates of largest value are kept, ties to the lower frontier
// index, then the lower token id.
//
// GPU formulation, two launches:
//   te_chunk   one workgroup per (sequence, frontier row, vocabulary chunk of
//              2048, 4096 or 8192 tokens, at most 64 chunks a row):
//              the chunk's maximum, its sum of exp((x - max)/t) (fp32
//              exponentials, fp64 sum), NaN/+inf detection and its k largest
//              logits with their ids (k rounds of a wave argmax per wave, then
//              a merge of the four waves' lists); one record per chunk.
//   te_select  one workgroup per sequence: one wave per frontier row reads
//              the row's score and chunk records in one round trip (lane c:
//              chunk c, its sorted list kept in registers), reduces the row's
//              maximum and normaliser, takes its top k as a k-step merge of
//              the chunks' lists and values them s_f + (x - max)/t - log Z in
//              fp64 (the row's candidates go to LDS); then every candidate is
//              ranked by counting the candidates before it (value, then
//              frontier index, then position in its row) and written to its
//              slot; adjacent ranks up to the kept/dropped boundary are
//              tested for near ties.
//   te_rerank  (separate call) the final tree from the chained steps.
// Within a row the value is a monotone function of the logit, so a row's
// list sorted by logit is sorted by value too.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ev_internal.h"

namespace ev {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr float kNegInf = -__builtin_inff();
constexpr double kNear = 1e-6;                      // near-tie margin of the ranking (log-probability units)

template <typename TL>
__device__ __forceinline__ float logit_at(const TL* row, int v) {
  if constexpr (sizeof(TL) == 2) return __uint_as_float(static_cast<uint32_t>(row[v]) << 16);
  else return row[v];
}

// ---- wave reductions through DPP: row shifts 1, 2, 4, 8 (a scan within each
// row of 16 lanes), then row broadcasts 15 and 31, so that lane 63 ends up
// with the reduction of all 64 lanes; read out as a wave-uniform value.  Only
// the ALU pipeline is used (no LDS round trips as with lane shuffles).  Every
// lane of the wave must be active.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t old, uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(static_cast<int>(old), static_cast<int>(v), CTRL, ROW_MASK, 0xf, false));
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_mov64(uint64_t old, uint64_t v) {
  const uint32_t lo = dpp_mov<CTRL, ROW_MASK>(static_cast<uint32_t>(old), static_cast<uint32_t>(v));
  const uint32_t hi = dpp_mov<CTRL, ROW_MASK>(static_cast<uint32_t>(old >> 32), static_cast<uint32_t>(v >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

template <typename Op>
__device__ __forceinline__ uint64_t wave_reduce64(uint64_t x, const uint64_t ident, Op op) {
  x = op(x, dpp_mov64<0x111, 0xf>(ident, x));   // row_shr:1
  x = op(x, dpp_mov64<0x112, 0xf>(ident, x));   // row_shr:2
  x = op(x, dpp_mov64<0x114, 0xf>(ident, x));   // row_shr:4
  x = op(x, dpp_mov64<0x118, 0xf>(ident, x));   // row_shr:8 (lane 15 of a row: the row)
  x = op(x, dpp_mov64<0x142, 0xa>(ident, x));   // row_bcast:15 into rows 1 and 3
  x = op(x, dpp_mov64<0x143, 0xc>(ident, x));   // row_bcast:31 into rows 2 and 3
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), 63));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x >> 32), 63));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce32(uint32_t x, const uint32_t ident, Op op) {
  x = op(x, dpp_mov<0x111, 0xf>(ident, x));
  x = op(x, dpp_mov<0x112, 0xf>(ident, x));
  x = op(x, dpp_mov<0x114, 0xf>(ident, x));
  x = op(x, dpp_mov<0x118, 0xf>(ident, x));
  x = op(x, dpp_mov<0x142, 0xa>(ident, x));
  x = op(x, dpp_mov<0x143, 0xc>(ident, x));
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), 63));
}

__device__ __forceinline__ uint64_t max_u64(uint64_t p, uint64_t q) { return p > q ? p : q; }
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) { return wave_reduce64(x, 0ull, max_u64); }

__device__ __forceinline__ float wave_max_f32(float x) {
  return __uint_as_float(wave_reduce32(__float_as_uint(x), __float_as_uint(kNegInf),
                                       [](uint32_t p, uint32_t q) { return __float_as_uint(fmaxf(__uint_as_float(p), __uint_as_float(q))); }));
}

__device__ __forceinline__ double wave_sum_f64(double x) {
  return __longlong_as_double(static_cast<long long>(wave_reduce64(
      static_cast<uint64_t>(__double_as_longlong(x)), 0ull, [](uint64_t p, uint64_t q) {
        return static_cast<uint64_t>(__double_as_longlong(__longlong_as_double(static_cast<long long>(p)) +
                                                          __longlong_as_double(static_cast<long long>(q))));
      })));
}

// Order-preserving keys: a larger key is a larger number (-0 and +0 map to
// one key, as they compare equal); key 0 lies below every number's key.
__device__ __forceinline__ uint32_t ord32(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);   // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unord32(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}
__device__ __forceinline__ uint64_t ord64(double d) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(d + 0.0));
  return (u >> 63) ? ~u : (u | (1ull << 63));
}
__device__ __forceinline__ double unord64(uint64_t k) {
  return __longlong_as_double(static_cast<long long>((k >> 63) ? (k & ~(1ull << 63)) : ~k));
}

// (logit, token) key of the top-k lists: larger logit first, then lower token
// id; 0 = no entry
__device__ __forceinline__ uint64_t cand_key(float x, int id) {
  return (static_cast<uint64_t>(ord32(x)) << 32) | static_cast<uint32_t>(~id);
}
__device__ __forceinline__ float key_logit(uint64_t k) { return unord32(static_cast<uint32_t>(k >> 32)); }
__device__ __forceinline__ int key_token(uint64_t k) { return static_cast<int>(~static_cast<uint32_t>(k)); }

// EPT logits per thread: chunks of 256 * EPT tokens (2048, 4096 or 8192,
// the smallest that keeps a row within 64 chunks)
template <typename TL, int EPT>
__global__ __launch_bounds__(kThreads) void te_chunk(const ExpandKernelArgs a) {
  constexpr int kPerThread = EPT;
  constexpr int kChunk = kThreads * EPT;
  __shared__ float rmax[kThreads / 64];
  __shared__ uint32_t rbad[kThreads / 64];
  __shared__ double rsum[kThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int NC = a.NC, V = a.V, K = a.K;
  const int c = blockIdx.x % NC;
  const int row = blockIdx.x / NC;   // b * F + f
  const TL* x = reinterpret_cast<const TL*>(a.logits) + static_cast<int64_t>(row) * V;
  const int v0 = c * kChunk, v1 = min(V, v0 + kChunk);

  // this thread's logits: tokens v0 + tid + 256 j
  float xs[kPerThread];
  float m = kNegInf;
  uint32_t bad = 0;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const int v = v0 + tid + kThreads * j;
    xs[j] = v < v1 ? logit_at<TL>(x, v) : kNegInf;
    if (xs[j] != xs[j] || xs[j] == __builtin_inff()) bad = 1;
    else m = fmaxf(m, xs[j]);
  }
  // block maximum and bad flag
  m = wave_max_f32(m);
  bad = __any(bad != 0) ? 1u : 0u;
  if (lane == 0) {
    rmax[wave] = m;
    rbad[wave] = bad;
  }
  __syncthreads();
  m = fmaxf(fmaxf(rmax[0], rmax[1]), fmaxf(rmax[2], rmax[3]));
  bad = rbad[0] | rbad[1] | rbad[2] | rbad[3];
  // sum of exp((x - m) / t) over the chunk: fp32 exponentials, fp64 sum
  double z = 0.0;
  if (m != kNegInf) {
    const float mc = -m * a.c2;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) z += static_cast<double>(__builtin_amdgcn_exp2f(__builtin_fmaf(xs[j], a.c2, mc)));
  }
  z = wave_sum_f64(z);
  if (lane == 0) rsum[wave] = z;

  // top K of the chunk: each wave first takes the K largest of its 64 * EPT
  // logits in K rounds (each lane offers its best not yet taken, the wave
  // keeps the winner), then wave 0 merges the four waves' sorted lists.
  // NaN and +inf are never candidates (the row is unusable anyway), -inf
  // neither.  Within a lane, a lower j is a lower token id.
#pragma unroll
  for (int j = 0; j < kPerThread; ++j)
    if (!(xs[j] < __builtin_inff())) xs[j] = kNegInf;
  __shared__ float wl_v[kThreads / 64][kMaxTopK];
  __shared__ int wl_i[kThreads / 64][kMaxTopK];
  uint32_t taken = 0;
  for (int q = 0; q < K; ++q) {
    float lb = kNegInf;
    int lj = -1;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j)
      if (!((taken >> j) & 1u) && xs[j] > lb) {
        lb = xs[j];
        lj = j;
      }
    const uint64_t key = lj >= 0 ? cand_key(lb, v0 + tid + kThreads * lj) : 0ull;
    const uint64_t best = wave_max_u64(key);
    if (lj >= 0 && key == best) taken |= 1u << lj;   // token ids are unique: one lane wins
    if (lane == 0) {
      wl_v[wave][q] = best ? key_logit(best) : kNegInf;
      wl_i[wave][q] = best ? key_token(best) : -1;
    }
  }
  __syncthreads();
  ChunkRecord* const rec = a.chunks + static_cast<int64_t>(row) * NC + c;
  if (tid == 0) {
    rec->m = m;
    rec->bad = bad;
    rec->z = (rsum[0] + rsum[1]) + (rsum[2] + rsum[3]);
  }
  if (wave == 0) {   // lanes 0..3 hold the heads of the four waves' lists
    int hd = 0;
    for (int q = 0; q < K; ++q) {
      const uint64_t key = (lane < kThreads / 64 && hd < K && wl_i[lane][hd] >= 0)
                               ? cand_key(wl_v[lane][hd], wl_i[lane][hd]) : 0ull;
      uint64_t best = max_u64(key, dpp_mov64<0xB1, 0xf>(0ull, key));   // quad_perm 1,0,3,2
      best = max_u64(best, dpp_mov64<0x4E, 0xf>(0ull, best));          // quad_perm 2,3,0,1
      best = (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(best >> 32), 0))) << 32) |
             static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(best), 0));
      if (key != 0ull && key == best) ++hd;
      if (lane == 0) {
        rec->val[q] = best ? key_logit(best) : kNegInf;
        rec->id[q] = best ? key_token(best) : -1;
      }
    }
  }
}

constexpr int kSelWaves = 8;   // frontier rows worked on at once by one workgroup
constexpr int kRecVal = static_cast<int>(offsetof(ChunkRecord, val));
constexpr int kRecId = static_cast<int>(offsetof(ChunkRecord, id));
static_assert(offsetof(ChunkRecord, z) == 8 && kRecVal % 16 == 0 && kRecId % 16 == 0 && sizeof(ChunkRecord) % 16 == 0,
              "chunk records are read as 16-byte groups");

// One workgroup per sequence.  Row phase: wave w takes frontier rows
// w, w + 8, ...; for each, lane c reads chunk c's record (its sorted list
// stays in the lane's registers), the wave reduces the row's maximum,
// normaliser and unusable flag, and takes the row's top K as a K-step merge
// of the chunks' lists (each step the best head), valued
// s + (x - max)/t - log Z in fp64, into LDS.  Selection phase (all threads):
// each candidate's rank is the number of candidates before it, and it is
// written straight to that output slot.
__global__ __launch_bounds__(64 * kSelWaves) void te_select(const ExpandKernelArgs a) {
  __shared__ double sv[kMaxTree][kMaxTopK];   // row f's candidates: value
  __shared__ int st[kMaxTree][kMaxTopK];      // and token, sorted
  __shared__ float sx[kMaxTree][kMaxTopK];    // and logit (equal logits of one row tie exactly)
  __shared__ int scnt[kMaxTree], sbad[kMaxTree];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, b = blockIdx.x;
  const int F = a.F, M = a.M, NC = a.NC, K = a.K;

  for (int f = wave; f < F; f += kSelWaves) {
    const int row = b * F + f;
    // the row's score and every chunk record (lane c: chunk c) are requested
    // together: one memory round trip for the row.  The chunk's list stays in
    // registers (16-byte groups of logits and of ids).
    const float s = a.scores[row];
    const ChunkRecord* const rec = a.chunks + static_cast<int64_t>(row) * NC;
    const int nq = (K + 3) / 4;
    u32x4_t w0 = {0u, 0u, 0u, 0u}, wv[kMaxTopK / 4], wi[kMaxTopK / 4];
    if (lane < NC) {
      const u32x4_t* r4 = reinterpret_cast<const u32x4_t*>(rec + lane);
      w0 = r4[0];
#pragma unroll
      for (int j = 0; j < kMaxTopK / 4; ++j)
        if (j < nq) {
          wv[j] = r4[kRecVal / 16 + j];
          wi[j] = r4[kRecId / 16 + j];
        }
    }
    if (!(s > kNegInf)) {   // inactive (NaN and -inf): no candidates, not flagged
      if (lane == 0) {
        scnt[f] = 0;
        sbad[f] = 0;
      }
      continue;
    }
    const float mc = lane < NC ? __uint_as_float(w0[0]) : kNegInf;
    const uint32_t bad = lane < NC ? w0[1] : 0u;
    const double zc = __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(w0[3]) << 32) | w0[2]));
    const float mx = wave_max_f32(mc);
    if (__any(bad != 0) || mx == kNegInf) {   // unusable row: skipped, the sequence is flagged
      if (lane == 0) {
        scnt[f] = 0;
        sbad[f] = 1;
      }
      continue;
    }
    const double z = wave_sum_f64(
        (lane < NC && mc != kNegInf) ? zc * exp2((static_cast<double>(mc) - mx) * static_cast<double>(a.c2)) : 0.0);
    const double lz = log(z);
    int hd = 0, cnt = 0;
    for (int q = 0; q < K; ++q) {
      // this lane's head: entry hd of its chunk's list
      uint32_t hv = 0u, hi = 0xFFFFFFFFu;
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j)
        if (j < K && j == hd) {
          hv = wv[j / 4][j % 4];
          hi = wi[j / 4][j % 4];
        }
      const uint64_t key = (lane < NC && hd < K && static_cast<int>(hi) >= 0)
                               ? cand_key(__uint_as_float(hv), static_cast<int>(hi)) : 0ull;
      const uint64_t best = wave_max_u64(key);
      if (best == 0ull) break;   // every list is exhausted
      if (key == best) ++hd;     // token ids are unique: one lane wins
      const float bv = key_logit(best);
      const int bi = key_token(best);
      if (lane == 0) {
        sx[f][cnt] = bv;
        st[f][cnt] = bi;
        sv[f][cnt] = static_cast<double>(s) + (static_cast<double>(bv) - mx) * a.inv_tau - lz;
      }
      ++cnt;
    }
    if (lane == 0) {
      scnt[f] = cnt;
      sbad[f] = 0;
    }
  }
  __syncthreads();

  // Selection by rank: candidate (f, q) of slot t = f * K + q ranks by the
  // number of candidates before it (larger value, then lower frontier index,
  // then earlier in its row: lower token id among equal values), so every
  // thread writes its own output slot; the rows' lists are read from LDS as
  // broadcasts.  Rank r and r + 1 (up to the kept/dropped boundary) form the
  // decisions tested for near ties.
  __shared__ int byrank[kMaxKeep + 1];
  __shared__ double cv[kMaxTree * kMaxTopK];   // slot f * K + q: candidate value, -inf past a row's list
  int n_valid = 0;
  bool any_bad = false;
  const int tot = F * K;
  for (int t = threadIdx.x; t < tot; t += 64 * kSelWaves) {
    const int f = t / K, q = t - f * K;
    cv[t] = q < scnt[f] ? sv[f][q] : -__builtin_inf();
  }
  for (int t = threadIdx.x; t < F; t += 64 * kSelWaves) any_bad = any_bad || sbad[t] != 0;
  __syncthreads();
  {
    for (int t0 = 0; t0 < tot; t0 += 64 * kSelWaves) {
      const int t = t0 + threadIdx.x;
      const double v = t < tot ? cv[t] : -__builtin_inf();
      const bool valid = v > -__builtin_inf();   // candidate values are finite
      n_valid += __syncthreads_count(valid);
      if (!valid) continue;
      const int f = t / K, q = t - f * K;
      // slots before t in (f, q) order are exactly the indices below t
      int rank = 0;
#pragma unroll 8
      for (int j = 0; j < tot; ++j) {
        const double w = cv[j];
        rank += (w > v || (w == v && j < t)) ? 1 : 0;
      }
      if (rank <= M) byrank[rank] = (f << 8) | q;
      if (rank < M) {
        a.parent[b * M + rank] = f;
        a.token[b * M + rank] = st[f][q];
        a.value[b * M + rank] = static_cast<float>(v);
      }
    }
  }
  any_bad = __syncthreads_or(any_bad);
  // padding past the candidates, and the near ties of adjacent ranks
  const int t = threadIdx.x;
  if (t >= n_valid && t < M) {
    a.parent[b * M + t] = -1;
    a.token[b * M + t] = -1;
    a.value[b * M + t] = kNegInf;
  }
  bool near = false;
  if (t + 1 < n_valid && t + 1 <= M) {
    const int e0 = byrank[t], e1 = byrank[t + 1];
    const int f0 = e0 >> 8, q0 = e0 & 255, f1 = e1 >> 8, q1 = e1 & 255;
    near = sv[f0][q0] - sv[f1][q1] < kNear && !(f0 == f1 && sx[f0][q0] == sx[f1][q1]);
  }
  const int nnear = __syncthreads_count(near);
  if (t == 0) {
    a.flags[b] = any_bad ? EAGLE_FLAG_NONFINITE : 0u;
    a.near_ties[b] = nnear;
  }
}

// Final draft tree from D chained expansion steps: the N nodes of largest
// value (ties: earlier step, then better rank), written in (step, rank)
// order after the root, so parents precede children.  One wave per
// sequence: lane d walks step d's ranked list; each of the N selections takes
// the largest head (ties: the lowest lane = earliest step), then the kept
// nodes get their row numbers step by step with a ballot prefix count.
__global__ __launch_bounds__(64) void te_rerank(const RerankKernelArgs a) {
  __shared__ uint8_t kept[kMaxSteps][kMaxKeep];
  __shared__ int16_t rowof[kMaxSteps][kMaxKeep];
  const int lane = threadIdx.x, b = blockIdx.x;
  const int D = a.D, M = a.M, N = a.N, B = a.B;
  for (int i = lane; i < kMaxSteps * kMaxKeep; i += 64) {
    kept[i / kMaxKeep][i % kMaxKeep] = 0;
    rowof[i / kMaxKeep][i % kMaxKeep] = -1;
  }
  __syncthreads();
  int pos = 0;
  int taken = 0;
  for (int step = 0; step < N; ++step) {
    float hv = kNegInf;
    bool has = false;
    if (lane < D && pos < M) {
      const int64_t at = (static_cast<int64_t>(lane) * B + b) * M + pos;
      has = a.parent[at] >= 0;
      if (has) hv = a.value[at];
    }
    const uint32_t key = has ? ord32(hv) : 0u;
    const uint32_t bkey = static_cast<uint32_t>(wave_max_u64(key));
    const uint64_t hit = __ballot(has && key == bkey);
    if (!hit) break;   // no candidate left
    const int w = __ffsll(static_cast<long long>(hit)) - 1;
    if (lane == w) {
      kept[lane][pos] = 1;
      ++pos;
    }
    ++taken;
  }
  __syncthreads();
  // row numbers in (step, rank) order, then parents and tokens
  int base = 1;
  for (int d = 0; d < D; ++d) {
    const bool k = lane < M && kept[d][lane];
    const uint64_t mask = __ballot(k);
    if (k) rowof[d][lane] = static_cast<int16_t>(base + __popcll(mask & ((1ull << lane) - 1ull)));
    base += __popcll(mask);
    __syncthreads();
  }
  int32_t* const par = a.parents + static_cast<int64_t>(b) * (N + 1);
  int32_t* const tok = a.tokens + static_cast<int64_t>(b) * (N + 1);
  // rows past the last kept node are padding: token -1 under a valid parent
  // (the root), which is how trees of different sizes share a batch
  for (int i = lane; i <= N; i += 64) {
    par[i] = i == 0 ? -1 : 0;
    tok[i] = -1;
  }
  __syncthreads();
  if (lane == 0) tok[0] = a.root_tokens[b];
  for (int d = 0; d < D; ++d) {
    if (lane < M && kept[d][lane]) {
      const int64_t at = (static_cast<int64_t>(d) * B + b) * M + lane;
      const int row = rowof[d][lane];
      const int pi = a.parent[at];   // an index outside the previous list leaves the row without a parent
      par[row] = d == 0 ? 0 : ((pi >= 0 && pi < M) ? rowof[d - 1][pi] : -1);
      tok[row] = a.token[at];
    }
  }
  if (lane == 0) a.rows[b] = 1 + taken;
}

template <typename TL>
hipError_t launch_t(const ExpandKernelArgs& a, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(a.B * a.F * a.NC));
  if (a.chunk == 2048) hipLaunchKernelGGL((te_chunk<TL, 8>), grid, dim3(kThreads), 0, st, a);
  else if (a.chunk == 4096) hipLaunchKernelGGL((te_chunk<TL, 16>), grid, dim3(kThreads), 0, st, a);
  else hipLaunchKernelGGL((te_chunk<TL, 32>), grid, dim3(kThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(te_select, dim3(static_cast<unsigned>(a.B)), dim3(64 * kSelWaves), 0, st, a);
  return hipGetLastError();
}

}  // namespace

int launch_tree_rerank(const RerankKernelArgs& args, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(te_rerank, dim3(static_cast<unsigned>(args.B)), dim3(64), 0, st, args);
  return static_cast<int>(hipGetLastError());
}

int launch_tree_expand(const ExpandKernelArgs& args, int logits_bf16, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const hipError_t e = logits_bf16 ? launch_t<uint16_t>(args, st) : launch_t<float>(args, st);
  return static_cast<int>(e);
}

}  // namespace ev
