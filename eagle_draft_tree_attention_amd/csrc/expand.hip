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

#include "ev_device.h"
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

// timeline mark k of workgroup slot `slot` (thread 0 only; diagnostic)
__device__ __forceinline__ void mark(uint64_t* stamps, int64_t slot, int k) {
  if (stamps && threadIdx.x == 0) stamps[slot * 32 + k] = __builtin_amdgcn_s_memrealtime();
}

// EPT logits of this thread (tokens v .. v + EPT - 1), -inf at or past `end`.
// VEC: the row starts on a 16-byte boundary and holds whole 16-byte groups.
template <typename TL, int EPT, bool VEC>
__device__ __forceinline__ void load_run(const TL* row, int v, int end, float (&xs)[EPT]) {
  if constexpr (VEC) {
    constexpr int G = 16 / static_cast<int>(sizeof(TL));   // tokens per 16-byte group
    u32x4_t w[EPT / G];
#pragma unroll
    for (int g = 0; g < EPT / G; ++g)
      w[g] = (v + g * G < end) ? *reinterpret_cast<const u32x4_t*>(row + v + g * G) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int g = 0; g < EPT / G; ++g) {
      const bool in = v + g * G < end;
#pragma unroll
      for (int e = 0; e < G; ++e) {
        float x;
        if constexpr (sizeof(TL) == 2)
          x = __uint_as_float((e & 1) ? (w[g][e >> 1] & 0xFFFF0000u) : (w[g][e >> 1] << 16));
        else
          x = __uint_as_float(w[g][e]);
        xs[g * G + e] = in ? x : kNegInf;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < EPT; ++j) xs[j] = (v + j < end) ? logit_at<TL>(row, v + j) : kNegInf;
  }
}

__device__ __forceinline__ uint32_t umax32(uint32_t p, uint32_t q) { return p > q ? p : q; }

// Chunks of 256 * EPT tokens (2048, 4096 or 8192, the smallest that keeps a
// row within 64 chunks).  Thread t owns the EPT consecutive tokens v0 + EPT t
// .. + EPT - 1, so lane order and wave order follow token order: among equal
// logits the lowest lane holds the lowest token id, and a ballot's first
// lane breaks ties.
template <typename TL, int EPT, bool VEC>
__global__ __launch_bounds__(kThreads) void te_chunk(const ExpandKernelArgs a) {
  constexpr int kWaves = kThreads / 64;
  __shared__ float wmax[kWaves];
  __shared__ uint32_t wbad[kWaves];
  __shared__ double wsum[kWaves];
  __shared__ float wl_v[kWaves][kMaxTopK];
  __shared__ int wl_t[kWaves][kMaxTopK];
  __shared__ int wl_n[kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int NC = a.NC, V = a.V, K = a.K;
  const int c = blockIdx.x % NC;
  const int row = blockIdx.x / NC;   // b * F + f
  const TL* x = reinterpret_cast<const TL*>(a.logits) + static_cast<int64_t>(row) * V;
  const int v0 = c * a.chunk;
  const int vt = v0 + EPT * tid;   // this thread's first token
  mark(a.stamps, blockIdx.x, 0);

  float xs[EPT];
  load_run<TL, EPT, VEC>(x, vt, min(V, v0 + a.chunk), xs);
  // chunk maximum and NaN/+inf flag (NaN and +inf make the row unusable and
  // are never candidates; -inf neither)
  float m = kNegInf;
  uint32_t bad = 0;
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    if (xs[j] != xs[j] || xs[j] == __builtin_inff()) {
      bad = 1;
      xs[j] = kNegInf;
    }
    m = fmaxf(m, xs[j]);
  }
  m = wave_max_f32(m);
  bad = __any(bad != 0) ? 1u : 0u;
  if (lane == 0) {
    wmax[wave] = m;
    wbad[wave] = bad;
  }
  __syncthreads();
  mark(a.stamps, blockIdx.x, 1);
  m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  bad = wbad[0] | wbad[1] | wbad[2] | wbad[3];
  // sum of exp((x - m) / t): fp32 exponentials of the exact difference, fp64 sum
  double z = 0.0;
  if (m != kNegInf) {
#pragma unroll
    for (int j = 0; j < EPT; ++j) z += static_cast<double>(__builtin_amdgcn_exp2f((xs[j] - m) * a.c2));
  }
  z = wave_sum_f64(z);
  if (lane == 0) wsum[wave] = z;

  // the wave's k largest: each round every lane offers its best untaken
  // logit (lowest token first among equal ones), the wave keeps the largest
  // (lowest lane among equal ones) and only the winning lane moves on
  uint32_t taken = 0;
  float lb = kNegInf;
  int lj = -1;
  auto rescan = [&]() {
    lb = kNegInf;
    lj = -1;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const bool better = !((taken >> j) & 1u) && xs[j] > lb;
      lb = better ? xs[j] : lb;
      lj = better ? j : lj;
    }
  };
  rescan();
  int nq = 0;
  for (; nq < K; ++nq) {
    const uint32_t key = lj >= 0 ? ord32(lb) : 0u;
    const uint32_t kmax = wave_reduce32(key, 0u, umax32);
    if (kmax == 0u) break;   // every logit of the wave is taken or -inf
    const int wl = __ffsll(static_cast<long long>(__ballot(key == kmax))) - 1;
    if (lane == wl) {
      wl_v[wave][nq] = lb;
      wl_t[wave][nq] = vt + lj;
      taken |= 1u << lj;
      rescan();
    }
  }
  if (lane == 0) wl_n[wave] = nq;
  __syncthreads();
  mark(a.stamps, blockIdx.x, 2);

  // the chunk's k largest from the waves' lists: lane i holds entry i of the
  // concatenated lists and counts the entries ahead of it by lane reads
  ChunkRecord* const rec = a.chunks + static_cast<int64_t>(row) * NC + c;
  if (wave == 0) {
    const int wq = min(lane / K, kWaves - 1), rq = lane - (lane / K) * K;
    const bool valid = lane < kWaves * K && rq < wl_n[wq];
    const float cv = valid ? wl_v[wq][rq] : kNegInf;
    const int ct = valid ? wl_t[wq][rq] : 0;
    const uint64_t key = valid ? cand_key(cv, ct) : 0ull;   // larger logit, then lower token: larger key
    const uint32_t klo = static_cast<uint32_t>(key), khi = static_cast<uint32_t>(key >> 32);
    int rank = 0;
    for (int j = 0; j < kWaves * K; ++j) {
      const uint64_t kj = (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(khi), j))) << 32) |
                          static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(klo), j));
      rank += kj > key ? 1 : 0;
    }
    const int total = wl_n[0] + wl_n[1] + wl_n[2] + wl_n[3];
    if (valid && rank < K) {
      rec->val[rank] = cv;
      rec->id[rank] = ct;
    }
    if (lane >= total && lane < K) {   // past the chunk's candidates
      rec->val[lane] = kNegInf;
      rec->id[lane] = -1;
    }
    if (lane == 0) {
      rec->m = m;
      rec->bad = bad;
      rec->z = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
    }
  }
  mark(a.stamps, blockIdx.x, 3);
}

constexpr int kSelWaves = 8;   // frontier rows worked on at once by one workgroup
constexpr int kRecVal = static_cast<int>(offsetof(ChunkRecord, val));
constexpr int kRecId = static_cast<int>(offsetof(ChunkRecord, id));
static_assert(offsetof(ChunkRecord, z) == 8 && kRecVal % 16 == 0 && kRecId % 16 == 0 && sizeof(ChunkRecord) % 16 == 0,
              "chunk records are read as 16-byte groups");

// One workgroup per sequence.  Row phase: wave w takes frontier rows
// w, w + 8, ...; for each, lane c reads chunk c's record (its sorted list
// stays in the lane's registers, KMAX >= k entries), the wave reduces the
// row's maximum, normaliser and unusable flag, and takes the row's top k as
// a k-step merge of the chunks' lists (each step the largest head: a 32-bit
// key maximum, ties to the lowest chunk, which holds the lowest token ids);
// then lane q values entry q as s + (x - max)/t - log Z in fp64.  Selection
// phase: each candidate's rank is the number of candidates before it (every
// wave counts against its share of the others, read from LDS as broadcasts,
// and adds its count with an LDS atomic), and it is written straight to
// that output slot.
template <int KMAX>
__global__ __launch_bounds__(64 * kSelWaves) void te_select(const ExpandKernelArgs a) {
  constexpr int kSel = 64 * kSelWaves;
  __shared__ double sv[kMaxTree * kMaxTopK];   // slot f * K + q: candidate value, -inf past a row's list
  __shared__ int st[kMaxTree * kMaxTopK];      // its token
  __shared__ float sx[kMaxTree * kMaxTopK];    // and logit (equal logits of one row tie exactly)
  __shared__ uint64_t skey[kMaxTree * kMaxTopK];   // order-preserving key of the value (0: no candidate)
  __shared__ int srank[kMaxTree * kMaxTopK];
  __shared__ int byrank[kMaxKeep + 1];
  // block-wide counts and flags through LDS words and plain barriers (the
  // runtime's barrier reductions first load the workgroup size from the
  // dispatch packet, a scalar-cache miss on the critical path)
  __shared__ int nvalid_lds, anybad_lds, nnear_lds;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, b = blockIdx.x;
  const int F = a.F, M = a.M, NC = a.NC, K = a.K;
  const int64_t mslot = static_cast<int64_t>(a.B) * F * NC + b;   // timeline slot
  mark(a.stamps, mslot, 0);
  if (threadIdx.x == 0) {   // published by the barrier after the row phase
    nvalid_lds = 0;
    anybad_lds = 0;
    nnear_lds = 0;
  }

  for (int f = wave; f < F; f += kSelWaves) {
    const int row = b * F + f;
    // the row's score and every chunk record (lane c: chunk c) are requested
    // together: one memory round trip for the row.  The chunk's list stays in
    // registers (16-byte groups of logits and of ids).
    const float s = a.scores[row];
    const ChunkRecord* const rec = a.chunks + static_cast<int64_t>(row) * NC;
    u32x4_t w0 = {0u, 0u, 0u, 0u}, wv[KMAX / 4], wi[KMAX / 4];
#pragma unroll
    for (int j = 0; j < KMAX / 4; ++j) wv[j] = wi[j] = u32x4_t{0u, 0u, 0u, 0u};
    if (lane < NC) {
      const u32x4_t* r4 = reinterpret_cast<const u32x4_t*>(rec + lane);
      w0 = r4[0];
#pragma unroll
      for (int j = 0; j < KMAX / 4; ++j) {
        wv[j] = r4[kRecVal / 16 + j];
        wi[j] = r4[kRecId / 16 + j];
      }
    }
    int cnt = 0;
    int rbad = 0;
    if (s > kNegInf) {   // inactive rows (NaN, -inf) have no candidates and are not flagged
      const float mc = lane < NC ? __uint_as_float(w0[0]) : kNegInf;
      const uint32_t cb = lane < NC ? w0[1] : 0u;
      const double zc = __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(w0[3]) << 32) | w0[2]));
      const float mx = wave_max_f32(mc);
      if (f == 0) mark(a.stamps, mslot, 1);
      if (__any(cb != 0) || mx == kNegInf) {   // unusable row: skipped, the sequence is flagged
        rbad = 1;
      } else {
        const double z = wave_sum_f64(
            (lane < NC && mc != kNegInf) ? zc * exp2((static_cast<double>(mc) - mx) * static_cast<double>(a.c2)) : 0.0);
        const double lz = log(z);
        if (f == 0) mark(a.stamps, mslot, 2);
        int hd = 0;
        for (; cnt < K; ++cnt) {
          // this lane's head: entry hd of its chunk's list (entries past K
          // are never reached: hd < K is tested below)
          uint32_t hv = 0u, hi = 0xFFFFFFFFu;
#pragma unroll
          for (int j = 0; j < KMAX; ++j)
            if (j == hd) {
              hv = wv[j / 4][j % 4];
              hi = wi[j / 4][j % 4];
            }
          const uint32_t key = (lane < NC && hd < K && static_cast<int>(hi) >= 0) ? ord32(__uint_as_float(hv)) : 0u;
          const uint32_t kmax = wave_reduce32(key, 0u, umax32);
          if (kmax == 0u) break;   // every list is exhausted
          const int wl = __ffsll(static_cast<long long>(__ballot(key == kmax))) - 1;
          const int bi = __builtin_amdgcn_readlane(static_cast<int>(hi), wl);
          if (lane == wl) ++hd;
          if (lane == 0) {
            st[f * K + cnt] = bi;
            sx[f * K + cnt] = unord32(kmax);
          }
        }
        if (lane < cnt) {
          const double v = static_cast<double>(s) + (static_cast<double>(sx[f * K + lane]) - mx) * a.inv_tau - lz;
          sv[f * K + lane] = v;
          skey[f * K + lane] = ord64(v);   // candidate values are finite: keys above 0
        }
      }
    }
    if (lane >= cnt && lane < K) {   // past the row's candidates
      sv[f * K + lane] = -__builtin_inf();
      skey[f * K + lane] = 0ull;
    }
    if (lane < K) srank[f * K + lane] = 0;
    if (lane == 0) {
      if (rbad) anybad_lds = 1;
      if (cnt) atomicAdd(&nvalid_lds, cnt);
    }
    if (f == 0) mark(a.stamps, mslot, 3);
  }
  __syncthreads();
  mark(a.stamps, mslot, 4);

  // Selection by rank: candidate slot t = f * K + q ranks by the number of
  // candidates before it (larger value, then lower frontier index, then
  // earlier in its row: lower token id among equal values).  Rank r and
  // r + 1 (up to the kept/dropped boundary) form the decisions tested for
  // near ties.
  const int tot = F * K;
  const int t = threadIdx.x;
  {
    // wave w counts, for every candidate (lane = candidate within a block of
    // 64), the candidates j of its share that come first
    const int share = (tot + kSelWaves - 1) / kSelWaves;
    const int j0 = wave * share, j1 = min(tot, j0 + share);
    for (int c0 = 0; c0 < tot; c0 += 64) {
      const int cidx = c0 + lane;
      const uint64_t kc = cidx < tot ? skey[cidx] : 0ull;
      int part = 0;
#pragma unroll 4
      for (int j = j0; j < j1; ++j) {
        const uint64_t kj = skey[j];
        part += (kj > kc || (kj == kc && j < cidx)) ? 1 : 0;
      }
      if (cidx < tot && kc != 0ull && part > 0) atomicAdd(&srank[cidx], part);
    }
  }
  __syncthreads();
  mark(a.stamps, mslot, 5);
  for (int i = t; i < tot; i += kSel) {
    if (skey[i] == 0ull) continue;
    const int rank = srank[i];
    if (rank <= M) byrank[rank] = i;
    if (rank < M) {
      a.parent[b * M + rank] = i / K;
      a.token[b * M + rank] = st[i];
      a.value[b * M + rank] = static_cast<float>(sv[i]);
    }
  }
  __syncthreads();
  const int nvalid = nvalid_lds;
  // padding past the candidates, and the near ties of adjacent ranks
  if (t >= nvalid && t < M) {
    a.parent[b * M + t] = -1;
    a.token[b * M + t] = -1;
    a.value[b * M + t] = kNegInf;
  }
  bool near = false;
  if (t + 1 < nvalid && t + 1 <= M) {
    const int e0 = byrank[t], e1 = byrank[t + 1];
    near = sv[e0] - sv[e1] < kNear && !(e0 / K == e1 / K && sx[e0] == sx[e1]);
  }
  if (near) atomicAdd(&nnear_lds, 1);
  __syncthreads();
  if (t == 0) {
    a.flags[b] = anybad_lds ? EAGLE_FLAG_NONFINITE : 0u;
    a.near_ties[b] = nnear_lds;
  }
  mark(a.stamps, mslot, 6);
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

template <typename TL, bool VEC>
void launch_chunks(const ExpandKernelArgs& a, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(a.B * a.F * a.NC));
  if (a.chunk == 2048) hipLaunchKernelGGL((te_chunk<TL, 8, VEC>), grid, dim3(kThreads), 0, st, a);
  else if (a.chunk == 4096) hipLaunchKernelGGL((te_chunk<TL, 16, VEC>), grid, dim3(kThreads), 0, st, a);
  else hipLaunchKernelGGL((te_chunk<TL, 32, VEC>), grid, dim3(kThreads), 0, st, a);
}

template <typename TL>
hipError_t launch_t(const ExpandKernelArgs& a, hipStream_t st) {
  // whole 16-byte groups per row, from a 16-byte aligned base: vector loads
  const bool vec = (reinterpret_cast<uintptr_t>(a.logits) % 16 == 0) &&
                   (static_cast<int64_t>(a.V) * static_cast<int64_t>(sizeof(TL))) % 16 == 0;
  if (vec) launch_chunks<TL, true>(a, st);
  else launch_chunks<TL, false>(a, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 sg(static_cast<unsigned>(a.B)), sb(64 * kSelWaves);
  if (a.K <= 4) hipLaunchKernelGGL(te_select<4>, sg, sb, 0, st, a);
  else if (a.K <= 8) hipLaunchKernelGGL(te_select<8>, sg, sb, 0, st, a);
  else hipLaunchKernelGGL(te_select<16>, sg, sb, 0, st, a);
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
