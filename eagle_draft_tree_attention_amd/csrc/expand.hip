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
// GPU formulation, three launches:
//   te_chunk   one workgroup per (sequence, frontier row, vocabulary chunk of
//              2048, 4096 or 8192 tokens, at most 64 chunks a row):
//              the chunk's maximum, its sum of exp((x - max)/t) (fp32
//              exponentials, fp64 sum), NaN/+inf detection and its k largest
//              logits with their ids (k rounds of a wave argmax per wave, then
//              a merge of the four waves' lists); one record per chunk.
//   te_row     one wave per (sequence, frontier row), lane c = chunk c: the
//              row's maximum and normaliser, its top k as a k-step merge of
//              the chunks' sorted lists, the candidates' values
//              s_f + (x - max)/t - log Z in fp64.
//   te_select  one wave per sequence, lane f = frontier row f: the global
//              ranking as a merge of the rows' sorted lists: each step the wave picks the
//              largest head (ties: the lowest lane), M + 1 steps, the last one
//              only to see whether the boundary is a near tie.
//   te_rerank  (separate call) the final tree from the chained steps.
// Within a row the value is a monotone function of the logit, so a row's
// list sorted by logit is sorted by value too.
#include <hip/hip_runtime.h>
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

// (value, id) order of the chunk lists: larger value first, then lower id
__device__ __forceinline__ bool before(float a, int ia, float b, int ib) {
  return a > b || (a == b && ia < ib);
}

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
  for (int off = 32; off > 0; off >>= 1) {
    m = fmaxf(m, __shfl_xor(m, off));
    bad |= __shfl_xor(bad, off);
  }
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
  for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off);
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
    const int lid = lj >= 0 ? v0 + tid + kThreads * lj : 0x7FFFFFFF;
    float bv = lb;
    int bi = lid;
    for (int off = 32; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (before(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (lj >= 0 && lid == bi) taken |= 1u << lj;
    if (lane == 0) {
      wl_v[wave][q] = bv;
      wl_i[wave][q] = bv > kNegInf ? bi : -1;
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
      float hv = kNegInf;
      int hi = 0x7FFFFFFF;
      if (lane < kThreads / 64 && hd < K && wl_i[lane][hd] >= 0) {
        hv = wl_v[lane][hd];
        hi = wl_i[lane][hd];
      }
      float bv = hv;
      int bi = hi;
      for (int off = 2; off > 0; off >>= 1) {   // lanes 0..3
        const float ov = __shfl_xor(bv, off);
        const int oi = __shfl_xor(bi, off);
        if (before(ov, oi, bv, bi)) {
          bv = ov;
          bi = oi;
        }
      }
      if (lane < kThreads / 64 && hv == bv && hi == bi && bv > kNegInf) ++hd;
      if (lane == 0) {
        rec->val[q] = bv;
        rec->id[q] = bv > kNegInf ? bi : -1;
      }
    }
  }
}

// One wave per (sequence, frontier row), lane c = chunk c: the row's maximum,
// normaliser and unusable flag from its chunk records, then its top K as a
// K-step merge of the chunks' sorted lists (each step the wave takes the best
// head), valued s + (x - max)/t - log Z in fp64.
__global__ __launch_bounds__(64) void te_row(const ExpandKernelArgs a) {
  __shared__ float lv[kMaxChunksExpand][kMaxTopK];
  __shared__ int li[kMaxChunksExpand][kMaxTopK];
  const int lane = threadIdx.x, row = blockIdx.x;   // row = b * F + f
  const int NC = a.NC, K = a.K;
  RowRecord* const out = a.rows + row;
  const float s = a.scores[row];
  if (!(s > kNegInf)) {   // inactive (NaN and -inf): no candidates, not flagged
    if (lane == 0) {
      out->count = 0;
      out->unusable = 0;
    }
    return;
  }
  const ChunkRecord* const rec = a.chunks + static_cast<int64_t>(row) * NC;
  float mc = kNegInf;
  uint32_t bad = 0;
  double zc = 0.0;
  if (lane < NC) {
    mc = rec[lane].m;
    bad = rec[lane].bad;
    zc = rec[lane].z;
    for (int q = 0; q < K; ++q) {
      lv[lane][q] = rec[lane].val[q];
      li[lane][q] = rec[lane].id[q];
    }
  }
  float mx = mc;
  for (int off = 32; off > 0; off >>= 1) {
    mx = fmaxf(mx, __shfl_xor(mx, off));
    bad |= __shfl_xor(bad, off);
  }
  const bool unusable = bad != 0 || mx == kNegInf;
  if (unusable) {
    if (lane == 0) {
      out->count = 0;
      out->unusable = 1;
    }
    return;
  }
  double z = (lane < NC && mc != kNegInf) ? zc * exp2((static_cast<double>(mc) - mx) * static_cast<double>(a.c2)) : 0.0;
  for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off);
  const double lz = log(z);
  __syncthreads();   // the lists are in LDS
  int hd = 0, cnt = 0;
  for (int q = 0; q < K; ++q) {
    float hv = kNegInf;
    int hi = 0x7FFFFFFF;
    if (lane < NC && hd < K && li[lane][hd] >= 0) {
      hv = lv[lane][hd];
      hi = li[lane][hd];
    }
    float bv = hv;
    int bi = hi;
    for (int off = 32; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (before(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (!(bv > kNegInf)) break;   // every list is exhausted
    if (hi == bi && hv == bv) ++hd;   // token ids are unique: one lane wins
    if (lane == 0) {
      out->logit[cnt] = bv;
      out->token[cnt] = bi;
      out->value[cnt] = static_cast<double>(s) + (static_cast<double>(bv) - mx) * a.inv_tau - lz;
    }
    ++cnt;
  }
  if (lane == 0) {
    out->count = cnt;
    out->unusable = 0;
  }
}

__global__ __launch_bounds__(64) void te_select(const ExpandKernelArgs a) {
  __shared__ double sv[64][kMaxTopK];   // lane f's candidates: value
  __shared__ int st[64][kMaxTopK];      // and token, sorted
  __shared__ float sx[64][kMaxTopK];    // and logit (equal logits of one row tie exactly)
  const int lane = threadIdx.x, b = blockIdx.x;
  const int F = a.F, M = a.M;
  int cnt = 0;            // candidates of row `lane`
  bool unusable = false;
  if (lane < F) {   // every entry up to K is requested at once; the count says which are valid
    const RowRecord* const r = a.rows + b * F + lane;
    for (int q = 0; q < a.K; ++q) {
      sv[lane][q] = r->value[q];
      st[lane][q] = r->token[q];
      sx[lane][q] = r->logit[q];
    }
    cnt = r->count;
    unusable = r->unusable != 0;
  }
  // global ranking: merge of the rows' lists, the largest head each step,
  // ties to the lowest lane (frontier index)
  int pos = 0;
  double prev_v = 0.0;
  int prev_f = -1;
  float prev_x = 0.f;
  int near = 0;
  for (int step = 0; step <= M; ++step) {
    const double hv = (lane < F && pos < cnt) ? sv[lane][pos] : -__builtin_inf();
    double best = hv;
    for (int off = 32; off > 0; off >>= 1) best = fmax(best, __shfl_xor(best, off));
    if (!(best > -__builtin_inf())) {   // no candidate left: pad
      if (lane == 0 && step < M) {
        a.parent[b * M + step] = -1;
        a.token[b * M + step] = -1;
        a.value[b * M + step] = kNegInf;
      }
      continue;
    }
    const uint64_t hit = __ballot(hv == best && lane < F && pos < cnt);
    const int w = __ffsll(static_cast<long long>(hit)) - 1;
    const int wt = __shfl(lane < F && pos < cnt ? st[lane][pos] : 0, w);
    const float wx = __shfl(lane < F && pos < cnt ? sx[lane][pos] : 0.f, w);
    if (step > 0 && prev_v - best < kNear && !(prev_f == w && prev_x == wx)) ++near;
    prev_v = best;
    prev_f = w;
    prev_x = wx;
    if (lane == 0 && step < M) {
      a.parent[b * M + step] = w;
      a.token[b * M + step] = wt;
      a.value[b * M + step] = static_cast<float>(best);
    }
    if (lane == w) ++pos;
  }
  const bool any_bad = __any(unusable);
  if (lane == 0) {
    a.flags[b] = any_bad ? EAGLE_FLAG_NONFINITE : 0u;
    a.near_ties[b] = near;
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
    float best = has ? hv : kNegInf;
    for (int off = 32; off > 0; off >>= 1) best = fmaxf(best, __shfl_xor(best, off));
    const uint64_t hit = __ballot(has && hv == best);
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
  for (int i = lane; i <= N; i += 64) {
    par[i] = -1;
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
  hipLaunchKernelGGL(te_row, dim3(static_cast<unsigned>(a.B * a.F)), dim3(64), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(te_select, dim3(static_cast<unsigned>(a.B)), dim3(64), 0, st, a);
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
