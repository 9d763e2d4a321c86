// Keep-thresholds of top-k / top-p filtered distributions, gfx950 (MI355X).
//
// Sampling a token from a distribution truncated to its k most probable
// tokens (top-k) or to the smallest most-probable set holding a fraction p of
// the mass (top-p, nucleus) keeps every token whose logit is at least some
// value theta of its row.  The EAGLE notes page's tree drafting samples k
// children per node; a request that verifies with such filters uses the
// filtered target q' and the filtered draft p' (from which the children were
// drawn), and the acceptance rule is then lossless for q'.  Definitions
// (per row x, q = softmax(x / t)):
//   top-k: theta_k = the k-th largest logit, duplicates counted (ties at
//          theta_k are all kept); k = 0 or k >= V keeps everything.
//   top-p: among the tokens kept by top-k, keep v iff the mass of the tokens
//          with a strictly larger logit is below p times the kept mass, i.e.
//          theta_p = the largest logit value u with mass(x >= u) >= p Z.
//          p = 0 or p = 1 keeps everything.
// theta = theta_p (or theta_k without top-p).  A top-p boundary whose
// cumulative mass lies within 1e-6 Z of p Z on either side is reported as a
// near tie of that row.
//
// One workgroup of 1024 threads per row (target rows of every real node,
// draft rows of nodes with children).  Masses are summed exactly in 2^-40
// fixed point (64-bit integers), so every decision is independent of the
// order of the additions.  The threshold is found by histograms over the
// distance from the row maximum: 256 bins over [0, max - min], the bin where
// the cumulative count (or mass) crosses the target is refined by another
// 256 bins, up to four levels, until it holds a single value or at most 4096
// elements, which are then sorted (bitonic, in LDS) and scanned exactly.  A
// row that still does not resolve takes an exact bisection over the value
// keys.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ev_internal.h"

namespace ev {
namespace {

constexpr int kFT = 1024;          // threads per row
constexpr int kFWaves = kFT / 64;
constexpr int kCap = 4096;         // candidates sorted in LDS
constexpr int kLevels = 4;
constexpr float kNegInf = -__builtin_inff();
constexpr double kFix = 1099511627776.0;   // 2^40: fixed-point unit of a weight <= 1

template <typename TL>
__device__ __forceinline__ float ld(const TL* r, int v) {
  if constexpr (sizeof(TL) == 2) return __uint_as_float(static_cast<uint32_t>(r[v]) << 16);
  else return r[v];
}

// order-preserving 32-bit key of a float (larger value, larger key)
__device__ __forceinline__ uint32_t fkey(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unkey(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

struct FilterShared {
  uint64_t hist[256];          // weight per bin
  uint32_t hcnt[256];          // elements per bin
  float cx[kCap];              // candidates: logits ...
  uint64_t cw[kCap];           // ... and their weights, sorted by logit, descending
  uint64_t u64s[kFWaves];
  float f32s[kFWaves];
  uint32_t u32s[kFWaves];
  uint32_t ncand;
  int32_t bsel;                // boundary bin of this level
  uint64_t above_add;          // weight of the bins before it
  int32_t done;
};

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t lo = __shfl_xor(static_cast<uint32_t>(x), o);
    const uint32_t hi = __shfl_xor(static_cast<uint32_t>(x >> 32), o);
    x += (static_cast<uint64_t>(hi) << 32) | lo;
  }
  return x;
}
__device__ uint64_t block_sum_u64(uint64_t x, FilterShared& sh) {
  x = wave_sum_u64(x);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sh.u64s[w] = x;
  __syncthreads();
  uint64_t t = 0;
  for (int i = 0; i < kFWaves; ++i) t += sh.u64s[i];
  __syncthreads();
  return t;
}
template <bool MAX>
__device__ float block_ext_f32(float x, FilterShared& sh) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float y = __shfl_xor(x, o);
    x = MAX ? fmaxf(x, y) : fminf(x, y);
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sh.f32s[w] = x;
  __syncthreads();
  float t = sh.f32s[0];
  for (int i = 1; i < kFWaves; ++i) t = MAX ? fmaxf(t, sh.f32s[i]) : fminf(t, sh.f32s[i]);
  __syncthreads();
  return t;
}
template <bool MAX>
__device__ int block_ext_i32(int x, FilterShared& sh) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const int y = __shfl_xor(x, o);
    x = MAX ? max(x, y) : min(x, y);
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sh.u32s[w] = static_cast<uint32_t>(x);
  __syncthreads();
  int t = static_cast<int>(sh.u32s[0]);
  for (int i = 1; i < kFWaves; ++i) t = MAX ? max(t, static_cast<int>(sh.u32s[i])) : min(t, static_cast<int>(sh.u32s[i]));
  __syncthreads();
  return t;
}
// exclusive prefix sum over the block, in thread order
__device__ uint64_t block_excl_scan_u64(uint64_t x, FilterShared& sh) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint64_t inc = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t lo = __shfl_up(static_cast<uint32_t>(inc), o);
    const uint32_t hi = __shfl_up(static_cast<uint32_t>(inc >> 32), o);
    if (lane >= o) inc += (static_cast<uint64_t>(hi) << 32) | lo;
  }
  if (lane == 63) sh.u64s[w] = inc;
  __syncthreads();
  uint64_t off = 0;
  for (int i = 0; i < w; ++i) off += sh.u64s[i];
  __syncthreads();
  return off + inc - x;
}
__device__ uint32_t block_or_u32(uint32_t x, FilterShared& sh) {
  x = __any(x != 0) ? 1u : 0u;
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sh.u32s[w] = x;
  __syncthreads();
  uint32_t t = 0;
  for (int i = 0; i < kFWaves; ++i) t |= sh.u32s[i];
  __syncthreads();
  return t;
}

// weight of one logit: 1 (count mode) or exp((x - m) / t) in 2^-40 units
__device__ __forceinline__ uint64_t weight(bool mass, float x, float m, float c2) {
  if (!mass) return 1ull;
  return static_cast<uint64_t>(static_cast<double>(__builtin_amdgcn_exp2f((x - m) * c2)) * kFix);
}

// The chain of bins of one element: its bin at every level up to `lev` must
// be the boundary bin chosen there for the element to lie in the current
// range.  Returns the element's bin at level `lev`, or -1 when it left the
// range at an earlier level (or lies below the floor).
struct Levels {
  float base[kLevels];
  float inv[kLevels];
  int sel[kLevels];
};
__device__ __forceinline__ int bin_at(const Levels& L, int lev, float dist) {
  int b = -1;
  for (int l = 0; l <= lev; ++l) {
    const float t = (dist - L.base[l]) * L.inv[l];
    b = static_cast<int>(fminf(fmaxf(t, 0.f), 255.f));
    if (l < lev && b != L.sel[l]) return -1;
  }
  return b;
}

// Largest logit value u of the row with W(x >= u) >= target, counting only
// x >= floor (W = count or fixed-point mass); -inf when the total is below
// target.  Also the weights W(x > u) and W(x >= u).
template <typename TL>
__device__ float find_threshold(const TL* row, int V, bool mass, float m, float mn, float c2, float floor,
                                uint64_t target, uint64_t& w_gt, uint64_t& w_ge, FilterShared& sh) {
  const int tid = threadIdx.x;
  Levels L;
  L.base[0] = 0.f;
  L.inv[0] = (m > mn) ? 254.99f / (m - mn) : 0.f;
  // a range too wide for float bins (max - min overflows) goes straight to
  // the bisection
  const int levels = (m - mn <= 3.0e38f) ? kLevels : 0;
  uint64_t above = 0;
  for (int lev = 0; lev < levels; ++lev) {
    for (int i = tid; i < 256; i += kFT) {
      sh.hist[i] = 0;
      sh.hcnt[i] = 0;
    }
    __syncthreads();
    for (int v = tid; v < V; v += kFT) {
      const float x = ld<TL>(row, v);
      if (!(x >= floor) || x == kNegInf) continue;
      const int b = bin_at(L, lev, m - x);
      if (b < 0) continue;
      atomicAdd(reinterpret_cast<unsigned long long*>(&sh.hist[b]),
                static_cast<unsigned long long>(weight(mass, x, m, c2)));
      atomicAdd(&sh.hcnt[b], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      uint64_t cum = above;
      int bd = -1;
      for (int b = 0; b < 256; ++b) {
        if (cum + sh.hist[b] >= target) {
          bd = b;
          break;
        }
        cum += sh.hist[b];
      }
      sh.bsel = bd;
      sh.above_add = cum - above;
      sh.ncand = 0;
    }
    __syncthreads();
    const int bd = sh.bsel;
    if (bd < 0) {   // the whole range holds less than target: keep everything
      w_gt = w_ge = 0;
      return kNegInf;
    }
    above += sh.above_add;
    const uint32_t nb = sh.hcnt[bd];
    // candidates of the boundary bin: their value range, and up to kCap of them
    float lo = __builtin_inff(), hi = kNegInf;
    L.sel[lev] = bd;
    for (int v = tid; v < V; v += kFT) {
      const float x = ld<TL>(row, v);
      if (!(x >= floor) || x == kNegInf) continue;
      if (bin_at(L, lev, m - x) != bd) continue;
      lo = fminf(lo, x);
      hi = fmaxf(hi, x);
      if (nb <= kCap) {
        const uint32_t j = atomicAdd(&sh.ncand, 1u);
        sh.cx[j] = x;
        sh.cw[j] = weight(mass, x, m, c2);
      }
    }
    lo = block_ext_f32<false>(lo, sh);
    hi = block_ext_f32<true>(hi, sh);
    if (lo == hi) {   // one value: it is the threshold
      w_gt = above;
      w_ge = above + sh.hist[bd];
      return lo;
    }
    if (nb <= kCap) {
      // sort the candidates by logit, descending (padding: -inf, weight 0)
      int n = 1;
      while (n < static_cast<int>(nb)) n <<= 1;
      for (int i = static_cast<int>(nb) + tid; i < n; i += kFT) {
        sh.cx[i] = kNegInf;
        sh.cw[i] = 0;
      }
      __syncthreads();
      for (int k = 2; k <= n; k <<= 1)
        for (int j = k >> 1; j > 0; j >>= 1) {
          for (int i = tid; i < n; i += kFT) {
            const int p = i ^ j;
            if (p > i) {
              const bool desc = (i & k) == 0;
              const float a = sh.cx[i], b = sh.cx[p];
              if (desc ? (a < b) : (a > b)) {
                sh.cx[i] = b;
                sh.cx[p] = a;
                const uint64_t t = sh.cw[i];
                sh.cw[i] = sh.cw[p];
                sh.cw[p] = t;
              }
            }
          }
          __syncthreads();
        }
      // running weights (above + inclusive prefix) in place: thread t owns
      // positions 4t .. 4t + 3
      uint64_t loc[4], run = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * tid + e;
        run += (i < static_cast<int>(nb)) ? sh.cw[i] : 0ull;
        loc[e] = run;
      }
      const uint64_t before = above + block_excl_scan_u64(run, sh);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * tid + e;
        if (i < static_cast<int>(nb)) sh.cw[i] = before + loc[e];
      }
      __syncthreads();
      // the first position whose running weight reaches the target (the
      // bin's total does), then the extent of its value's run
      int first = 0x7FFFFFFF;
#pragma unroll
      for (int e = 3; e >= 0; --e) {
        const int i = 4 * tid + e;
        if (i < static_cast<int>(nb) && sh.cw[i] >= target) first = i;
      }
      const int i0 = min(block_ext_i32<false>(first, sh), static_cast<int>(nb) - 1);   // the bin reaches the target
      const float u = sh.cx[i0];
      int j0 = 0x7FFFFFFF, j1 = -1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * tid + e;
        if (i < static_cast<int>(nb) && sh.cx[i] == u) {
          j0 = min(j0, i);
          j1 = max(j1, i);
        }
      }
      j0 = block_ext_i32<false>(j0, sh);
      j1 = block_ext_i32<true>(j1, sh);
      w_gt = j0 > 0 ? sh.cw[j0 - 1] : above;
      w_ge = sh.cw[j1];
      __syncthreads();
      return u;
    }
    // refine the boundary bin by 256 finer bins
    if (lev + 1 < kLevels) {
      const float w = 1.f / L.inv[lev];
      L.base[lev + 1] = L.base[lev] + static_cast<float>(bd) * w;
      L.inv[lev + 1] = 256.f / w;
    }
  }
  // exact bisection over the value keys of the row: the largest key u with
  // W(x >= unkey(u)) >= target (W counts x >= floor)
  uint32_t klo = fkey(floor == kNegInf ? mn : floor), khi = fkey(m);
  auto wsum_ge = [&](uint32_t k) -> uint64_t {
    uint64_t s = 0;
    for (int v = tid; v < V; v += kFT) {
      const float x = ld<TL>(row, v);
      if (!(x >= floor) || x == kNegInf) continue;
      if (fkey(x) >= k) s += weight(mass, x, m, c2);
    }
    return block_sum_u64(s, sh);
  };
  while (klo < khi) {   // invariant: W(>= klo) >= target
    const uint32_t mid = klo + static_cast<uint32_t>((static_cast<uint64_t>(khi) - klo + 1) / 2);
    if (wsum_ge(mid) >= target) klo = mid;
    else khi = mid - 1;
  }
  // klo is the key of an element (W changes only at element keys)
  w_ge = wsum_ge(klo);
  w_gt = klo == 0xFFFFFFFFu ? 0 : wsum_ge(klo + 1);
  return unkey(klo);
}

template <typename TL>
__global__ __launch_bounds__(kFT) void sa_filter(const FilterKernelArgs a) {
  __shared__ FilterShared sh;
  const int tid = threadIdx.x;
  const int r = blockIdx.x & 1;                  // 0 target row, 1 draft row
  const int n = (blockIdx.x >> 1) % a.T;
  const int b = (blockIdx.x >> 1) / a.T;
  const int T = a.T, V = a.V;
  float* const out = a.thr + (static_cast<int64_t>(b) * T + n) * 2 + r;
  int32_t* const near = a.near + (static_cast<int64_t>(b) * T + n) * 2 + r;
  // is the row read?  target rows of real nodes, draft rows of real nodes
  // with children (rows past the first padding row are padding)
  if (tid < 64) {
    const int lane = tid;
    const int li = b * T + (lane < T ? lane : T - 1);
    const int par = a.parents[li];
    const int tok = a.tokens[li];
    const bool pad = lane >= 1 && lane < T && tok == -1;
    const uint64_t padm = __ballot(pad);
    const int nreal = padm ? __ffsll(static_cast<long long>(padm)) - 1 : T;
    const bool child = lane >= 1 && lane < nreal && par == n;
    const bool used = n < nreal && (r == 0 || __any(child));
    if (lane == 0) sh.done = used ? 0 : 1;
  }
  __syncthreads();
  if (sh.done) {
    if (tid == 0) {
      *out = kNegInf;
      *near = 0;
    }
    return;
  }
  const TL* row = reinterpret_cast<const TL*>(r == 0 ? a.target : a.draft) + (static_cast<int64_t>(b) * T + n) * V;
  // row maximum, minimum finite value, and usability (NaN / +inf / all -inf:
  // the acceptance reports the row; nothing is filtered)
  float m = kNegInf, mn = __builtin_inff();
  uint32_t bad = 0;
  for (int v = tid; v < V; v += kFT) {
    const float x = ld<TL>(row, v);
    if (x != x || x == __builtin_inff()) bad = 1;
    else if (x != kNegInf) {
      m = fmaxf(m, x);
      mn = fminf(mn, x);
    }
  }
  bad = block_or_u32(bad, sh);
  m = block_ext_f32<true>(m, sh);
  mn = block_ext_f32<false>(mn, sh);
  float theta = kNegInf;
  int32_t nt = 0;
  if (!bad && m != kNegInf) {
    uint64_t gt = 0, ge = 0;
    if (a.top_k > 0 && a.top_k < V)
      theta = find_threshold<TL>(row, V, false, m, mn, a.c2, kNegInf, static_cast<uint64_t>(a.top_k), gt, ge, sh);
    if (a.top_p > 0.f && a.top_p < 1.f) {
      uint64_t z = 0;
      for (int v = tid; v < V; v += kFT) {
        const float x = ld<TL>(row, v);
        if (x >= theta && x != kNegInf) z += weight(true, x, m, a.c2);
      }
      z = block_sum_u64(z, sh);
      const double zd = static_cast<double>(z);
      const double pz = static_cast<double>(a.top_p) * zd;
      uint64_t target = static_cast<uint64_t>(ceil(pz));
      if (target < 1) target = 1;
      theta = find_threshold<TL>(row, V, true, m, mn, a.c2, theta, target, gt, ge, sh);
      nt = (static_cast<double>(ge) - pz < 1e-6 * zd || pz - static_cast<double>(gt) < 1e-6 * zd) ? 1 : 0;
    }
  }
  if (tid == 0) {
    *out = theta;
    *near = nt;
  }
}

}  // namespace

int launch_filter(const FilterKernelArgs& a, int logits_bf16, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>(a.B * a.T * 2));
  if (logits_bf16) hipLaunchKernelGGL(sa_filter<uint16_t>, grid, dim3(kFT), 0, st, a);
  else hipLaunchKernelGGL(sa_filter<float>, grid, dim3(kFT), 0, st, a);
  return static_cast<int>(hipGetLastError());
}

}  // namespace ev
