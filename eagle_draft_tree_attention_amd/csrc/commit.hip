// Committing the accepted path into the KV cache, gfx950 (MI355X).
//
// Rule (lesson page, the "KV cache rollback" section and build step 4, KV
// accounting): the verification forward wrote K/V rows for every tree node
// behind the sequence's prefix (node i at row L_b + i).  Once the walk is
// known, the root and the accepted nodes become the next positions of the
// cache and the logical length moves past them; the rows of rejected nodes
// are left where they are (rolled back by the length alone).  The accepted
// nodes of a tree are not contiguous, so their rows are compacted in place:
// row L_b + i receives row L_b + path_i, path_0 = 0 (the root),
// path_i = accepted_nodes[b, i - 1], i = 0 .. accept_len[b].  With paged K/V
// these are the sequence's logical rows, mapped through its page table.
//
// GPU formulation.  One workgroup per (layer, sequence, KV head) owns that
// head's slice (D elements of K and of V) of every row of the sequence in
// that layer's cache, so no two workgroups touch the same bytes; one launch
// covers every layer.  Wave 0 reads the path one lane per node
// and validates it (strictly increasing indices in [1, T): a root path of a
// tree whose parents precede their children) together with the KV range.
// Every source slice that moves is then read into LDS before any
// destination is written, so overlapping sources and destinations (path_i
// equal to a later i) are safe.  Rows with path_i == i stay untouched.
// Traffic: 2 x (moved rows) x Hkv x D x element size, read once and written
// once; the kernel is bound by two dependent memory round trips, not bytes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ev_internal.h"

namespace ev {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kCommitThreads = 256;

template <typename TK, int D>
__global__ __launch_bounds__(kCommitThreads) void kv_commit_rows(const CommitKernelArgs a) {
  constexpr int VPR = D * static_cast<int>(sizeof(TK)) / 16;   // 16-byte vectors per (row, head) slice
  __shared__ u32x4_t stage[2 * kMaxTree * VPR];                // K slices, then V slices
  __shared__ int32_t path[kMaxTree];
  __shared__ int32_t moved[kMaxTree];                          // path positions whose row moves
  __shared__ int32_t nmove_sh, ok_sh;
  const int tid = threadIdx.x;
  const int layer = blockIdx.x / (a.B * a.Hkv);
  const int b = (blockIdx.x / a.Hkv) % a.B, h = blockIdx.x % a.Hkv;
  const int T = a.T, L = a.L[b];

  const bool paged = a.page_size != 0;
  if (tid < 64) {
    bool range_ok;
    if (paged) {   // every page of the sequence's L + T rows lies inside the array
      const int64_t np = (static_cast<int64_t>(L) + T + a.page_size - 1) / a.page_size;
      bool ok = true;
      for (int64_t j = tid; j < np; j += 64) {
        const int64_t pg = a.page_table[static_cast<int64_t>(b) * a.pps + j];
        ok = ok && pg >= 0 && pg < a.num_pages;
      }
      range_ok = !__any(!ok);
    } else {
      const int64_t lo = a.kv_indptr[b], hi = a.kv_indptr[b + 1];
      range_ok = lo >= 0 && lo + L + T <= hi && hi <= a.num_kv_rows;
    }
    const int n = a.accept_len[b];
    const int nn = n < 0 ? 0 : n;
    // lane i holds path_i (i <= nn), -1 past the path
    int node = -1;
    if (tid == 0) node = 0;
    else if (tid <= nn && tid - 1 < T) node = a.accepted_nodes[b * T + tid - 1];
    const int prev = __shfl_up(node, 1);
    const bool lane_ok = tid == 0 || tid > nn || (node > 0 && node < T && node > prev);
    const bool path_ok = n < T && __all(lane_ok);
    const bool moves = path_ok && range_ok && tid >= 1 && tid <= nn && node != tid;
    const uint64_t mv = __ballot(moves);
    if (moves) moved[__popcll(mv & ((1ull << tid) - 1ull))] = tid;
    path[tid] = node;
    if (tid == 0) {
      nmove_sh = __popcll(mv);
      ok_sh = range_ok && path_ok;
      if (h == 0 && layer == 0) {
        a.new_lens[b] = !range_ok ? -1 : (path_ok ? L + nn + 1 : L + 1);
        a.flags[b] = !range_ok ? EAGLE_FLAG_BAD_KV_RANGE : (path_ok ? 0u : EAGLE_FLAG_BAD_TREE);
      }
    }
  }
  __syncthreads();
  if (!ok_sh) return;
  const int nmove = nmove_sh;
  if (nmove == 0) return;

  // physical row of the sequence's logical row x (validated above)
  const int64_t base = paged ? 0 : a.kv_indptr[b];
  auto phys = [&](int64_t x) -> int64_t {
    if (!paged) return base + x;
    return static_cast<int64_t>(a.page_table[static_cast<int64_t>(b) * a.pps + x / a.page_size]) * a.page_size +
           x % a.page_size;
  };
  // slice of row r for this head, as 16-byte vectors
  const int64_t rowstride = static_cast<int64_t>(a.Hkv) * VPR;
  const int64_t loff = static_cast<int64_t>(layer) * (a.layer_stride * static_cast<int64_t>(sizeof(TK)) / 16);
  u32x4_t* const kp = reinterpret_cast<u32x4_t*>(a.k) + loff + static_cast<int64_t>(h) * VPR;
  u32x4_t* const vp = reinterpret_cast<u32x4_t*>(a.v) + loff + static_cast<int64_t>(h) * VPR;
  const int total = 2 * nmove * VPR;
  for (int idx = tid; idx < total; idx += kCommitThreads) {
    const int which = idx / (nmove * VPR);   // 0: K, 1: V
    const int rem = idx - which * nmove * VPR;
    const int j = rem / VPR, c = rem - j * VPR;
    const int64_t src = phys(L + path[moved[j]]) * rowstride + c;
    stage[idx] = which ? vp[src] : kp[src];
  }
  __syncthreads();   // every source read before any destination is written
  for (int idx = tid; idx < total; idx += kCommitThreads) {
    const int which = idx / (nmove * VPR);
    const int rem = idx - which * nmove * VPR;
    const int j = rem / VPR, c = rem - j * VPR;
    const int64_t dst = phys(L + moved[j]) * rowstride + c;
    if (which) vp[dst] = stage[idx];
    else kp[dst] = stage[idx];
  }
}

template <typename TK>
hipError_t launch_t(const CommitKernelArgs& a, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(a.layers * a.B * a.Hkv)), block(kCommitThreads);
  if (a.D == 128) hipLaunchKernelGGL((kv_commit_rows<TK, 128>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((kv_commit_rows<TK, 64>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace

int launch_kv_commit(const CommitKernelArgs& args, int kv_bf16, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const hipError_t e = kv_bf16 ? launch_t<uint16_t>(args, st) : launch_t<float>(args, st);
  return static_cast<int>(e);
}

}  // namespace ev
