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
// GPU formulation.  One workgroup per (layer, sequence, group of KV heads)
// owns that layer's rows of the sequence for those heads (a row's heads are
// contiguous, so a group's part of a row is one run), so no two workgroups
// touch the same bytes; one launch covers every layer.  The host picks the
// groups so that a launch has at most about 256 workgroups: one head each
// for a single sequence, whole rows for a large batch.  Wave 0 reads the path one
// lane per node and validates it (strictly increasing indices in [1, T): a
// root path of a tree whose parents precede their children) together with
// the KV range, and resolves each moving row's physical source and
// destination once.  The moves, laid end to end in path order, are then
// copied in fixed-size chunks (a move may span two): every source vector of a
// chunk is read into registers before any destination of the chunk is
// written, so a source equal to a destination of the same chunk (path_i equal
// to a later i) is read in time, and a later chunk's sources (rows
// L_b + path_j, path_j >= j, of moves j at or past the earlier chunk's) are
// never an earlier chunk's destinations (rows L_b + i, i <= j, path_j != j).
// Rows with path_i == i stay untouched.
// Traffic: 2 x (moved rows) x Hkv x D x element size, read once and written
// once; the kernel is bound by two dependent memory round trips, not bytes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ev_device.h"
#include "ev_internal.h"

namespace ev {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kCommitThreads = 256;

constexpr int kCommitRegs = 8;    // 16-byte vectors a thread carries per chunk

template <typename TK, int D>
__global__ __launch_bounds__(kCommitThreads) void kv_commit_rows(const CommitKernelArgs a) {
  __shared__ int64_t src_row[kMaxTree], dst_row[kMaxTree];     // physical rows of move j
  __shared__ int32_t nmove_sh, ok_sh;
  const int tid = threadIdx.x;
  const int hg = blockIdx.x % a.head_groups;
  const int layer = blockIdx.x / (a.B * a.head_groups), b = (blockIdx.x / a.head_groups) % a.B;
  const int T = a.T, L = a.L[b];

  const bool paged = a.page_size != 0;
  // physical row of the sequence's logical row x (validated before use)
  auto phys = [&](int64_t x) -> int64_t {
    if (!paged) return a.kv_indptr[b] + x;
    return static_cast<int64_t>(a.page_table[static_cast<int64_t>(b) * a.pps + x / a.page_size]) * a.page_size +
           x % a.page_size;
  };
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
    if (moves) {
      const int j = __popcll(mv & ((1ull << tid) - 1ull));
      src_row[j] = phys(L + node);
      dst_row[j] = phys(L + tid);
    }
    if (tid == 0) {
      nmove_sh = __popcll(mv);
      ok_sh = range_ok && path_ok;
      if (layer == 0 && hg == 0) {
        a.new_lens[b] = !range_ok ? -1 : (path_ok ? L + nn + 1 : L + 1);
        a.flags[b] = !range_ok ? EAGLE_FLAG_BAD_KV_RANGE : (path_ok ? 0u : EAGLE_FLAG_BAD_TREE);
      }
    }
  }
  __syncthreads();
  if (!ok_sh) return;
  const int nmove = nmove_sh;
  if (nmove == 0) return;

  // this group's part of a row (its heads), as 16-byte vectors, and the row stride
  const int vhead = D * static_cast<int>(sizeof(TK)) / 16;
  const int vrow = a.Hkv / a.head_groups * vhead;
  const int64_t vstride = static_cast<int64_t>(a.Hkv) * vhead;
  const int64_t loff = static_cast<int64_t>(layer) * (a.layer_stride * static_cast<int64_t>(sizeof(TK)) / 16) +
                       static_cast<int64_t>(hg) * vrow;
  u32x4_t* const kp = reinterpret_cast<u32x4_t*>(a.k) + loff;
  u32x4_t* const vp = reinterpret_cast<u32x4_t*>(a.v) + loff;
  const int per_move = 2 * vrow;   // K row, then V row
  // the nmove * per_move vectors are copied in chunks of one vector per slot
  // of every thread; slot k of a thread covers vector idx = start + tid +
  // k * kCommitThreads, i.e. (move j, position rem within it), and the pair
  // advances by a fixed step per slot, so only the chunk's first slot divides
  constexpr int kChunk = kCommitThreads * kCommitRegs;
  const int dj = kCommitThreads / per_move, dr = kCommitThreads % per_move;
  const int total = nmove * per_move;
  for (int start = 0; start < total; start += kChunk) {
    const int end = min(start + kChunk, total);
    const int rounds = (end - start + kCommitThreads - 1) / kCommitThreads;   // the same in every wave
    const int jfirst = start / per_move;
    // the reads of a round have no per-lane condition (a lane past the chunk
    // re-reads its position of the chunk's first move), so a thread's
    // requests are in flight together
    u32x4_t r[kCommitRegs];
    {
      int idx = start + tid, j = idx / per_move, rem = idx % per_move;
#pragma unroll
      for (int k = 0; k < kCommitRegs; ++k) {
        if (k < rounds) {
          const bool v = rem >= vrow;
          const u32x4_t* const base = v ? vp : kp;
          r[k] = base[src_row[idx < end ? j : jfirst] * vstride + (v ? rem - vrow : rem)];
        }
        idx += kCommitThreads;
        j += dj;
        rem += dr;
        if (rem >= per_move) { rem -= per_move; ++j; }
      }
    }
    loads_after();     // this thread's reads have landed ...
    __syncthreads();   // ... and so have every thread's: no destination of the chunk is written before
    {
      int idx = start + tid, j = idx / per_move, rem = idx % per_move;
#pragma unroll
      for (int k = 0; k < kCommitRegs; ++k) {
        if (idx < end) {
          const bool v = rem >= vrow;
          const int64_t dst = dst_row[j] * vstride + (v ? rem - vrow : rem);
          if (v) vp[dst] = r[k];
          else kp[dst] = r[k];
        }
        idx += kCommitThreads;
        j += dj;
        rem += dr;
        if (rem >= per_move) { rem -= per_move; ++j; }
      }
    }
  }
}

template <typename TK>
hipError_t launch_t(const CommitKernelArgs& a, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(a.layers * a.B * a.head_groups)), block(kCommitThreads);
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
