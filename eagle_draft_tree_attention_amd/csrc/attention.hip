// Tree-masked attention for EAGLE verification, gfx950 (MI355X).
//
// Every draft-tree node i of sequence b attends to the whole prefix KV cache
// of b plus the tree rows of the nodes on its root path, itself included
// (EAGLE notes page: core mechanism §3/§5 and the "tree attention" term;
// lesson page: the glossary entry for tree attention, a standard flash
// attention call whose mask follows the tree topology).  Query head h reads
// KV head h / g (GQA, g = Hq / Hkv).
//
// Work decomposition (split-KV, flash-decoding style):
//   * the R = T * g query rows that share one KV head are processed together,
//     so each K/V tile is read from HBM once and shared by every tree node
//     and every query head of the group;
//   * the prefix of each sequence is cut into splits of `chunk` keys; the last
//     split of a sequence also takes the T tree keys, masked with a per-node
//     64-bit ancestor bitmask built in LDS from the parent array;
//   * each split produces (O, m, l) per row; splits of one sequence are merged
//     by log-sum-exp (the streaming-softmax fusion the Didi page uses to merge
//     ring-attention partials), or written directly when a sequence has one.
//
// Two kernels do the split work:
//   tree_attn_mfma  bf16, R >= 16: 256 threads = 4 waves, each wave owns
//       16*MB rows; 64-key K and V tiles are staged in LDS (V transposed) and
//       shared by the four waves.  S^T = K Q^T and O^T = V^T P^T run on
//       v_mfma_f32_16x16x32_bf16, laid out so that lane (l % 16) owns one query
//       row in both products: softmax statistics and the O rescale stay
//       lane-local and P goes from the S accumulators straight into the B
//       operand of the PV product, with no LDS round trip.  P enters the PV
//       product as a bf16 hi/lo pair (two MFMAs), keeping the output within
//       a few 1e-6 of fp32 arithmetic.
//   tree_attn_fma   fp32 inputs (or bf16 with R < 16): one wave per query row,
//       scalar FMA dot products.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "ev_device.h"
#include "ev_internal.h"

namespace ev {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kRescaleLog2 = 8.f;   // lazy softmax rescale threshold (log2 units)

// Workgroups are handed to the 8 XCDs round-robin; renumber them so that
// consecutive logical ids (the row tiles of one KV chunk) share an XCD and
// therefore its L2.
__device__ __forceinline__ int xcd_remap(int bid, int nwg) {
  const int q = nwg >> 3, r = nwg & 7;
  const int xcd = bid & 7, idx = bid >> 3;
  return (xcd < r) ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

__device__ __forceinline__ int find_seq(const AttnKernelArgs& a, int split) {
  int b = 0;
  while (b + 1 < a.B && a.split_base[b + 1] <= split) ++b;
  return b;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// ---- paged K/V: sequence b's logical row x lives in page
// page_table[b * pps + x / page_size]; an entry outside the array reads page
// 0 instead (the sequence is flagged by paged_range_ok and poisoned)
__device__ __forceinline__ int64_t page_of(const AttnKernelArgs& a, int b, int64_t x) {
  const int64_t pg = a.page_table[static_cast<int64_t>(b) * a.pps + x / a.page_size];
  return (pg >= 0 && pg < a.num_pages) ? pg : 0;
}
__device__ __forceinline__ int64_t paged_row(const AttnKernelArgs& a, int b, int64_t x) {
  return page_of(a, b, x) * a.page_size + x % a.page_size;
}
// every page of sequence b (its L_b + T rows) lies inside the array (all
// lanes of the wave return the same answer)
__device__ __forceinline__ bool paged_range_ok(const AttnKernelArgs& a, int b, int lane) {
  const int64_t np = (static_cast<int64_t>(a.L[b]) + a.T + a.page_size - 1) / a.page_size;
  bool ok = true;
  for (int64_t j = lane; j < np; j += 64) {
    const int64_t pg = a.page_table[static_cast<int64_t>(b) * a.pps + j];
    ok = ok && pg >= 0 && pg < a.num_pages;
  }
  return !__any(!ok);
}

// Flags of sequence b from values already loaded: p = parents[b][lane] (lane
// < T), kv0/kv1 = kv_indptr[b], kv_indptr[b + 1] (contiguous K/V).  All lanes
// of the wave return the same word.
__device__ __forceinline__ uint32_t seq_flags(const AttnKernelArgs& a, int b, int lane, int p, int64_t kv0, int64_t kv1) {
  const bool ok = lane >= a.T || ((lane == 0) ? (p == -1) : (p >= 0 && p < lane));
  uint32_t bad = __any(!ok) ? EAGLE_FLAG_BAD_TREE : 0u;
  if (a.page_size) {
    if (!paged_range_ok(a, b, lane)) bad |= EAGLE_FLAG_BAD_KV_RANGE;
  } else if (!(kv0 >= 0 && kv1 <= a.num_kv_rows && kv1 - kv0 >= (int64_t)a.L[b] + a.T)) {
    bad |= EAGLE_FLAG_BAD_KV_RANGE;
  }
  return bad;
}

// Validate sequence b (parent array + KV range) using one wave's lanes; all
// lanes return the same flag word.
__device__ __forceinline__ uint32_t validate_seq(const AttnKernelArgs& a, int b, int lane, int32_t* par_out) {
  const int T = a.T;
  int p = 0;
  bool ok = true;
  if (lane < T) {
    p = a.parents[b * T + lane];
    ok = (lane == 0) ? (p == -1) : (p >= 0 && p < lane);
  }
  if (par_out && lane < 64) par_out[lane] = p;
  uint32_t bad = __any(!ok) ? EAGLE_FLAG_BAD_TREE : 0u;
  if (a.page_size) {
    if (!paged_range_ok(a, b, lane)) bad |= EAGLE_FLAG_BAD_KV_RANGE;
    return bad;
  }
  const int64_t kv0 = a.kv_indptr[b], kv1 = a.kv_indptr[b + 1];
  if (!(kv0 >= 0 && kv1 <= a.num_kv_rows && kv1 - kv0 >= (int64_t)a.L[b] + T)) bad |= EAGLE_FLAG_BAD_KV_RANGE;
  return bad;
}

__device__ __forceinline__ uint64_t ancestors_of(const int32_t* par, int node) {
  uint64_t m = 0;
  for (int n = node; n >= 0; n = par[n]) m |= 1ull << n;
  return m;
}

// ------------------------------------------------------------- MFMA kernel
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// gfx950 transposing LDS read: in each 16-lane group, lane j supplies the
// address of 4 consecutive 16-bit values (row j of a 16x4 block) and lane i
// receives rows 4e + i/4, column i%4 (e = 0..3).  Pointing lane j at
// V[key0 + j/4][d0 + 4*(j%4)] of a key-major V tile therefore hands lane i
// the four values V[key0 + e][d0 + i]: a column of V, i.e. a row of V^T.
__device__ __forceinline__ i16x4_t lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4_t*)((__attribute__((address_space(3))) char*)(const_cast<uint16_t*>(p))));
}

// One (sequence, KV head, key split, row tile) per workgroup of 4 waves;
// each wave owns MB blocks of 16 query rows.  Per 64-key tile:
//   S^T[key][row] = K Q^T       MB x 4 x D/32 v_mfma_f32_16x16x32_bf16
//   online softmax per row      lane-local (lane % 16 = row)
//   O^T[d][row] += V^T P^T      with P split into bf16 hi + lo
// Key k of block kb sits in S^T row 16*kb + (k%16); lane group lg = lane/16
// holds keys 16*kb + 4*lg + i, which is exactly the k-slot order the PV
// operands need (slots 0..3 from block 2*ks, 4..7 from block 2*ks+1).
//
// K/V tiles move HBM -> LDS with global_load_lds_dwordx4 (lane l of an
// instruction lands at LDS base + 16 l, so no registers are spent on
// staging), through a ring of NST stages: the loads of tile t + NST - 1 are
// issued while tile t is computed, and one barrier per tile both publishes
// tile t and frees the stage tile t - 1 used.  Tiles are stored unpadded
// with 16-byte chunks XOR-swizzled per row, so the K reads (16 rows, one
// chunk column) and the transposing V reads (4 rows x 32 bytes per lane
// group) hit distinct banks.
template <int D>
__device__ __forceinline__ int swz_k(int r) { return r & (D / 8 - 1); }
template <int D>
__device__ __forceinline__ int swz_v(int r) { return 2 * (r & (D / 16 - 1)); }

// wait until at most N of this wave's vector-memory operations are pending
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// LDS byte address of a pointer into a __shared__ array
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) const char*)(p)));
}

// 16 bytes per lane, global -> LDS at lds_base + 16 * lane (lds_base is
// wave-uniform).  Written as inline assembly so that the compiler, which
// cannot see which LDS bytes the transfer writes, does not make every later
// LDS read wait for it: completion is awaited explicitly (wait_vmcnt) before
// the barrier that publishes a tile.
__device__ __forceinline__ void lds_dma16(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "s"(lds_base)
               : "memory", "m0");
}

// The same transfer from a wave-uniform base address held in scalar
// registers plus a 32-bit per-lane byte offset (no 64-bit address per lane).
__device__ __forceinline__ void lds_dma16_sbase(const void* sbase, uint32_t voff_bytes, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff_bytes), "s"(sbase), "s"(lds_base)
               : "memory", "m0");
}
// 4 bytes per lane, global -> LDS at lds_base + 4 * lane (lds_base is
// wave-uniform); like lds_dma16, completion is awaited explicitly.
__device__ __forceinline__ void lds_dma4(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(gptr), "s"(lds_base)
               : "memory", "m0");
}

// 64-bit value of lane src
__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  const uint32_t lo = static_cast<uint32_t>(__shfl(static_cast<int>(static_cast<uint32_t>(v)), src));
  const uint32_t hi = static_cast<uint32_t>(__shfl(static_cast<int>(static_cast<uint32_t>(v >> 32)), src));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Ancestor word (bit j set for every node j on the root path, the node
// included) of node `lane`, for a validated parent array (par < lane for
// lane >= 1), built on the wave's lanes by pointer jumping: lane i holds the
// nodes of its path from i up to, not including, the node it points at
// (initially itself and its parent), and each round appends the pointed-at
// lane's segment and takes over its pointer, doubling the reach.  A depth of
// at most 63 needs at most 6 rounds.  Lanes at or past T return the root.
__device__ __forceinline__ uint64_t ancestor_word(int lane, int T, int par) {
  uint64_t m = lane < T ? (1ull << lane) : 0ull;
  int p = (lane > 0 && lane < T) ? par : 0;
  for (int it = 0; it < 6 && __any(p != 0); ++it) {
    const uint64_t mp = shfl_u64(m, p);
    const int pp = __shfl(p, p);
    m |= mp;
    p = pp;
  }
  return m | 1ull;
}

__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
  return reinterpret_cast<const void*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// cache policy of partial results that workgroups on other XCDs read inside
// the same launch: system-coherent (sc0 sc1), i.e. past the XCD's own L2
constexpr int kSysCoherent = 1 | 16;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t part_rsrc(const float* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, 0x7fffffff, 0x00020000);
}

// MB = 1: two workgroups per CU (two waves per SIMD, 256 registers each);
// MB = 2: one workgroup per CU, whose waves may then hold 512 registers
// PAGED: K/V rows through per-sequence page tables (a separate instantiation,
// so that the contiguous kernel carries none of it)
template <int D, int MB, int NST, int KG, bool PAGED = false>
__global__ __launch_bounds__(256, MB > 1 ? 1 : 2) void tree_attn_mfma(const AttnKernelArgs a) {
  static_assert(KG == 1 || (KG == 2 && MB == 1), "key halves are split only between single row blocks");
  constexpr int KSTEPS = D / 32;          // QK^T contraction steps
  constexpr int DBLK = D / 16;            // output column blocks
  constexpr int CH = D / 8;               // 16-byte chunks per row
  constexpr int TILE = kTileKeys * D;     // elements of one K or V tile
  constexpr int RPI = 64 / CH;            // rows per 1 KB load instruction
  constexpr int IPW = kTileKeys / RPI / 4;   // K (and V) load instructions per wave and tile
  static_assert(IPW >= 1 && 2 * IPW * (NST - 1) < 64, "load geometry");

  __shared__ __attribute__((aligned(1024))) uint16_t kv_lds[NST * 2 * TILE];
  __shared__ int32_t par_lds[4][kMaxTree];   // each wave's copy of the parent array

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lg = lane >> 4, ln = lane & 15;
  // KG = 2: waves w and w + 2 own the same row block and take the first and
  // the second 32 keys of every tile; their states are combined at the end
  const int rw = wave % (4 / KG);
  const int kh = __builtin_amdgcn_readfirstlane(wave / (4 / KG));
  // The launch scalars (and the first sequence's split range, prefix length
  // and expected row offset) are requested together and waited for once,
  // instead of one dependent round trip per use: first one field of each
  // 64-byte line of the argument block that the prologue reads.
  {
    const void* l0 = a.k;
    const int l1 = a.nwg;
    uint64_t* const l2 = a.stamps;
    const int l3 = a.L[0], l19 = a.split_base[1], l35 = a.kv0_guess[0];
    asm volatile("" ::"s"(l0), "s"(l1), "s"(l2), "s"(l3), "s"(l19), "s"(l35));
  }
  const int a_nwg = a.nwg, a_rt = a.row_tiles, a_ts = a.total_splits, a_B = a.B;
  const int T = a.T, g = a.g, R = a.R, Hq = a.Hq;
  const int b0_base = 0, b0_next = a.split_base[1], b0_L = a.L[0], b0_guess = a.kv0_guess[0];
  const void* const a_k = a.k;
  const void* const a_v = a.v;
  const int32_t* const a_par = a.parents;
  uint64_t* const a_stamps = a.stamps;
  asm volatile("" ::"s"(a_nwg), "s"(a_rt), "s"(a_ts), "s"(a_B), "s"(T), "s"(g), "s"(R), "s"(Hq), "s"(b0_next), "s"(b0_L),
               "s"(b0_guess), "s"(a_k), "s"(a_v), "s"(a_par), "s"(a_stamps));
  stamp(a_stamps, 0);
  const int logical = xcd_remap(blockIdx.x, a_nwg);
  // logical order: row tile fastest, then key split, then KV head, so the
  // row tiles of one K/V chunk share an XCD's L2 and every XCD receives its
  // share of the splits that carry the tree tile
  const int rt = logical % a_rt;
  const int split = (logical / a_rt) % a_ts;
  const int hk = logical / (a_rt * a_ts);
  const int64_t slot = logical;   // partial-row slot of this workgroup
  const int b = a_B == 1 ? 0 : find_seq(a, split);
  const int sb0 = b == 0 ? b0_base : a.split_base[b];
  const int s_local = split - sb0;
  const int S = (b == 0 ? b0_next : a.split_base[b + 1]) - sb0;
  const int L = b == 0 ? b0_L : a.L[b];
  const int row_base = rt * a.rows_per_tile + rw * 16 * MB;   // lane rows: row_base + 16*rb + ln

  // The parent array (each wave its own copy, straight into LDS), the query
  // rows and the first tile are requested in that order, the tile from the
  // expected row offset of the sequence, without waiting for kv_indptr[b].
  // The sequence is validated and its ancestor words are built once the
  // parents and the query rows have landed, while the tile is in flight.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  lds_dma4(a_par + b * T + min(lane, T - 1), lds_offset(&par_lds[wave_u][0]));
  constexpr bool paged = PAGED;
  const int guess = b == 0 ? b0_guess : a.kv0_guess[b];
  int64_t kv0 = paged ? 0 : (guess >= 0 ? (int64_t)guess : a.kv_indptr[b]);
  const uint16_t* __restrict__ kbase = reinterpret_cast<const uint16_t*>(a_k) + (int64_t)hk * D;
  const uint16_t* __restrict__ vbase = reinterpret_cast<const uint16_t*>(a_v) + (int64_t)hk * D;
  const int64_t row_stride = (int64_t)a.Hkv * D;   // elements between consecutive KV rows
  const int64_t last_row = a.num_kv_rows - 1;

  const int k_begin = s_local * a.chunk;
  const int k_end = min(k_begin + a.chunk, L);
  const int n_prefix = k_end > k_begin ? (k_end - k_begin + kTileKeys - 1) / kTileKeys : 0;
  const int n_full = (k_end - k_begin) / kTileKeys > 0 ? (k_end - k_begin) / kTileKeys : 0;   // unmasked tiles
  const int n_tiles = n_prefix + (s_local == S - 1 ? 1 : 0);

  // K/V tile t -> ring stage t % NST.  Full tiles of a split whose prefix
  // rows all lie inside the KV array use precomputed per-lane offsets; any
  // other tile repeats its last valid row past the key count (masked in the
  // softmax) and clamps every row index into the array, so the loads stay in
  // bounds even for a sequence that the validation below rejects.
  const int l_row = lane / CH, l_pos = lane % CH;
  const uint32_t lds_kv = lds_offset(kv_lds);
  // per-lane byte offsets of this wave's transfer lanes inside a tile whose
  // rows are all valid (row r of the tile = row0 + r)
  uint32_t koff[IPW], voff[IPW];
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int r = (wave_u * IPW + j) * RPI + l_row;
    koff[j] = static_cast<uint32_t>(r * row_stride + (l_pos ^ swz_k<D>(r)) * 8) * 2;
    voff[j] = static_cast<uint32_t>(r * row_stride + (l_pos ^ swz_v<D>(r)) * 8) * 2;
  }
  // every prefix row of this split lies inside the KV array (checked once, so
  // full tiles need no per-row clamping)
  bool split_in_bounds = paged || (kv0 >= 0 && kv0 + k_end <= a.num_kv_rows);
  // paged K/V: lane j holds the page of this split's j-th page (a full tile
  // lies inside one page: tiles start at multiples of 64 and pages hold a
  // multiple of 64 rows)
  const int first_page = paged ? k_begin / a.page_size : 0;
  const int64_t my_page = (paged && static_cast<int64_t>(first_page + lane) * a.page_size < (int64_t)L + T)
                              ? page_of(a, b, static_cast<int64_t>(first_page + lane) * a.page_size)
                              : 0;
  auto issue = [&](int t) {
    const uint32_t kdst = lds_kv + static_cast<uint32_t>((t % NST) * 2 * TILE * 2);
    const uint32_t vdst = kdst + TILE * 2;
    if (t < n_full && split_in_bounds) {
      int64_t row0 = kv0 + k_begin + (int64_t)t * kTileKeys;
      if (paged) {
        const int x = k_begin + t * kTileKeys;
        const int pi = x / a.page_size - first_page;
        const int64_t pg = pi < 64 ? (int64_t)__builtin_amdgcn_readlane(static_cast<int>(my_page), pi)
                                   : page_of(a, b, x);
        row0 = pg * a.page_size + x % a.page_size;
      }
      const void* kt = uniform_ptr(kbase + row0 * row_stride);
      const void* vt = uniform_ptr(vbase + row0 * row_stride);
#pragma unroll
      for (int j = 0; j < IPW; ++j) {
        const uint32_t ldsoff = static_cast<uint32_t>((wave_u * IPW + j) * RPI * D * 2);
        lds_dma16_sbase(kt, koff[j], kdst + ldsoff);
        lds_dma16_sbase(vt, voff[j], vdst + ldsoff);
      }
      return;
    }
    const bool tree = t >= n_prefix;
    const int start = tree ? L : k_begin + t * kTileKeys;
    const int cnt = tree ? T : min(kTileKeys, k_end - start);
    const int64_t row0 = kv0 + start;
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      const int r0 = (wave_u * IPW + j) * RPI;
      const int r = r0 + l_row;
      const int64_t gr = paged ? paged_row(a, b, start + min(r, cnt - 1))
                               : min(max(row0 + min(r, cnt - 1), (int64_t)0), last_row);
      lds_dma16(kbase + gr * row_stride + (l_pos ^ swz_k<D>(r)) * 8, kdst + static_cast<uint32_t>(r0 * D * 2));
      lds_dma16(vbase + gr * row_stride + (l_pos ^ swz_v<D>(r)) * 8, vdst + static_cast<uint32_t>(r0 * D * 2));
    }
  };
  // query rows -> B operands of S^T = K Q^T (zero for padding rows)
  bool row_ok[MB];
  int node[MB], head[MB];
  bf16x8_t qf[MB][KSTEPS];
#pragma unroll
  for (int rb = 0; rb < MB; ++rb) {
    const int r = row_base + 16 * rb + ln;
    row_ok[rb] = r < R;
    node[rb] = row_ok[rb] ? r / g : 0;
    head[rb] = hk * g + (row_ok[rb] ? r % g : 0);
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)(b * T + node[rb]) * Hq + head[rb]) * D + 8 * lg;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      const u32x4_t w = row_ok[rb] ? *reinterpret_cast<const u32x4_t*>(qp + 32 * s) : u32x4_t{0, 0, 0, 0};
      qf[rb][s] = __builtin_bit_cast(bf16x8_t, w);
    }
  }
  static_assert(NST == 2, "the prologue requests one tile");
  if (n_tiles > 0) issue(0);

  const int64_t kv0_true = paged ? 0 : a.kv_indptr[b];
  const int64_t kv1_true = paged ? 0 : a.kv_indptr[b + 1];
  // every request before the tile's 2 IPW transfers has completed: the
  // parents and the query rows
  if (n_tiles > 0) wait_vmcnt<2 * IPW>();
  else wait_vmcnt<0>();
  asm volatile("" ::: "memory");   // the parents are read from LDS only after the wait
  stamp(a.stamps, 1);   // parents and query rows
  const int par_lane = lane < T ? par_lds[wave_u][lane] : 0;
  if (kv0 != kv0_true) {   // the expected offset was wrong: request the first tile again
    wait_vmcnt<0>();       // (the first request has landed: no two transfers into one stage)
    kv0 = kv0_true;
    split_in_bounds = kv0 >= 0 && kv0 + k_end <= a.num_kv_rows;
    if (n_tiles > 0) issue(0);
  }
  const uint32_t bad = seq_flags(a, b, lane, par_lane, kv0_true, kv1_true);
  if (s_local == 0 && hk == 0 && rt == 0 && tid == 0) a.flags[b] = bad;
  if (bad) {
    wait_vmcnt<0>();   // no transfer into LDS may outlive the workgroup
    // NaN rows: written here when no separate merge follows (one split, or
    // the merge is done inside this kernel: then split 0 writes its tile)
    if ((S == 1 || (a.fused_merge && s_local == 0)) && kh == 0) {
      for (int rb = 0; rb < MB; ++rb) {
        const int r = row_base + 16 * rb + ln;
        if (r >= R) continue;
        float* o = a.out + ((int64_t)(b * T + r / g) * Hq + hk * g + r % g) * D;
        for (int db = 0; db < DBLK; ++db)
          *reinterpret_cast<f32x4_t*>(o + 16 * db + 4 * lg) = f32x4_t{__builtin_nanf(""), __builtin_nanf(""),
                                                                       __builtin_nanf(""), __builtin_nanf("")};
      }
    }
    return;
  }
  // ancestor words on the wave's own lanes (no LDS, no barrier)
  const uint64_t anc_lane = ancestor_word(lane, T, par_lane);
  uint64_t anc_row[MB];
#pragma unroll
  for (int rb = 0; rb < MB; ++rb) anc_row[rb] = shfl_u64(anc_lane, node[rb]);
  stamp(a.stamps, 2);   // ancestor words

  // O^T accumulators, and the row sums of P: the matrix unit adds them as the
  // product of an all-ones block with P^T (every lane of a row then holds the
  // row's whole sum, of exactly the hi + lo values that enter O)
  f32x4_t o[MB][DBLK], lacc[MB];
  float m_run[MB], l_run[MB];
#pragma unroll
  for (int rb = 0; rb < MB; ++rb) {
    m_run[rb] = kNegInf;
    lacc[rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int db = 0; db < DBLK; ++db) o[rb][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const bf16x8_t ones = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f,
                         (__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};
  const float c = a.scale_log2;

  // One 64-key tile from ring stage ST (a compile-time constant, so every LDS
  // address below is a per-lane register plus an immediate).  MASK: partial
  // prefix tile (key < cnt) or tree tile (key < T and key an ancestor of the
  // row's node).  The tile is processed as two 32-key halves.
  auto tile = [&](auto mask_tag, const uint16_t* kst, bool is_tree, int cnt) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const uint16_t* vst = kst + TILE;
    f32x4_t sacc[4][MB];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int rb = 0; rb < MB; ++rb) sacc[kb][rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // S^T for keys 32 h .. 32 h + 31 (key blocks 2h, 2h+1).  All K fragments
    // of the half are read before the first product; the products of one
    // block accumulate back to back (same shape, same accumulator).
    auto qk = [&](auto h_tag) __attribute__((always_inline)) {
      constexpr int H = decltype(h_tag)::value;
      if constexpr (MB > 1) {   // each fragment feeds MB products: read it just before them
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            const int r = 16 * (2 * H + kk) + ln;
            const bf16x8_t f = *reinterpret_cast<const bf16x8_t*>(kst + r * D + (((lg + 4 * s) ^ swz_k<D>(r)) * 8));
#pragma unroll
            for (int rb = 0; rb < MB; ++rb)
              sacc[2 * H + kk][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f, qf[rb][s], sacc[2 * H + kk][rb], 0, 0, 0);
          }
        return;
      }
      bf16x8_t kf[KSTEPS][2];
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int r = 16 * (2 * H + kk) + ln;
          kf[s][kk] = *reinterpret_cast<const bf16x8_t*>(kst + r * D + (((lg + 4 * s) ^ swz_k<D>(r)) * 8));
        }
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int rb = 0; rb < MB; ++rb)
            sacc[2 * H + kk][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s][kk], qf[rb][s], sacc[2 * H + kk][rb], 0, 0, 0);
    };
    // Masks of the half (partial prefix tile: key < cnt; tree tile: ancestors).
    auto mask_half = [&](auto h_tag) __attribute__((always_inline)) {
      constexpr int H = decltype(h_tag)::value;
      if constexpr (MASK) {
#pragma unroll
        for (int rb = 0; rb < MB; ++rb) {
          // visible keys of this row as a 64-bit word: the ancestor bits on
          // the tree tile, the first cnt keys on a partial prefix tile
          const uint64_t vis = is_tree ? anc_row[rb] : (cnt >= 64 ? ~0ull : ((1ull << cnt) - 1ull));
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            const uint32_t nib = static_cast<uint32_t>(vis >> (16 * (2 * H + kk) + 4 * lg)) & 0xFu;
#pragma unroll
            for (int i = 0; i < 4; ++i)
              sacc[2 * H + kk][rb][i] = ((nib >> i) & 1u) ? sacc[2 * H + kk][rb][i] : kNegInf;
          }
        }
      }
    };
    // this lane's largest score of key blocks [kb0, kb1)
    auto lane_max = [&](int rb, int kb0, int kb1) __attribute__((always_inline)) -> float {
      float tmax = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        if (kb >= kb0 && kb < kb1)
          tmax = fmaxf(tmax, fmaxf(fmaxf(sacc[kb][rb][0], sacc[kb][rb][1]), fmaxf(sacc[kb][rb][2], sacc[kb][rb][3])));
      return tmax;
    };
    // The reference maximum of a row moves only when a score exceeds it by
    // more than 2^kRescaleLog2 (P then stays below that, harmless in fp32
    // and in the bf16 hi/lo pair), so most tiles skip the cross-lane maximum
    // and the rescale of O.  The test is wave-uniform.
    auto rescale = [&](int rb, float tmax) __attribute__((always_inline)) {
      if (__any(tmax * c > m_run[rb] + kRescaleLog2)) {
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float m_new = fmaxf(m_run[rb], tmax * c);
        const float alpha = (m_new == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_run[rb] - m_new);
        lacc[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < DBLK; ++db) o[rb][db] *= alpha;
        m_run[rb] = m_new;
      }
    };
    // P of the half from the current reference maximum: exp2, then the bf16
    // pair hi = bf16(p), lo = bf16(p - hi), two values at a time (the packed
    // hi word gives both hi values back as fp32 by a shift and a mask)
    auto p_half = [&](auto h_tag, bf16x8_t (&pb)[MB], bf16x8_t (&pl)[MB]) __attribute__((always_inline)) {
      constexpr int H = decltype(h_tag)::value;
#pragma unroll
      for (int rb = 0; rb < MB; ++rb) {
        const float m_use = (m_run[rb] == kNegInf) ? 0.f : m_run[rb];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[2 * H + (e >> 2)][rb][e & 3], c, -m_use));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[2 * H + (e >> 2)][rb][(e & 3) + 1], c, -m_use));
          const bf16x2_t h = {(__bf16)p0, (__bf16)p1};
          const uint32_t hw = __builtin_bit_cast(uint32_t, h);
          const bf16x2_t l = {(__bf16)(p0 - __uint_as_float(hw << 16)), (__bf16)(p1 - __uint_as_float(hw & 0xFFFF0000u))};
          pb[rb][e] = h[0];
          pb[rb][e + 1] = h[1];
          pl[rb][e] = l[0];
          pl[rb][e + 1] = l[1];
        }
      }
    };
    // P for the half: masks, lazy reference maximum, exp2, bf16 hi/lo pair
    auto softmax = [&](auto h_tag, bf16x8_t (&pb)[MB], bf16x8_t (&pl)[MB]) __attribute__((always_inline)) {
      constexpr int H = decltype(h_tag)::value;
      mask_half(h_tag);
#pragma unroll
      for (int rb = 0; rb < MB; ++rb) rescale(rb, lane_max(rb, 2 * H, 2 * H + 2));
      p_half(h_tag, pb, pl);
    };
    // V^T fragments of the half: lane (lg, ln) points the transposing read
    // at key 32 h + 4 lg + ln/4 (and + 16), dims 16 db + 4 (ln % 4) .. + 3
    auto read_v = [&](auto h_tag, bf16x8_t (&va)[DBLK]) __attribute__((always_inline)) {
      constexpr int H = decltype(h_tag)::value;
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
        const int r = 32 * H + 4 * lg + (ln >> 2);
        const int chunk = 2 * db + ((ln & 3) >> 1);
        const uint16_t* vp = vst + r * D + ((chunk ^ swz_v<D>(r)) * 8) + 4 * (ln & 1);
        const i16x4_t lo4 = lds_read_tr16(vp);
        const i16x4_t hi4 = lds_read_tr16(vp + 16 * D);   // key + 16: same swizzle (r & 7 unchanged)
        va[db] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    };
    // hi products of every column block, then the lo products: the two
    // MFMAs into one accumulator are DBLK instructions apart
    auto pv_mfma = [&](const bf16x8_t (&va)[DBLK], const bf16x8_t (&pb)[MB], const bf16x8_t (&pl)[MB]) __attribute__((always_inline)) {
#pragma unroll
      for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int rb = 0; rb < MB; ++rb) o[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[db], pb[rb], o[rb][db], 0, 0, 0);
#pragma unroll
      for (int rb = 0; rb < MB; ++rb) lacc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[rb], lacc[rb], 0, 0, 0);
#pragma unroll
      for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int rb = 0; rb < MB; ++rb) o[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[db], pl[rb], o[rb][db], 0, 0, 0);
#pragma unroll
      for (int rb = 0; rb < MB; ++rb) lacc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pl[rb], lacc[rb], 0, 0, 0);
    };
    // O^T += V^T P^T for keys 32 h .. 32 h + 31
    auto pv = [&](auto h_tag, const bf16x8_t (&pb)[MB], const bf16x8_t (&pl)[MB]) __attribute__((always_inline)) {
      bf16x8_t va[DBLK];
      read_v(h_tag, va);
      pv_mfma(va, pb, pl);
    };
    using H0 = std::integral_constant<int, 0>;
    using H1 = std::integral_constant<int, 1>;
    bf16x8_t pb0[MB], pl0[MB], pb1[MB], pl1[MB];
    if constexpr (KG == 1) {
      // one reference-maximum test for the whole tile, and every V fragment
      // requested before the softmax: the exponentials of both halves and
      // the PV products then form one straight run (no branch between them),
      // so the matrix work of one half overlaps the vector work of the other
      // and the LDS reads of V overlap the softmax
      qk(H0{});
      qk(H1{});
      bf16x8_t va0[DBLK], va1[DBLK];
      read_v(H0{}, va0);
      read_v(H1{}, va1);
      mask_half(H0{});
      mask_half(H1{});
      // exponent arguments x = s c - m of the lane's 16 scores of each row
      // block; the rescale test runs on them (results of an fma need no NaN
      // quieting before a maximum, raw matrix results would)
#pragma unroll
      for (int rb = 0; rb < MB; ++rb) {
        const float m_use = (m_run[rb] == kNegInf) ? 0.f : m_run[rb];
        float xs[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) xs[i] = __builtin_fmaf(sacc[i >> 2][rb][i & 3], c, -m_use);
        float tx = xs[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) tx = fmaxf(tx, xs[i]);
        // same test as rescale(): some score exceeds the reference maximum by
        // more than 2^kRescaleLog2 (any finite score while there is none)
        if (__any(tx > (m_run[rb] == kNegInf ? kNegInf : kRescaleLog2))) {
          tx = fmaxf(tx, __shfl_xor(tx, 16));
          tx = fmaxf(tx, __shfl_xor(tx, 32));
          const float m_new = fmaxf(m_run[rb], tx + m_use);
          const float alpha = (m_new == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_run[rb] - m_new);
          lacc[rb] *= alpha;
#pragma unroll
          for (int db = 0; db < DBLK; ++db) o[rb][db] *= alpha;
          m_run[rb] = m_new;
          const float m_nu = (m_new == kNegInf) ? 0.f : m_new;
#pragma unroll
          for (int i = 0; i < 16; ++i) xs[i] = __builtin_fmaf(sacc[i >> 2][rb][i & 3], c, -m_nu);
        }
        // P = 2^x as the bf16 pair hi = bf16(p), lo = bf16(p - hi), two at a time
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
          const float p0 = __builtin_amdgcn_exp2f(xs[e]), p1 = __builtin_amdgcn_exp2f(xs[e + 1]);
          const bf16x2_t h = {(__bf16)p0, (__bf16)p1};
          const uint32_t hw = __builtin_bit_cast(uint32_t, h);
          const bf16x2_t l = {(__bf16)(p0 - __uint_as_float(hw << 16)), (__bf16)(p1 - __uint_as_float(hw & 0xFFFF0000u))};
          bf16x8_t& hb = e < 8 ? pb0[rb] : pb1[rb];
          bf16x8_t& lb = e < 8 ? pl0[rb] : pl1[rb];
          hb[e & 7] = h[0];
          hb[(e & 7) + 1] = h[1];
          lb[e & 7] = l[0];
          lb[(e & 7) + 1] = l[1];
        }
      }
      pv_mfma(va0, pb0, pl0);
      pv_mfma(va1, pb1, pl1);
    } else if (kh == 0) {
      qk(H0{});
      softmax(H0{}, pb0, pl0);
      pv(H0{}, pb0, pl0);
    } else {
      qk(H1{});
      softmax(H1{}, pb1, pl1);
      pv(H1{}, pb1, pl1);
    }
  };

  auto run_tile = [&](int t, const uint16_t* kst) __attribute__((always_inline)) {
    if (t < n_full) {
      tile(std::integral_constant<bool, false>{}, kst, false, kTileKeys);
    } else {
      const bool is_tree = t >= n_prefix;
      const int cnt = is_tree ? T : min(kTileKeys, k_end - (k_begin + t * kTileKeys));
      tile(std::integral_constant<bool, true>{}, kst, is_tree, cnt);
    }
  };
  // Older waves win issue arbitration, so a workgroup dispatched onto a CU
  // after another one (or in a later dispatch round) falls behind and ends
  // last.  With several tiles per workgroup, the later half of the grid
  // runs at a raised priority, which evens out the finish times.
  if (a.late_priority && static_cast<int>(blockIdx.x) >= a_nwg / 2) __builtin_amdgcn_s_setprio(1);   // a_nwg = grid size
  // two stages: the stage of every LDS address is a compile-time constant
  static_assert(NST == 2, "the tile loop alternates two ring stages");
  auto step = [&](int t, auto stage_tag) __attribute__((always_inline)) {
    constexpr int ST = decltype(stage_tag)::value;
    wait_vmcnt<0>();   // this wave's loads of tile t have landed
    __syncthreads();   // every wave's part of tile t is in LDS; the other stage is free
    if (t + 1 < n_tiles) issue(t + 1);
    run_tile(t, kv_lds + ST * 2 * TILE);
  };
  for (int t = 0; t < n_tiles; t += 2) {
    step(t, std::integral_constant<int, 0>{});
    if (t + 1 < n_tiles) step(t + 1, std::integral_constant<int, 1>{});
  }
  stamp(a.stamps, 3);   // tile loop done
  stamp_value(a.stamps, 30, static_cast<uint64_t>(n_tiles));
  stamp_value(a.stamps, 31, static_cast<uint64_t>(s_local) | (static_cast<uint64_t>(hk) << 16) |
                                (static_cast<uint64_t>(rt) << 32) | (static_cast<uint64_t>(b) << 48));

  // every lane of a row holds the row's whole sum: a quarter per lane keeps
  // the sums over the row's four lanes below exact (powers of two)
#pragma unroll
  for (int rb = 0; rb < MB; ++rb) l_run[rb] = lacc[rb][0] * 0.25f;

  if constexpr (KG == 2) {
    // the key-half states of each row meet in the (now free) K/V ring:
    // M = max(m0, m1), O = 2^(m0-M) O0 + 2^(m1-M) O1, l likewise
    __syncthreads();   // every wave has finished its last tile
    f32x4_t* xo = reinterpret_cast<f32x4_t*>(kv_lds);   // [row block][db][lane]
    float* xm = reinterpret_cast<float*>(xo + 2 * DBLK * 64);   // [row block][lane][m, l]
    if (kh == 1) {
#pragma unroll
      for (int db = 0; db < DBLK; ++db) xo[(rw * DBLK + db) * 64 + lane] = o[0][db];
      xm[(rw * 64 + lane) * 2] = m_run[0];
      xm[(rw * 64 + lane) * 2 + 1] = l_run[0];
    }
    __syncthreads();
    if (kh == 0) {
      const float m1 = xm[(rw * 64 + lane) * 2], l1 = xm[(rw * 64 + lane) * 2 + 1];
      const float M = fmaxf(m_run[0], m1);
      const float Mu = (M == kNegInf) ? 0.f : M;
      const float a0 = __builtin_amdgcn_exp2f(m_run[0] - Mu), a1 = __builtin_amdgcn_exp2f(m1 - Mu);
#pragma unroll
      for (int db = 0; db < DBLK; ++db) o[0][db] = o[0][db] * a0 + xo[(rw * DBLK + db) * 64 + lane] * a1;
      l_run[0] = l_run[0] * a0 + l1 * a1;
      m_run[0] = M;
    }
  }

  // epilogue (KG = 2: the waves of the first key half hold the rows)
  const bool fused = S > 1 && a.fused_merge;
  float l_fin[MB];
#pragma unroll
  for (int rb = 0; rb < MB; ++rb) {
    float l_tot = l_run[rb];
    l_tot += __shfl_xor(l_tot, 16);
    l_tot += __shfl_xor(l_tot, 32);
    l_fin[rb] = l_tot;
    const int r = row_base + 16 * rb + ln;
    if (!row_ok[rb] || kh != 0) continue;
    if (S == 1) {
      const float inv = 1.f / l_tot;
      float* op = a.out + ((int64_t)(b * T + node[rb]) * Hq + head[rb]) * D + 4 * lg;
#pragma unroll
      for (int db = 0; db < DBLK; ++db) *reinterpret_cast<f32x4_t*>(op + 16 * db) = o[rb][db] * inv;
    } else {
      const int64_t prow = slot * a.rows_per_tile + (r - rt * a.rows_per_tile);
      float* op = a.opart + prow * D + 4 * lg;
      if (fused) {   // read by workgroups on other XCDs: written through to memory
        const __amdgpu_buffer_rsrc_t prs = part_rsrc(a.opart);
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, o[rb][db]), prs,
                                                 static_cast<int>((prow * D + 16 * db + 4 * lg) * 4), 0, kSysCoherent);
      } else {
#pragma unroll
        for (int db = 0; db < DBLK; ++db) *reinterpret_cast<f32x4_t*>(op + 16 * db) = o[rb][db];
        if (lg == 0)
          *reinterpret_cast<uint64_t*>(a.mlpart + 2 * prow) = static_cast<uint64_t>(__float_as_uint(m_run[rb])) |
                                                              (static_cast<uint64_t>(__float_as_uint(l_tot)) << 32);
      }
    }
  }
  stamp(a.stamps, 4);   // partial (or final) rows stored
  if (!fused) return;

  // ---- in-kernel merge.  Each partial row's m and l are published as two
  // words tagged with the call's epoch, once the workgroup's partial O rows
  // have reached memory.  Each split then merges its own slice of the tile's
  // rows as soon as the words of all S splits for those rows carry the tag:
  //   out = sum_s w_s O_s,  w_s = 2^(m_s - M) / sum_s' 2^(m_s' - M) l_s'
  const uint64_t tag = static_cast<uint64_t>(static_cast<uint32_t>(a.epoch)) << 32;
  // "some split not arrived" flags of the merge polls, slot it % 3 for poll
  // it.  Poll it clears the slot of poll it + 1: every wave read that slot
  // (as poll it - 2's) before reaching the barrier of poll it - 1, and no
  // wave writes it before passing the barrier of poll it, so one barrier a
  // poll suffices (the runtime's barrier reductions would also load the
  // workgroup size from the kernel's hidden arguments first)
  __shared__ int pending[3];
  if (tid < 3) pending[tid] = 0;
  stores_done();
  __syncthreads();   // every wave's partial O rows are in memory
#pragma unroll
  for (int rb = 0; rb < MB; ++rb) {
    const int r = row_base + 16 * rb + ln;
    if (!row_ok[rb] || lg != 0 || kh != 0) continue;
    uint64_t* rec = a.mlrec + 2 * (slot * a.rows_per_tile + (r - rt * a.rows_per_tile));
    st_u64(rec, tag | __float_as_uint(m_run[rb]));
    st_u64(rec + 1, tag | __float_as_uint(l_fin[rb]));
  }
  stamp(a.stamps, 5);   // m and l published

  constexpr int CG = D / 4;   // 4-column groups per row
  const int rpt = a.rows_per_tile;
  const int rps = (rpt + S - 1) / S;
  const int r_lo = s_local * rps;
  const int nr = min(min(r_lo + rps, rpt), R - rt * rpt) - r_lo;   // rows this split merges
  if (nr <= 0) return;
  const int64_t stride = (int64_t)a.row_tiles * rpt;   // partial rows between splits
  const int64_t prow_lo = ((int64_t)hk * a.total_splits + a.split_base[b]) * stride + (int64_t)rt * rpt + r_lo;
  const int np = nr * S;
  // the K/V ring is free now: [0, 4 KB) lane partials, then m / weights
  // [np] and l [np] (the host keeps 2 np floats within the ring)
  f32x4_t* red = reinterpret_cast<f32x4_t*>(kv_lds);
  float* wsm = reinterpret_cast<float*>(kv_lds) + 1024;
  for (uint32_t it = 0, slot3 = 0;; ++it, slot3 = slot3 == 2 ? 0 : slot3 + 1) {
    int ready = 1;
    for (int p = tid; p < np; p += 256) {
      const int i = p / S, sj = p - i * S;
      const uint64_t* rec = a.mlrec + 2 * (prow_lo + i + (int64_t)sj * stride);
      const uint64_t wm = ld_u64(rec), wl = ld_u64(rec + 1);
      if ((wm & ~0xffffffffull) != tag || (wl & ~0xffffffffull) != tag) ready = 0;
      wsm[p] = __uint_as_float(static_cast<uint32_t>(wm));
      wsm[np + p] = __uint_as_float(static_cast<uint32_t>(wl));
    }
    if (!ready) pending[slot3] = 1;
    if (tid == 0) pending[slot3 == 2 ? 0 : slot3 + 1] = 0;   // the slot of poll it + 1
    __syncthreads();
    if (pending[slot3] == 0) break;
    if (it >= a.spin_limit) {   // gave up: this split's rows are poisoned and the sequence flagged
      for (int e = tid; e < nr * D; e += 256) {
        const int r = rt * rpt + r_lo + e / D;
        a.out[((int64_t)(b * T + r / g) * Hq + hk * g + r % g) * D + e % D] = __builtin_nanf("");
      }
      if (tid == 0)
        __hip_atomic_fetch_or(&a.flags[b], static_cast<uint32_t>(EAGLE_FLAG_INTERNAL), __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_SYSTEM);
      return;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  loads_after();
  stamp(a.stamps, 6);   // every split of the rows has arrived
  // weighted sum: slot = (row, column group, split lane); spl lanes share a
  // (row, column group) and take the splits sl, sl + spl, ... in rounds of
  // 8 loads issued together.  A thread's first round is requested before
  // the weights are formed.
  const __amdgpu_buffer_rsrc_t prs = part_rsrc(a.opart);
  const int items = nr * CG;
  const int spl = items >= 256 ? 1 : min(256 / items, S);
  const int slots = items * spl;
  const int bstride = static_cast<int>(stride * D * 4);
  u32x4_t ov[8];
  auto load_round = [&](int i, int cg, int s0) {
    const int boff = static_cast<int>(((prow_lo + i) * D + 4 * cg) * 4);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      ov[j] = __builtin_amdgcn_raw_buffer_load_b128(prs, boff + min(s0 + j * spl, S - 1) * bstride, 0, kSysCoherent);
  };
  if (tid < slots) {
    const int item = tid % items;
    load_round(item / CG, item % CG, tid / items);
  }
  __syncthreads();
  for (int i = wave; i < nr; i += 4) {   // one wave per row
    float* mw = wsm + i * S;
    const float* lw = wsm + np + i * S;
    float mx = kNegInf;
    for (int sj = lane; sj < S; sj += 64) mx = fmaxf(mx, mw[sj]);
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) mx = fmaxf(mx, __shfl_xor(mx, x));
    const float Mu = (mx == kNegInf) ? 0.f : mx;
    float den = 0.f;
    for (int sj = lane; sj < S; sj += 64) den += __builtin_amdgcn_exp2f(mw[sj] - Mu) * lw[sj];
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) den += __shfl_xor(den, x);
    const float inv = 1.f / den;
    for (int sj = lane; sj < S; sj += 64) mw[sj] = __builtin_amdgcn_exp2f(mw[sj] - Mu) * inv;
  }
  __syncthreads();
  for (int t = tid; t < slots; t += 256) {
    const int item = t % items, sl = t / items;
    const int i = item / CG, cg = item % CG;
    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int s0 = sl; s0 < S; s0 += 8 * spl) {
      if (t != tid || s0 != sl) load_round(i, cg, s0);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float w = (s0 + j * spl < S) ? wsm[i * S + s0 + j * spl] : 0.f;
        acc += w * __builtin_bit_cast(f32x4_t, ov[j]);
      }
    }
    if (spl == 1) {
      const int r = rt * rpt + r_lo + i;
      *reinterpret_cast<f32x4_t*>(a.out + ((int64_t)(b * T + r / g) * Hq + hk * g + r % g) * D + 4 * cg) = acc;
    } else {
      red[sl * items + item] = acc;
    }
  }
  if (spl == 1) {
    stamp(a.stamps, 7);   // merged rows written
    return;
  }
  __syncthreads();
  if (tid < items) {
    f32x4_t acc = red[tid];
    for (int sl = 1; sl < spl; ++sl) acc += red[sl * items + tid];
    const int i = tid / CG, cg = tid % CG;
    const int r = rt * rpt + r_lo + i;
    *reinterpret_cast<f32x4_t*>(a.out + ((int64_t)(b * T + r / g) * Hq + hk * g + r % g) * D + 4 * cg) = acc;
  }
  stamp(a.stamps, 7);   // merged rows written
}

// -------------------------------------------------------------- FMA kernel
template <typename TIn>
__device__ __forceinline__ float load_elem(const TIn* p, int64_t i);
template <>
__device__ __forceinline__ float load_elem<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p, int64_t i) { return bf16_bits_to_f32(p[i]); }

template <typename TIn, int D>
__global__ __launch_bounds__(64) void tree_attn_fma(const AttnKernelArgs a) {
  constexpr int DPL = D / 64;   // output columns per lane
  __shared__ float q_lds[D];
  __shared__ float p_lds[kTileKeys];
  __shared__ int32_t par_lds[kMaxTree];

  const int lane = threadIdx.x;
  const int logical = blockIdx.x;
  const int R = a.R;
  const int r = logical % R;
  const int split = (logical / R) % a.total_splits;
  const int hk = logical / (R * a.total_splits);
  const int b = find_seq(a, split);
  const int s_local = split - a.split_base[b];
  const int S = a.split_base[b + 1] - a.split_base[b];
  const int L = a.L[b];
  const int T = a.T, g = a.g, Hq = a.Hq, Hkv = a.Hkv;
  const int nodei = r / g, head = hk * g + r % g;

  const uint32_t bad = validate_seq(a, b, lane, par_lds);
  if (s_local == 0 && hk == 0 && r == 0 && lane == 0) a.flags[b] = bad;
  if (bad) {
    if (S == 1) {
      float* o = a.out + ((int64_t)(b * T + nodei) * Hq + head) * D;
      for (int e = 0; e < DPL; ++e) o[lane + 64 * e] = __builtin_nanf("");
    }
    return;
  }
  __syncthreads();
  const uint64_t anc = ancestors_of(par_lds, nodei);
  const TIn* qp = reinterpret_cast<const TIn*>(a.q) + ((int64_t)(b * T + nodei) * Hq + head) * D;
  for (int e = 0; e < DPL; ++e) q_lds[lane + 64 * e] = load_elem<TIn>(qp, lane + 64 * e);
  __syncthreads();

  const TIn* kb = reinterpret_cast<const TIn*>(a.k);
  const TIn* vb = reinterpret_cast<const TIn*>(a.v);
  const bool paged = a.page_size != 0;
  const int64_t kv0 = paged ? 0 : a.kv_indptr[b];
  __shared__ int64_t prow[kTileKeys];   // physical rows of the tile's keys (paged K/V)
  const int k_begin = s_local * a.chunk;
  const int k_end = min(k_begin + a.chunk, L);
  const int n_prefix_tiles = k_end > k_begin ? (k_end - k_begin + kTileKeys - 1) / kTileKeys : 0;
  const int n_tiles = n_prefix_tiles + ((s_local == S - 1) ? 1 : 0);
  const float c = a.scale_log2;

  float acc[DPL];
  for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
  float m_run = kNegInf, l_run = 0.f;
  for (int t = 0; t < n_tiles; ++t) {
    const bool is_tree = t >= n_prefix_tiles;
    const int start = is_tree ? L : k_begin + t * kTileKeys;
    const int cnt = is_tree ? T : min(kTileKeys, k_end - start);
    const int64_t row0 = kv0 + start;
    __syncthreads();   // the previous tile's rows are no longer read
    if (lane < kTileKeys) prow[lane] = paged ? paged_row(a, b, start + min(lane, cnt - 1)) : row0 + lane;
    __syncthreads();
    float s = kNegInf;
    const bool valid = lane < cnt && (!is_tree || ((anc >> lane) & 1ull));
    if (valid) {
      const TIn* kr = kb + (prow[lane] * Hkv + hk) * D;
      float dot = 0.f;
      for (int d = 0; d < D; ++d) dot = __builtin_fmaf(q_lds[d], load_elem<TIn>(kr, d), dot);
      s = dot;
    }
    float tmax = s;
    for (int o = 32; o > 0; o >>= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, o));
    const float m_new = fmaxf(m_run, tmax * c);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    const float p = exp2f(__builtin_fmaf(s, c, -m_use));
    float psum = p;
    for (int o = 32; o > 0; o >>= 1) psum += __shfl_xor(psum, o);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    __syncthreads();
    p_lds[lane] = p;
    __syncthreads();
    for (int e = 0; e < DPL; ++e) {
      float sum = 0.f;
      for (int k = 0; k < cnt; ++k) sum = __builtin_fmaf(p_lds[k], load_elem<TIn>(vb, (prow[k] * Hkv + hk) * D + lane + 64 * e), sum);
      acc[e] = acc[e] * alpha + sum;
    }
  }
  if (S == 1) {
    float* o = a.out + ((int64_t)(b * T + nodei) * Hq + head) * D;
    const float inv = 1.f / l_run;
    for (int e = 0; e < DPL; ++e) o[lane + 64 * e] = acc[e] * inv;
  } else {
    const int64_t prow = (int64_t)logical;   // one row per slot
    for (int e = 0; e < DPL; ++e) a.opart[prow * D + lane + 64 * e] = acc[e];
    if (lane == 0) {
      a.mlpart[2 * prow] = m_run;
      a.mlpart[2 * prow + 1] = l_run;
    }
  }
}

// ------------------------------------------------------------ LSE merge
// out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s, M = max_s m_s.
// SPL adjacent lanes share one (query row, 4 output columns): lane sl folds
// the splits sl, sl + SPL, ... in rounds of up to 8 whose loads are all
// issued before any is used, then the SPL partial states are combined by
// log-sum-exp over lane shuffles.  SPL is chosen from the largest split
// count so that a lane needs at most two rounds.  A block covers
// 256 / (SPL * D/4) query rows of one (sequence, KV head).  A sequence the
// split kernel found invalid (its flags word, written by that kernel) gets
// NaN rows.
constexpr int kMergeRound = 8;   // splits folded per lane per load round

template <int D, int SPL>
__global__ __launch_bounds__(256) void tree_attn_merge(const AttnKernelArgs a) {
  constexpr int CG = D / 4;                  // column groups per row
  constexpr int RPB = 256 / (CG * SPL);      // rows per block
  const int R = a.R;
  const int nrb = (R + RPB - 1) / RPB;
  const int hk = (blockIdx.x / nrb) % a.Hkv;
  const int b = blockIdx.x / (nrb * a.Hkv);
  const int base = a.split_base[b];
  const int S = a.split_base[b + 1] - base;
  if (S <= 1) return;
  const int tid = threadIdx.x;
  const int sl = tid % SPL;
  const int cg = (tid / SPL) % CG;
  const int r = (blockIdx.x % nrb) * RPB + tid / (SPL * CG);
  const bool live = r < R;                   // whole groups of SPL lanes agree
  const int rr = live ? r : R - 1;
  const int T = a.T, g = a.g, Hq = a.Hq, rpt = a.rows_per_tile;
  const int rt = rr / rpt, rl = rr % rpt;
  const int64_t stride = (int64_t)a.row_tiles * rpt;    // partial rows between splits
  const int64_t prow0 = ((int64_t)hk * a.total_splits + base) * stride + (int64_t)rt * rpt + rl;
  float M = kNegInf, den = 0.f;
  f32x4_t num = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int s0 = sl; s0 < S; s0 += SPL * kMergeRound) {
    float m[kMergeRound], l[kMergeRound];
    f32x4_t o[kMergeRound];
#pragma unroll
    for (int j = 0; j < kMergeRound; ++j) {
      const int sj = s0 + j * SPL;
      m[j] = kNegInf;
      l[j] = 0.f;
      o[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (sj < S) {
        const int64_t prow = prow0 + (int64_t)sj * stride;
        m[j] = a.mlpart[2 * prow];
        l[j] = a.mlpart[2 * prow + 1];
        o[j] = *reinterpret_cast<const f32x4_t*>(a.opart + prow * D + 4 * cg);
      }
    }
    float Mn = M;
#pragma unroll
    for (int j = 0; j < kMergeRound; ++j) Mn = fmaxf(Mn, m[j]);
    const float Mu = (Mn == kNegInf) ? 0.f : Mn;
    const float sc = __builtin_amdgcn_exp2f(M - Mu);
    den *= sc;
    num *= sc;
#pragma unroll
    for (int j = 0; j < kMergeRound; ++j) {
      const float w = __builtin_amdgcn_exp2f(m[j] - Mu);
      den += w * l[j];
      num += w * o[j];
    }
    M = Mn;
  }
  // combine the SPL lanes' states
#pragma unroll
  for (int x = 1; x < SPL; x <<= 1) {
    const float Mo = __shfl_xor(M, x);
    const float Do = __shfl_xor(den, x);
    f32x4_t No;
#pragma unroll
    for (int i = 0; i < 4; ++i) No[i] = __shfl_xor(num[i], x);
    const float Mn = fmaxf(M, Mo);
    const float Mu = (Mn == kNegInf) ? 0.f : Mn;
    const float ws = __builtin_amdgcn_exp2f(M - Mu), wo = __builtin_amdgcn_exp2f(Mo - Mu);
    den = den * ws + Do * wo;
    num = num * ws + No * wo;
    M = Mn;
  }
  if (!live || sl != 0) return;
  const uint32_t bad = a.flags[b];
  const float nan = __builtin_nanf("");
  float* op = a.out + ((int64_t)(b * T + r / g) * Hq + hk * g + r % g) * D + 4 * cg;
  *reinterpret_cast<f32x4_t*>(op) = bad ? f32x4_t{nan, nan, nan, nan} : num * (1.f / den);
}

template <int D, int SPL>
hipError_t launch_merge(const AttnKernelArgs& a, hipStream_t st) {
  const unsigned rpb = 256 / ((D / 4) * SPL);
  const unsigned nrb = (unsigned)((a.R + rpb - 1) / rpb);
  hipLaunchKernelGGL((tree_attn_merge<D, SPL>), dim3((unsigned)(a.B * a.Hkv) * nrb), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnPlan& p, const AttnKernelArgs& a, int kv_bf16, hipStream_t st) {
  if (p.path == 1) {
    const dim3 grid((unsigned)p.workgroups), block(256);
    const int v = mfma_variant(p);
    const void* fn = nullptr;
    if (a.page_size) {
      switch (v) {
        case 0: fn = reinterpret_cast<const void*>(&tree_attn_mfma<D, 1, 2, 1, true>); break;
        case 1: fn = reinterpret_cast<const void*>(&tree_attn_mfma<D, 2, 2, 1, true>); break;
        case 2: fn = reinterpret_cast<const void*>(&tree_attn_mfma<D, 1, 2, 2, true>); break;
        default: return hipErrorInvalidValue;
      }
    } else {
      switch (v) {
        case 0: fn = reinterpret_cast<const void*>(&tree_attn_mfma<D, 1, 2, 1>); break;
        case 1: fn = reinterpret_cast<const void*>(&tree_attn_mfma<D, 2, 2, 1>); break;
        case 2: fn = reinterpret_cast<const void*>(&tree_attn_mfma<D, 1, 2, 2>); break;
        default: return hipErrorInvalidValue;
      }
    }
    // with the merge inside, the splits wait for each other: a cooperative
    // launch makes every workgroup resident at once or is refused
    // (hipErrorCooperativeLaunchTooLarge, nothing enqueued; the caller then
    // runs the separate merge kernel)
    void* args[] = {const_cast<AttnKernelArgs*>(&a)};
    const hipError_t e = (a.fused_merge && a.coop) ? hipLaunchCooperativeKernel(fn, grid, block, args, 0, st)
                                                   : hipLaunchKernel(fn, grid, block, args, 0, st);
    if (e != hipSuccess) return e;
  } else {
    const dim3 grid((unsigned)p.workgroups), block(64);
    if (kv_bf16)
      hipLaunchKernelGGL((tree_attn_fma<uint16_t, D>), grid, block, 0, st, a);
    else
      hipLaunchKernelGGL((tree_attn_fma<float, D>), grid, block, 0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.merge_workgroups > 0 && !a.fused_merge) {
    int smax = 1;
    for (int b = 0; b < a.B; ++b) smax = std::max(smax, a.split_base[b + 1] - a.split_base[b]);
    // up to two load rounds per lane before lanes are added (measured best)
    if (smax <= 2 * kMergeRound)
      e = launch_merge<D, 1>(a, st);
    else if (smax <= 4 * kMergeRound)
      e = launch_merge<D, 2>(a, st);
    else if (smax <= 8 * kMergeRound)
      e = launch_merge<D, 4>(a, st);
    else
      e = launch_merge<D, 8>(a, st);
  }
  return e;
}

}  // namespace

int attention_capacity(int D, int variant, int num_cus) {
  int per_cu = 0;
  const void* fns128[kMfmaVariants] = {reinterpret_cast<const void*>(&tree_attn_mfma<128, 1, 2, 1>),
                                       reinterpret_cast<const void*>(&tree_attn_mfma<128, 2, 2, 1>),
                                       reinterpret_cast<const void*>(&tree_attn_mfma<128, 1, 2, 2>)};
  const void* fns64[kMfmaVariants] = {reinterpret_cast<const void*>(&tree_attn_mfma<64, 1, 2, 1>),
                                      reinterpret_cast<const void*>(&tree_attn_mfma<64, 2, 2, 1>),
                                      reinterpret_cast<const void*>(&tree_attn_mfma<64, 1, 2, 2>)};
  if (variant < 0 || variant >= kMfmaVariants) return 0;
  const void* fn = (D == 128) ? fns128[variant] : fns64[variant];
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, 0) != hipSuccess || per_cu <= 0) return 0;
  return per_cu * num_cus;
}

int launch_tree_attention(const AttnPlan& plan, const AttnKernelArgs& args, int kv_bf16, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = (args.D == 128) ? launch_d<128>(plan, args, kv_bf16, st) : launch_d<64>(plan, args, kv_bf16, st);
  return static_cast<int>(e);
}

}  // namespace ev
