// Internal definitions shared by the host library and the HIP kernels of
// libeagle_verify: launch plans, kernel argument blocks and the workspace
// layout.  Nothing here is part of the public C ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/eagle_verify.h"

namespace ev {

constexpr int kMaxBatch = 256;       // per-sequence plan travels in the kernel arguments
constexpr int kMaxTree = EAGLE_MAX_TREE_ROWS;
constexpr int kTileKeys = 64;        // keys per attention tile (one LDS stage)
constexpr int kStampSlots = 32;      // timeline words per workgroup (diagnostic)
constexpr int kVocabChunk = 8192;    // vocabulary elements per acceptance workgroup
constexpr int kNodeVocab = 32768;    // largest vocabulary of the node-parallel acceptance (one workgroup per node)
constexpr int kDefaultCUs = 256;     // MI355X compute units (planning without a device)
constexpr int64_t kAttnPartFloats = 32ll << 20;   // 128 MiB of split partials
// (row, split) pairs whose merge weights fit in the smallest (D = 64) MFMA
// K/V ring next to the 4 KB of lane partials: 2 floats per pair
constexpr int kFusedMergePairs = (2 * 2 * 64 * 64 * 2 - 4096) / 8;
constexpr int kRoundWords = kMaxTree;   // residual-mass rounds a node can need (< its children)

// ---------------------------------------------------------------- attention
struct AttnPlan {
  int path;            // 0 = FMA kernel (fp32, or bf16 with R < 16), 1 = MFMA kernel
  int R;               // rows per KV head = T * g
  int mb;              // MFMA: 16-row blocks per wave (rows per workgroup = 64 * mb), 1 or 2
  int stages;          // MFMA: K/V tiles in the LDS ring
  int kg;              // MFMA: key groups per tile (2: wave pairs take the two 32-key halves)
  int late_priority;   // MFMA: the later half of the grid runs at a raised wave priority
  int row_tiles;       // workgroups along R (FMA path: one row each)
  int rows_per_tile;
  int chunk;           // prefix keys per split (multiple of kTileKeys)
  int total_splits;
  int64_t workgroups;
  int64_t merge_workgroups;
  int64_t part_floats; // workspace floats used by split partials
  int32_t splits[kMaxBatch];
  int32_t split_base[kMaxBatch + 1];
};

struct AttnKernelArgs {
  const void* q;
  const void* k;
  const void* v;
  const int64_t* kv_indptr;
  const int32_t* parents;
  float* out;
  uint32_t* flags;
  float* opart;        // [slot][rows_per_tile][D]
  float* mlpart;       // [slot][rows_per_tile][2]  (m in log2 units, l)
  int64_t num_kv_rows;
  int B, T, Hq, Hkv, g, D, R;
  int row_tiles, rows_per_tile, chunk, total_splits;
  int nwg;
  float scale_log2;    // sm_scale * log2(e)
  // in-kernel merge (MFMA path, every workgroup co-resident): each split of a
  // (sequence, KV head, row tile) merges a slice of its rows once every
  // split has published the tagged m/l words of those rows
  int fused_merge;
  int coop;            // host side: launch the merge-inside kernel cooperatively
  int late_priority;   // raise the wave priority of the later half of the grid
  uint32_t spin_limit; // polls of the bounded wait; an expired wait flags EAGLE_FLAG_INTERNAL
  uint64_t epoch;      // strictly increasing per attention call on a handle (tags use its low 32 bits)
  uint64_t* mlrec;      // [slot][rows_per_tile][2]: m and l (low 32 bits), epoch tag (high 32 bits)
  uint64_t* stamps;     // phase timeline [workgroup][kStampSlots] (diagnostic), or NULL
  // paged K/V (page_size > 0): logical row x of sequence b is physical row
  // page_table[b * pps + x / page_size] * page_size + x % page_size
  const int32_t* page_table;
  int page_size, pps;
  int64_t num_pages;
  int32_t L[kMaxBatch];
  int32_t split_base[kMaxBatch + 1];
  // expected kv_indptr[b] (rows packed back to back, L_b + T per sequence),
  // -1 when it does not fit 31 bits or the array: the MFMA kernel requests
  // its first tile from there before kv_indptr[b] arrives, and fetches the
  // tile again if the guess was wrong
  int32_t kv0_guess[kMaxBatch];
};

// ---------------------------------------------------------------- acceptance
struct ChunkStat {     // one (sequence, node, row, vocab chunk)
  float m;             // chunk max of the raw logits (-inf if all -inf)
  uint32_t bad;        // 1 = NaN or +inf seen
  int32_t argmax;      // lowest id holding the chunk max (greedy mode)
  int32_t pad;
  double z;            // sum exp((x - m) / tau) over the chunk
};

enum NodeKind : int32_t { kNodeLeaf = 0, kNodeAccepted = 1, kNodeRejected = 2, kNodeNeedsPass = 3 };

struct NodeState {     // one (sequence, node)
  double zq, zp;       // softmax normalisers of target / draft rows
  double C, s;         // residual = max(0, q - C p) / s after the tested children
  float mq, mp;        // row maxima of target / draft logits
  int32_t kind;        // NodeKind
  int32_t outcome;     // accepted child (kNodeAccepted), else -1
  int32_t next_child;  // kNodeNeedsPass: ordinal of the next child to test
  int32_t argmax;      // greedy mode: target argmax
  uint32_t flags;      // NONFINITE for unusable rows, P_ZERO / DEGENERATE events
  int32_t near;        // near-threshold decisions taken at this node
};

struct AcceptKernelArgs {
  const void* target;
  const void* draft;
  const int32_t* parents;
  const int32_t* tokens;
  int32_t* accept_len;
  int32_t* accepted_nodes;
  int32_t* out_tokens;
  uint32_t* flags;
  int32_t* near_ties;
  ChunkStat* stats;    // [B][T][2][NC]
  NodeState* nodes;    // [B][T]
  double* fpart;       // [B][T][NC]
  double* spart;       // fused: [B][T][NC][4] tagged words (chunk masses); three-kernel path: [B][NC]
  uint32_t* cnt_stats; // [B][T]
  uint32_t* cnt_pass;  // [B][T]
  uint32_t* cnt_final; // [B]
  // fused path
  uint64_t* node_pub;     // [Bm][Tm] publication words, contiguous (one poll covers a sequence)
  uint64_t* round_sum;    // [Bm][Tm][kRoundWords]: (count << 57) | fixed-point residual mass
  uint64_t* round_clear;  // the other half, used by the previous fused call; cleared here
  int Tm;                 // node stride of node_pub and round_sum (max_tree_rows)
  int zero_b;             // batch of the previous fused call (extent of round_clear to clear)
  uint64_t epoch;         // strictly increasing per call on a handle
  uint32_t spin_limit;    // bounded waits: a wait that exceeds it flags the sequence
  uint64_t* stamps;       // fused path: phase timeline [workgroup][kStampSlots] (diagnostic), or NULL
  int node_priority;      // fused path: internal nodes' waves at a raised priority
  int leaf_wait;          // fused path, sampled, whole 16-byte groups, siblings with replacement:
                          // s_sleep(10) steps a leaf waits before requesting its rows (0: none)
  int fused;              // 2: node-parallel kernels; 1: one co-resident kernel; 0: three-kernel path
  int coop;               // host side: launch the fused kernel cooperatively
  int b0;                 // batch index of sequence 0 of this launch (a slice of the call's batch)
  int wr;                 // 1: siblings were drawn without replacement
  // three-kernel path with wr: per node, the residual weight each tried
  // sibling's token keeps ([B][T][kMaxTree], -1 for a repeated token) and, in
  // the last slot, the draft mass not yet tried
  double* wr_kept;
  int B, T, V, NC;
  int vec_ok;          // rows start 16-byte aligned
  // filtered distributions: logits below thr[(b * T + n) * 2 + r] count as
  // -inf (r = 0 target, 1 draft row of node n); NULL: no filter
  const float* thr;
  const int32_t* thr_near;   // per row: 1 adds a near tie to the node's decisions
  float tau;           // > 0 sampled, == 0 greedy
  float c2;            // log2(e) / tau
  double inv_tau;
  uint32_t seed_lo, seed_hi, off_lo, off_hi;
};

// Keep-thresholds of filtered (top-k / top-p) distributions, one per row:
// thr[(b * T + n) * 2 + r] (r = 0 target, 1 draft); -inf keeps every token.
struct FilterKernelArgs {
  const void* target;
  const void* draft;
  const int32_t* parents;
  const int32_t* tokens;
  float* thr;
  int32_t* near;       // 1: the row's top-p boundary lies within 1e-6 of its mass target
  int B, T, V;
  int top_k;           // 0: off
  float top_p;         // 0 or 1: off
  float c2;            // log2(e) / tau
};

// ---------------------------------------------------------------- KV commit
struct CommitKernelArgs {
  void* k;
  void* v;
  const int64_t* kv_indptr;
  const int32_t* accept_len;
  const int32_t* accepted_nodes;
  int32_t* new_lens;
  uint32_t* flags;
  int64_t num_kv_rows;
  int64_t layer_stride;   // elements between consecutive layers' k (and v)
  const int32_t* page_table;   // paged K/V (page_size > 0), as for attention
  int page_size, pps;
  int64_t num_pages;
  int B, T, Hkv, D, layers;
  int head_groups;     // workgroups per (layer, sequence): each moves the rows of Hkv / head_groups heads
  int32_t L[kMaxBatch];
};

// ---------------------------------------------------------------- tree expansion
constexpr int kMaxTopK = 16;          // children per frontier node
constexpr int kMaxKeep = 64;          // candidates kept per sequence
constexpr int kMaxChunksExpand = 64;  // vocabulary chunks of one row (V <= 64 * 8192)
// tokens per expansion chunk: the smallest of 2048, 4096, 8192 that keeps a
// row within kMaxChunksExpand chunks
inline int expand_chunk(int V) { return V <= 64 * 2048 ? 2048 : (V <= 64 * 4096 ? 4096 : 8192); }
inline int expand_chunks(int V) { return (V + expand_chunk(V) - 1) / expand_chunk(V); }

struct ChunkRecord {   // one (sequence, frontier row, vocab chunk)
  float m;             // chunk maximum (-inf if none finite)
  uint32_t bad;        // NaN or +inf seen
  double z;            // sum exp((x - m) / t)
  float val[kMaxTopK]; // the chunk's largest logits, descending (ties: lower id first)
  int32_t id[kMaxTopK];// their token ids, -1 past the last
};


struct ExpandKernelArgs {
  const void* logits;  // [B][F][V]
  const float* scores; // [B][F]
  ChunkRecord* chunks; // [B][F][NC]
  int32_t* parent;     // [B][M]
  int32_t* token;      // [B][M]
  float* value;        // [B][M]
  uint32_t* flags;     // [B]
  int32_t* near_ties;  // [B]
  int B, F, V, NC, K, M;
  int chunk;           // vocabulary tokens per chunk (2048, 4096 or 8192)
  float c2;            // log2(e) / t
  double inv_tau;      // 1 / t
  uint64_t* stamps;    // diagnostic timeline (32 words per chunk workgroup, then per sequence), or NULL
};

constexpr int kMaxSteps = 64;         // chained expansion steps one rerank reads

struct RerankKernelArgs {
  const int32_t* parent;     // [D][B][M]
  const int32_t* token;      // [D][B][M]
  const float* value;        // [D][B][M]
  const int32_t* root_tokens;// [B]
  int32_t* parents;          // [B][N + 1]
  int32_t* tokens;           // [B][N + 1]
  int32_t* rows;             // [B]
  int B, D, M, N;
};

// ---------------------------------------------------------------- host side
struct Workspace {
  uint64_t* node_pub = nullptr;
  uint64_t* round_sum = nullptr;
  float* attn_part = nullptr;   // kAttnPartFloats
  ChunkStat* stats = nullptr;
  NodeState* nodes = nullptr;
  double* fpart = nullptr;
  double* spart = nullptr;
  uint32_t* counters = nullptr; // cnt_stats | cnt_pass | cnt_final
  ChunkRecord* expand = nullptr; // [max_batch][max_tree_rows][expansion chunks of a row]
  double* wr_kept = nullptr;     // [max_batch][max_tree_rows][kMaxTree] (three-kernel path, without replacement)
  float* thr = nullptr;          // [max_batch][max_tree_rows][2] keep-thresholds of filtered rows
  int32_t* thr_near = nullptr;   // [max_batch][max_tree_rows][2]
  size_t bytes = 0;
};

// Acceptance scratch of one layout: statistics, node states, round
// partials, chunk masses, counters, publication and round words for Bm
// sequences of Tm rows and NC vocabulary chunks, placed from byte offset
// `off` of a 256-byte-aligned base.  Fills the acceptance fields of *ws
// (when base is not NULL) and returns the end offset.
size_t accept_layout(int64_t Bm, int64_t Tm, int NC, size_t off, char* base, Workspace* ws);

// Per-call state of the acceptance launches that outlives one launch: epochs
// tag cross-workgroup words, and the two halves of the round words alternate
// between fused launches (each clears the half the previous one used).
struct AcceptCallState {
  uint64_t epoch = 0;
  uint64_t fused_calls = 0;
  int last_fused_b = 0;
  int last_paths = 0;   // EAGLE_ACCEPT_PATH_* bits of the last successful call (0: none yet)
};

// One spec_accept call on workspace `ws` laid out for Bm x Tm (arguments
// already checked against the descriptor); fused_cap = co-resident
// fused-acceptance workgroups.  Messages go to err.
eagle_status run_spec_accept(const eagle_verify_desc& desc, const Workspace& ws, int64_t Bm, int64_t Tm,
                             int64_t fused_cap, AcceptCallState* cs, const eagle_spec_accept_args* a,
                             void* stream, char* err, size_t errlen, uint32_t spin_limit, bool coop,
                             uint64_t* stamps = nullptr, int64_t stamp_words = 0);

// Polls of a bounded device-side wait (each about a microsecond): past it the
// wait gives up and flags the sequence EAGLE_FLAG_INTERNAL.  The environment
// variable EAGLE_VERIFY_SPIN_LIMIT lowers it (tests of the give-up path).
constexpr uint32_t kSpinLimit = 1u << 16;
uint32_t spin_limit_from_env();
// cooperative launches of the kernels whose workgroups wait for each other:
// EAGLE_VERIFY_COOPERATIVE=1 (read when a handle is created) guarantees that
// every workgroup is resident (a refused launch falls back to the paths that
// do not wait), at a cost of about 16 us per launch
bool cooperative_from_env();

// thread-local message returned by eagle_verify_last_error(NULL)
void set_thread_error(const char* msg);

// plan.cpp (pure C++, no HIP)
eagle_status check_desc(const eagle_verify_desc* d, char* err, size_t errlen);
eagle_status plan_tree_attention(const eagle_verify_desc* d, const eagle_tree_attention_args* a,
                                 int num_cus, AttnPlan* plan, char* err, size_t errlen);
eagle_status check_spec_accept(const eagle_verify_desc* d, const eagle_spec_accept_args* a,
                               char* err, size_t errlen);
eagle_status check_kv_commit(const eagle_verify_desc* d, const eagle_kv_commit_args* a, char* err, size_t errlen);
eagle_status check_tree_expand(const eagle_verify_desc* d, const eagle_tree_expand_args* a, char* err,
                               size_t errlen);
eagle_status check_tree_rerank(const eagle_verify_desc* d, const eagle_tree_rerank_args* a, char* err,
                               size_t errlen);
int vocab_chunks(int V);

// attention.hip / accept.hip
int launch_tree_attention(const AttnPlan& plan, const AttnKernelArgs& args, int kv_bf16,
                          void* stream);
int launch_spec_accept(const AcceptKernelArgs& args, int logits_bf16, void* stream);
int launch_filter(const FilterKernelArgs& args, int logits_bf16, void* stream);        // filter.hip
int launch_kv_commit(const CommitKernelArgs& args, int kv_bf16, void* stream);   // commit.hip
int launch_tree_expand(const ExpandKernelArgs& args, int logits_bf16, void* stream);   // expand.hip
int launch_tree_rerank(const RerankKernelArgs& args, void* stream);                    // expand.hip
// workgroups of the fused acceptance kernel that can be co-resident on the
// device (0 if the query fails); the fused path is used when B*T*NC fits
int fused_accept_capacity(int logits_bf16, int num_cus);
// co-resident workgroups of the MFMA attention kernel for head_dim D and mb
// 16-row blocks per wave (0 if the query fails)
// MFMA kernel variants: 0 = one 16-row block per wave, 1 = two, 2 = key halves
// split between wave pairs (32 rows per workgroup)
constexpr int kMfmaVariants = 3;
inline int mfma_variant(const AttnPlan& p) { return p.kg == 2 ? 2 : p.mb - 1; }
int attention_capacity(int D, int variant, int num_cus);

}  // namespace ev
