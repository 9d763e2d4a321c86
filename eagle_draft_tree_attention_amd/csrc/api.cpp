// libeagle_verify: the exported C ABI (see include/eagle_verify.h).
// Handle lifetime, workspace, argument marshalling into kernel argument
// blocks, and launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>

#include "ev_internal.h"

struct eagle_verify {
  eagle_verify_desc desc;
  int device = 0;
  int num_cus = ev::kDefaultCUs;
  ev::Workspace ws;
  void* base = nullptr;
  hipStream_t last_stream = nullptr;
  bool used = false;
  ev::AcceptCallState accept_state;   // acceptance epochs and round-word halves
  uint64_t attn_epoch = 0;     // attention calls issued on this handle
  eagle_attention_plan last_plan{};         // of the last successful tree_attention call
  bool have_plan = false;
  int attn_cap[2][ev::kMfmaVariants] = {};   // co-resident MFMA attention workgroups [D == 128][kernel variant]
  int fused_cap[2] = {0, 0};   // co-resident fused-acceptance workgroups (f32, bf16)
  uint32_t spin_limit = ev::kSpinLimit;   // polls of a bounded device-side wait
  bool coop = false;           // cooperative launches of the self-synchronising kernels (opt-in)
  uint64_t* stamps = nullptr;  // diagnostic phase timeline (caller's device words), or NULL
  int64_t stamp_words = 0;
  char err[512] = {0};
};

namespace {

thread_local char g_err[512];

void set_err(eagle_verify* h, const char* msg) {
  char* dst = h ? h->err : g_err;
  std::snprintf(dst, 512, "%s", msg);
}

eagle_status hip_fail_to(char* dst, size_t len, const char* what, int code) {
  std::snprintf(dst, len, "%s failed: %s (%d)", what, hipGetErrorString(static_cast<hipError_t>(code)), code);
  return EAGLE_ERR_HIP;
}

eagle_status hip_fail(eagle_verify* h, const char* what, int code) {
  return hip_fail_to(h ? h->err : g_err, 512, what, code);
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

void public_plan(const ev::AttnPlan& p, eagle_attention_plan* plan) {
  plan->path = p.path;
  plan->rows_per_kv_head = p.R;
  plan->row_tiles = p.row_tiles;
  plan->rows_per_tile = p.rows_per_tile;
  plan->chunk_keys = p.chunk;
  plan->total_splits = p.total_splits;
  plan->workgroups = static_cast<int32_t>(p.workgroups);
  plan->merge_workgroups = static_cast<int32_t>(p.merge_workgroups);
  plan->merge_in_kernel = 0;
}

}  // namespace

namespace ev {

size_t accept_layout(int64_t Bm, int64_t Tm, int NC, size_t off, char* base, Workspace* ws) {
  const size_t o_stats = off;
  // per (sequence, node, row, chunk): a ChunkStat (three-kernel path) or four
  // tagged 64-bit words (fused path)
  off = align_up(off + std::max(sizeof(ChunkStat), 4 * sizeof(uint64_t)) * Bm * Tm * 2 * NC, 256);
  const size_t o_nodes = off;
  off = align_up(off + sizeof(NodeState) * Bm * Tm, 256);
  const size_t o_fpart = off;
  off = align_up(off + sizeof(double) * 2 * Bm * Tm * NC, 256);   // two round buffers
  const size_t o_spart = off;
  off = align_up(off + sizeof(uint64_t) * 4 * Bm * Tm * NC, 256);   // fused: four tagged words per chunk
  const size_t o_cnt = off;
  off = align_up(off + sizeof(uint32_t) * (2 * Bm * Tm + Bm), 256);
  const size_t o_sync = off;   // one publication word per node, contiguous per sequence
  off = align_up(off + sizeof(uint64_t) * Bm * Tm, 256);
  const size_t o_round = off;
  off = align_up(off + sizeof(uint64_t) * 2 * Bm * Tm * kRoundWords, 256);
  const size_t o_wr = off;
  off = align_up(off + sizeof(double) * Bm * Tm * kMaxTree, 256);
  const size_t o_thr = off;
  off = align_up(off + sizeof(float) * 2 * Bm * Tm, 256);
  const size_t o_thr_near = off;
  off = align_up(off + sizeof(int32_t) * 2 * Bm * Tm, 256);
  if (base && ws) {
    ws->stats = reinterpret_cast<ChunkStat*>(base + o_stats);
    ws->nodes = reinterpret_cast<NodeState*>(base + o_nodes);
    ws->fpart = reinterpret_cast<double*>(base + o_fpart);
    ws->spart = reinterpret_cast<double*>(base + o_spart);
    ws->counters = reinterpret_cast<uint32_t*>(base + o_cnt);
    ws->node_pub = reinterpret_cast<uint64_t*>(base + o_sync);
    ws->round_sum = reinterpret_cast<uint64_t*>(base + o_round);
    ws->wr_kept = reinterpret_cast<double*>(base + o_wr);
    ws->thr = reinterpret_cast<float*>(base + o_thr);
    ws->thr_near = reinterpret_cast<int32_t*>(base + o_thr_near);
  }
  return off;
}

void set_thread_error(const char* msg) { std::snprintf(g_err, sizeof(g_err), "%s", msg); }

bool cooperative_from_env() {
  // opt-in: a cooperative launch costs about 16 us more per launch on this
  // stack (measured: the 8B verification step 55.7 -> 91.5 us), so by default
  // residency rests on the occupancy check and the bounded waits
  const char* s = std::getenv("EAGLE_VERIFY_COOPERATIVE");
  return s && s[0] == '1';
}

uint32_t spin_limit_from_env() {
  // a test knob: the polls a bounded device-side wait makes before it gives up
  const char* s = std::getenv("EAGLE_VERIFY_SPIN_LIMIT");
  if (!s || !*s) return kSpinLimit;
  const long v = std::strtol(s, nullptr, 10);
  return v < 0 ? kSpinLimit : static_cast<uint32_t>(std::min<long>(v, kSpinLimit));
}

eagle_status run_spec_accept(const eagle_verify_desc& desc, const Workspace& ws, int64_t Bm, int64_t Tm,
                             int64_t cap, AcceptCallState* cs, const eagle_spec_accept_args* a, void* hip_stream,
                             char* err, size_t errlen, uint32_t spin_limit, bool coop, uint64_t* stamps,
                             int64_t stamp_words) {
  AcceptKernelArgs k;
  std::memset(&k, 0, sizeof(k));
  const int V = desc.vocab_size;
  const int bf16 = desc.logits_dtype == EAGLE_BF16 ? 1 : 0;
  const int esize = bf16 ? 2 : 4;
  k.target = a->target_logits;
  k.draft = a->draft_logits ? a->draft_logits : a->target_logits;
  k.parents = a->parents;
  k.tokens = a->tokens;
  k.accept_len = a->accept_len;
  k.accepted_nodes = a->accepted_nodes;
  k.out_tokens = a->out_tokens;
  k.flags = a->flags;
  k.near_ties = a->near_ties;
  k.stats = ws.stats;
  k.nodes = ws.nodes;
  k.fpart = ws.fpart;
  k.spart = ws.spart;
  k.cnt_stats = ws.counters;
  k.cnt_pass = ws.counters + Bm * Tm;
  k.cnt_final = ws.counters + 2 * Bm * Tm;
  k.B = a->batch;
  k.T = a->tree_rows;
  k.V = V;
  k.NC = vocab_chunks(V);
  k.vec_ok = ((static_cast<int64_t>(V) * esize) % 16) == 0 ? 1 : 0;
  k.tau = a->temperature;
  k.c2 = a->temperature > 0.f ? static_cast<float>(1.4426950408889634 / a->temperature) : 0.f;
  k.inv_tau = a->temperature > 0.f ? 1.0 / static_cast<double>(a->temperature) : 0.0;
  k.seed_lo = static_cast<uint32_t>(a->seed);
  k.seed_hi = static_cast<uint32_t>(a->seed >> 32);
  k.off_lo = static_cast<uint32_t>(a->offset);
  k.off_hi = static_cast<uint32_t>(a->offset >> 32);
  k.node_pub = ws.node_pub;
  k.Tm = static_cast<int>(Tm);
  k.epoch = ++cs->epoch;
  k.spin_limit = spin_limit;
  {   // tuning override: EAGLE_VERIFY_NODE_PRIORITY = 0 keeps every wave at the normal priority
    const char* np = std::getenv("EAGLE_VERIFY_NODE_PRIORITY");
    k.node_priority = (np && np[0] == '0') ? 0 : 1;
  }
  // The fused kernel needs every workgroup of a launch resident at once.  A
  // batch that does not fit is verified in slices of whole sequences, one
  // fused launch each, back to back on the stream (each slice is a fused
  // call of its own: its own epoch and round-word half); the uniforms keep
  // the sequence's index in the whole batch.  Only a single sequence that
  // does not fit takes the three-kernel path.
  // filtered distributions: one keep-threshold per row first (sampled mode only)
  if (a->temperature > 0.f && (a->top_k > 0 || (a->top_p > 0.f && a->top_p < 1.f))) {
    FilterKernelArgs f;
    std::memset(&f, 0, sizeof(f));
    f.target = k.target;
    f.draft = k.draft;
    f.parents = a->parents;
    f.tokens = a->tokens;
    f.thr = ws.thr;
    f.near = ws.thr_near;
    f.B = a->batch;
    f.T = a->tree_rows;
    f.V = V;
    f.top_k = a->top_k;
    f.top_p = a->top_p;
    f.c2 = k.c2;
    const int e = launch_filter(f, bf16, hip_stream);
    if (e != 0) return hip_fail_to(err, errlen, "filter launch", e);
    k.thr = ws.thr;
    k.thr_near = ws.thr_near;
  }
  const int64_t per_seq = static_cast<int64_t>(k.T) * k.NC;
  k.wr = (a->without_replacement && a->temperature > 0.f) ? 1 : 0;
  // Small vocabularies: one workgroup per node holds both rows whole, so the
  // nodes never wait for each other and a batch of any size is one launch
  // (then one wave per sequence walks the decisions).  A node then runs on
  // one CU instead of ceil(V / 8192), so it pays where the fused kernel
  // would need slices: batches beyond its co-resident capacity.
  // EAGLE_VERIFY_NODE_PARALLEL=1 / 0 forces it on / off.
  const char* npv = std::getenv("EAGLE_VERIFY_NODE_PARALLEL");
  const bool np_auto = static_cast<int64_t>(k.B) * per_seq > cap;
  const bool np = npv && (npv[0] == '0' || npv[0] == '1') ? npv[0] == '1' : np_auto;
  if (V <= kNodeVocab && !k.wr && np) {
    k.fused = 2;
    k.stamps = (stamps && static_cast<int64_t>(k.B) * (k.T + 1) * kStampSlots <= stamp_words) ? stamps : nullptr;
    const int e = launch_spec_accept(k, bf16, hip_stream);
    if (e != 0) return hip_fail_to(err, errlen, "spec accept launch", e);
    cs->last_paths = EAGLE_ACCEPT_PATH_NODE_PARALLEL;
    return EAGLE_OK;
  }
  if (per_seq > cap || k.NC > 64) {
    k.fused = 0;
    k.wr_kept = ws.wr_kept;
    const int e = launch_spec_accept(k, bf16, hip_stream);
    if (e != 0) return hip_fail_to(err, errlen, "spec accept launch", e);
    cs->last_paths = EAGLE_ACCEPT_PATH_THREE_KERNEL;
    return EAGLE_OK;
  }
  int paths = 0;
  const int slice = static_cast<int>(std::min<int64_t>(k.B, cap / per_seq));
  const int64_t row_bytes = static_cast<int64_t>(V) * esize;
  const AcceptKernelArgs whole = k;
  for (int b0 = 0; b0 < whole.B; b0 += slice) {
    k = whole;
    k.fused = 1;
    k.b0 = b0;
    k.B = std::min(slice, whole.B - b0);
    const int64_t rows0 = static_cast<int64_t>(b0) * whole.T;
    k.target = static_cast<const char*>(whole.target) + rows0 * row_bytes;
    if (whole.draft) k.draft = static_cast<const char*>(whole.draft) + rows0 * row_bytes;
    k.parents = whole.parents + rows0;
    k.tokens = whole.tokens + rows0;
    k.accept_len = whole.accept_len + b0;
    k.accepted_nodes = whole.accepted_nodes + rows0;
    k.out_tokens = whole.out_tokens + rows0;
    k.flags = whole.flags + b0;
    k.near_ties = whole.near_ties + b0;
    if (whole.thr) {
      k.thr = whole.thr + rows0 * 2;
      k.thr_near = whole.thr_near + rows0 * 2;
    }
    k.epoch = b0 == 0 ? whole.epoch : ++cs->epoch;
    // the two halves of the round words alternate between fused launches
    const int64_t half = Bm * Tm * kRoundWords;
    const int parity = static_cast<int>(cs->fused_calls & 1);
    k.round_sum = ws.round_sum + parity * half;
    k.round_clear = ws.round_sum + (1 - parity) * half;
    k.zero_b = cs->last_fused_b;
    k.coop = coop ? 1 : 0;
    // Sampled mode, launches that stage at least 8 MiB of target rows: a leaf
    // requests its rows 8 steps of 640 clocks (about 2.1 us) later, so that
    // the internal nodes' rows, which gate the decisions, are served first
    // from HBM.  Smaller launches gain nothing from the order, and there a
    // walk that ends at a leaf would wait for it; greedy walks end at leaves
    // soon after the statistics.  (LATE kernel of the common path.)
    if (k.tau > 0.f && k.vec_ok && !k.wr && static_cast<int64_t>(k.B) * k.T * row_bytes >= (8ll << 20))
      k.leaf_wait = 8;
    k.stamps = (stamps && static_cast<int64_t>(k.B) * per_seq * kStampSlots <= stamp_words) ? stamps : nullptr;
    int e = launch_spec_accept(k, bf16, hip_stream);
    if (e == static_cast<int>(hipErrorCooperativeLaunchTooLarge)) {
      // the slice's workgroups cannot all be resident now: the three-kernel
      // path (no waiting between workgroups) verifies it instead
      (void)hipGetLastError();
      k.fused = 0;
      k.wr_kept = ws.wr_kept;
      e = launch_spec_accept(k, bf16, hip_stream);
      if (e != 0) return hip_fail_to(err, errlen, "spec accept launch", e);
      paths |= EAGLE_ACCEPT_PATH_THREE_KERNEL;
      continue;
    }
    if (e != 0) return hip_fail_to(err, errlen, "spec accept launch", e);
    ++cs->fused_calls;
    cs->last_fused_b = k.B;
    paths |= EAGLE_ACCEPT_PATH_FUSED;
  }
  cs->last_paths = paths;
  return EAGLE_OK;
}

}  // namespace ev

extern "C" {

eagle_status eagle_verify_create(const eagle_verify_desc* desc, eagle_verify** out) {
  if (!out) {
    set_err(nullptr, "out is NULL");
    return EAGLE_ERR_ARG;
  }
  *out = nullptr;
  char msg[512] = {0};
  eagle_status st = ev::check_desc(desc, msg, sizeof(msg));
  if (st != EAGLE_OK) {
    set_err(nullptr, msg);
    return st;
  }
  eagle_verify* h = new (std::nothrow) eagle_verify();
  if (!h) {
    set_err(nullptr, "host allocation failed");
    return EAGLE_ERR_OOM;
  }
  h->desc = *desc;
  hipError_t e = hipGetDevice(&h->device);
  if (e != hipSuccess) {
    hip_fail(nullptr, "hipGetDevice", e);
    delete h;
    return EAGLE_ERR_HIP;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, h->device) == hipSuccess && cus > 0)
    h->num_cus = cus;

  const int64_t B = desc->max_batch, T = desc->max_tree_rows, NC = ev::vocab_chunks(desc->vocab_size);
  size_t off = 0;
  const size_t o_part = off;
  off = align_up(off + sizeof(float) * static_cast<size_t>(ev::kAttnPartFloats), 256);
  const size_t o_expand = off;   // tree-expansion chunk records
  const int64_t nce = std::min<int64_t>(ev::expand_chunks(desc->vocab_size), ev::kMaxChunksExpand);
  off = align_up(off + sizeof(ev::ChunkRecord) * B * T * nce, 256);
  const size_t o_accept = off;
  off = ev::accept_layout(B, T, static_cast<int>(NC), o_accept, nullptr, nullptr);

  e = hipMalloc(&h->base, off);
  if (e != hipSuccess) {
    hip_fail(nullptr, "hipMalloc(workspace)", e);
    delete h;
    return EAGLE_ERR_OOM;
  }
  char* p = static_cast<char*>(h->base);
  h->ws.attn_part = reinterpret_cast<float*>(p + o_part);
  h->ws.expand = reinterpret_cast<ev::ChunkRecord*>(p + o_expand);
  ev::accept_layout(B, T, static_cast<int>(NC), o_accept, p, &h->ws);
  h->ws.bytes = off;
  h->spin_limit = ev::spin_limit_from_env();
  h->coop = ev::cooperative_from_env();
  h->fused_cap[0] = ev::fused_accept_capacity(0, h->num_cus);
  h->fused_cap[1] = ev::fused_accept_capacity(1, h->num_cus);
  // the in-kernel split merge can be switched off for comparison (EAGLE_VERIFY_ATTN_FUSED_MERGE=0)
  const char* fm = std::getenv("EAGLE_VERIFY_ATTN_FUSED_MERGE");
  if (desc->kv_dtype == EAGLE_BF16 && !(fm && fm[0] == '0'))
    for (int v = 0; v < ev::kMfmaVariants; ++v)
      h->attn_cap[desc->head_dim == 128 ? 1 : 0][v] = ev::attention_capacity(desc->head_dim, v, h->num_cus);
  // The whole workspace starts at zero: counters (every call leaves them at
  // zero again), the fused path's publication, statistics and chunk-mass
  // words (tagged with the call epoch; each fused call clears the round words
  // the previous one used), and the attention partials (no tagged m/l word
  // holds a call's epoch before that call writes it).  The clear runs on a
  // private stream that is waited for here, so no device-wide
  // synchronisation is needed and the first call may use any stream.
  hipStream_t init = nullptr;
  e = hipStreamCreateWithFlags(&init, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipMemsetAsync(h->base, 0, off, init);
  if (e == hipSuccess) e = hipStreamSynchronize(init);
  if (init) (void)hipStreamDestroy(init);
  if (e != hipSuccess) {
    hip_fail(nullptr, "workspace initialisation", e);
    (void)hipFree(h->base);
    delete h;
    return EAGLE_ERR_HIP;
  }
  *out = h;
  return EAGLE_OK;
}

eagle_status eagle_verify_tree_attention(eagle_verify* h, const eagle_tree_attention_args* a, void* hip_stream) {
  if (!h) {
    set_err(nullptr, "handle is NULL");
    return EAGLE_ERR_ARG;
  }
  ev::AttnPlan plan;
  eagle_status st = ev::plan_tree_attention(&h->desc, a, h->num_cus, &plan, h->err, sizeof(h->err));
  if (st != EAGLE_OK) return st;
  ev::AttnKernelArgs k;
  std::memset(&k, 0, sizeof(k));
  k.q = a->q;
  k.k = a->k;
  k.v = a->v;
  k.kv_indptr = a->kv_indptr;
  k.parents = a->parents;
  k.out = a->out;
  k.flags = a->flags;
  k.opart = h->ws.attn_part;
  k.mlpart = h->ws.attn_part + plan.workgroups * static_cast<int64_t>(plan.rows_per_tile) * h->desc.head_dim;
  k.num_kv_rows = a->num_kv_rows;
  k.B = a->batch;
  k.T = a->tree_rows;
  k.Hq = h->desc.num_q_heads;
  k.Hkv = h->desc.num_kv_heads;
  k.g = k.Hq / k.Hkv;
  k.D = h->desc.head_dim;
  k.R = plan.R;
  k.row_tiles = plan.row_tiles;
  k.rows_per_tile = plan.rows_per_tile;
  k.chunk = plan.chunk;
  k.total_splits = plan.total_splits;
  k.nwg = static_cast<int>(plan.workgroups);
  k.late_priority = plan.late_priority;
  k.scale_log2 = a->sm_scale * 1.4426950408889634f;
  k.page_table = a->page_size ? a->page_table : nullptr;
  k.page_size = a->page_size;
  k.pps = a->pages_per_seq;
  k.num_pages = a->page_size ? a->num_kv_rows / a->page_size : 0;
  for (int b = 0; b < a->batch; ++b) {
    k.L[b] = a->prefix_lens_host[b];
    k.split_base[b] = plan.split_base[b];
  }
  k.split_base[a->batch] = plan.split_base[a->batch];
  int64_t packed = 0;
  for (int b = 0; b < a->batch; ++b) {
    const int64_t need = static_cast<int64_t>(a->prefix_lens_host[b]) + a->tree_rows;
    k.kv0_guess[b] = (packed + need <= a->num_kv_rows && packed <= INT32_MAX) ? static_cast<int32_t>(packed) : -1;
    packed += need;
  }
  k.epoch = ++h->attn_epoch;
  k.spin_limit = h->spin_limit;
  k.mlrec = reinterpret_cast<uint64_t*>(k.mlpart + 2 * plan.workgroups * static_cast<int64_t>(plan.rows_per_tile));
  k.stamps = (h->stamps && plan.workgroups * ev::kStampSlots <= h->stamp_words) ? h->stamps : nullptr;
  // the splits merge inside the kernel when every workgroup is resident at
  // once (they wait for each other); otherwise a separate merge kernel runs
  // once every workgroup has arrived, the weights of the rows a split merges
  // (at most rows_per_tile + S - 1 (row, split) pairs) are staged in its K/V ring
  int max_splits = 1;
  for (int b = 0; b < a->batch; ++b) max_splits = std::max(max_splits, plan.split_base[b + 1] - plan.split_base[b]);
  k.fused_merge = (plan.path == 1 && plan.merge_workgroups > 0 &&
                   plan.workgroups <= h->attn_cap[k.D == 128 ? 1 : 0][ev::mfma_variant(plan)] &&
                   plan.rows_per_tile + max_splits <= ev::kFusedMergePairs)
                      ? 1
                      : 0;
  // the partials of one launch must fit: O, (m, l) and the two tagged m/l
  // words per partial row
  const int64_t need = plan.workgroups * static_cast<int64_t>(plan.rows_per_tile) * (k.D + 6);
  if (plan.merge_workgroups > 0 && need > ev::kAttnPartFloats) {
    set_err(h, "split partials exceed the workspace");
    return EAGLE_ERR_CAPACITY;
  }
  hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
  k.coop = h->coop ? 1 : 0;
  int e = ev::launch_tree_attention(plan, k, h->desc.kv_dtype == EAGLE_BF16, stream);
  if (e == static_cast<int>(hipErrorCooperativeLaunchTooLarge) && k.fused_merge) {
    (void)hipGetLastError();
    k.fused_merge = 0;   // not every workgroup fits at once: merge in a separate kernel
    e = ev::launch_tree_attention(plan, k, h->desc.kv_dtype == EAGLE_BF16, stream);
  }
  h->last_stream = stream;
  h->used = true;
  if (e != 0) return hip_fail(h, "tree attention launch", e);
  public_plan(plan, &h->last_plan);
  h->last_plan.merge_in_kernel = k.fused_merge;
  h->have_plan = true;
  h->err[0] = 0;
  return EAGLE_OK;
}

eagle_status eagle_verify_spec_accept(eagle_verify* h, const eagle_spec_accept_args* a, void* hip_stream) {
  if (!h) {
    set_err(nullptr, "handle is NULL");
    return EAGLE_ERR_ARG;
  }
  eagle_status st = ev::check_spec_accept(&h->desc, a, h->err, sizeof(h->err));
  if (st != EAGLE_OK) return st;
  h->last_stream = reinterpret_cast<hipStream_t>(hip_stream);
  h->used = true;
  const int64_t cap = h->fused_cap[h->desc.logits_dtype == EAGLE_BF16 ? 1 : 0];
  st = ev::run_spec_accept(h->desc, h->ws, h->desc.max_batch, h->desc.max_tree_rows, cap, &h->accept_state, a,
                           hip_stream, h->err, sizeof(h->err), h->spin_limit, h->coop, h->stamps, h->stamp_words);
  if (st == EAGLE_OK) h->err[0] = 0;
  return st;
}

eagle_status eagle_verify_kv_commit(eagle_verify* h, const eagle_kv_commit_args* a, void* hip_stream) {
  if (!h) {
    set_err(nullptr, "handle is NULL");
    return EAGLE_ERR_ARG;
  }
  eagle_status st = ev::check_kv_commit(&h->desc, a, h->err, sizeof(h->err));
  if (st != EAGLE_OK) return st;
  ev::CommitKernelArgs k;
  std::memset(&k, 0, sizeof(k));
  k.k = a->k;
  k.v = a->v;
  k.kv_indptr = a->kv_indptr;
  k.accept_len = a->accept_len;
  k.accepted_nodes = a->accepted_nodes;
  k.new_lens = a->new_lens;
  k.flags = a->flags;
  k.num_kv_rows = a->num_kv_rows;
  k.B = a->batch;
  k.T = a->tree_rows;
  k.Hkv = h->desc.num_kv_heads;
  k.D = h->desc.head_dim;
  k.layers = a->num_layers;
  k.layer_stride = a->layer_stride;
  k.page_table = a->page_size ? a->page_table : nullptr;
  k.page_size = a->page_size;
  k.pps = a->pages_per_seq;
  k.num_pages = a->page_size ? a->num_kv_rows / a->page_size : 0;
  for (int b = 0; b < a->batch; ++b) k.L[b] = a->prefix_lens_host[b];
  // heads per workgroup: split each row into the largest number of head
  // groups (a power of two dividing Hkv) that keeps the launch within 256
  // workgroups, so a single sequence still spreads over the chip while a
  // large batch moves whole rows (thousands of one-head workgroups cost more
  // in per-workgroup set-up than they gain; 1024 was slower at B = 4)
  k.head_groups = 1;
  while (k.head_groups * 2 <= k.Hkv && k.Hkv % (k.head_groups * 2) == 0 &&
         static_cast<int64_t>(k.layers) * k.B * k.head_groups * 2 <= 256)
    k.head_groups *= 2;
  hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
  const int e = ev::launch_kv_commit(k, h->desc.kv_dtype == EAGLE_BF16, stream);
  h->last_stream = stream;
  h->used = true;
  if (e != 0) return hip_fail(h, "kv commit launch", e);
  h->err[0] = 0;
  return EAGLE_OK;
}

eagle_status eagle_verify_tree_expand(eagle_verify* h, const eagle_tree_expand_args* a, void* hip_stream) {
  if (!h) {
    set_err(nullptr, "handle is NULL");
    return EAGLE_ERR_ARG;
  }
  eagle_status st = ev::check_tree_expand(&h->desc, a, h->err, sizeof(h->err));
  if (st != EAGLE_OK) return st;
  ev::ExpandKernelArgs k;
  std::memset(&k, 0, sizeof(k));
  k.logits = a->draft_logits;
  k.scores = a->scores;
  k.chunks = h->ws.expand;
  k.parent = a->parent;
  k.token = a->token;
  k.value = a->value;
  k.flags = a->flags;
  k.near_ties = a->near_ties;
  k.B = a->batch;
  k.F = a->frontier;
  k.V = h->desc.vocab_size;
  k.chunk = ev::expand_chunk(k.V);
  k.NC = ev::expand_chunks(k.V);
  k.K = a->top_k;
  k.M = a->keep;
  k.c2 = static_cast<float>(1.4426950408889634 / a->temperature);
  k.inv_tau = 1.0 / static_cast<double>(a->temperature);
  k.stamps = (h->stamps && (static_cast<int64_t>(k.B) * k.F * k.NC + k.B) * ev::kStampSlots <= h->stamp_words)
                 ? h->stamps : nullptr;
  hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
  const int e = ev::launch_tree_expand(k, h->desc.logits_dtype == EAGLE_BF16, stream);
  h->last_stream = stream;
  h->used = true;
  if (e != 0) return hip_fail(h, "tree expansion launch", e);
  h->err[0] = 0;
  return EAGLE_OK;
}

eagle_status eagle_verify_tree_rerank(eagle_verify* h, const eagle_tree_rerank_args* a, void* hip_stream) {
  if (!h) {
    set_err(nullptr, "handle is NULL");
    return EAGLE_ERR_ARG;
  }
  eagle_status st = ev::check_tree_rerank(&h->desc, a, h->err, sizeof(h->err));
  if (st != EAGLE_OK) return st;
  ev::RerankKernelArgs k;
  std::memset(&k, 0, sizeof(k));
  k.parent = a->parent;
  k.token = a->token;
  k.value = a->value;
  k.root_tokens = a->root_tokens;
  k.parents = a->parents;
  k.tokens = a->tokens;
  k.rows = a->rows;
  k.B = a->batch;
  k.D = a->steps;
  k.M = a->keep;
  k.N = a->nodes;
  hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
  const int e = ev::launch_tree_rerank(k, stream);
  h->last_stream = stream;
  h->used = true;
  if (e != 0) return hip_fail(h, "tree rerank launch", e);
  h->err[0] = 0;
  return EAGLE_OK;
}

eagle_status eagle_verify_destroy(eagle_verify* h) {
  if (!h) return EAGLE_OK;
  eagle_status st = EAGLE_OK;
  if (h->used) {
    hipError_t e = hipStreamSynchronize(h->last_stream);
    if (e != hipSuccess) st = hip_fail(nullptr, "hipStreamSynchronize", e);
  }
  if (h->base) {
    hipError_t e = hipFree(h->base);
    if (e != hipSuccess && st == EAGLE_OK) st = hip_fail(nullptr, "hipFree", e);
  }
  delete h;
  return st;
}

const char* eagle_verify_last_error(const eagle_verify* h) { return h ? h->err : g_err; }

eagle_status eagle_verify_check_tree_attention(const eagle_verify_desc* desc, const eagle_tree_attention_args* a,
                                               eagle_attention_plan* plan) {
  ev::AttnPlan p;
  eagle_status st = ev::plan_tree_attention(desc, a, ev::kDefaultCUs, &p, g_err, sizeof(g_err));
  if (st != EAGLE_OK) return st;
  if (plan) public_plan(p, plan);
  g_err[0] = 0;
  return EAGLE_OK;
}

eagle_status eagle_verify_set_timeline(eagle_verify* h, uint64_t* device_words, int64_t num_words) {
  if (!h) {
    set_err(nullptr, "handle is NULL");
    return EAGLE_ERR_ARG;
  }
  if (num_words < 0 || (reinterpret_cast<uintptr_t>(device_words) & 7u) != 0) {
    set_err(h, "timeline: num_words < 0 or device_words not 8-byte aligned");
    return EAGLE_ERR_ARG;
  }
  h->stamps = (device_words && num_words > 0) ? device_words : nullptr;
  h->stamp_words = h->stamps ? num_words : 0;
  h->err[0] = 0;
  return EAGLE_OK;
}

eagle_status eagle_verify_last_attention_plan(const eagle_verify* h, eagle_attention_plan* plan) {
  if (!h || !plan || !h->have_plan) return EAGLE_ERR_ARG;
  *plan = h->last_plan;
  return EAGLE_OK;
}

eagle_status eagle_verify_last_accept_paths(const eagle_verify* h, int* paths) {
  if (!h || !paths || h->accept_state.last_paths == 0) return EAGLE_ERR_ARG;
  *paths = h->accept_state.last_paths;
  return EAGLE_OK;
}

eagle_status eagle_verify_check_spec_accept(const eagle_verify_desc* desc, const eagle_spec_accept_args* a) {
  eagle_status st = ev::check_spec_accept(desc, a, g_err, sizeof(g_err));
  if (st == EAGLE_OK) g_err[0] = 0;
  return st;
}

eagle_status eagle_verify_check_kv_commit(const eagle_verify_desc* desc, const eagle_kv_commit_args* a) {
  eagle_status st = ev::check_kv_commit(desc, a, g_err, sizeof(g_err));
  if (st == EAGLE_OK) g_err[0] = 0;
  return st;
}

eagle_status eagle_verify_check_tree_expand(const eagle_verify_desc* desc, const eagle_tree_expand_args* a) {
  eagle_status st = ev::check_tree_expand(desc, a, g_err, sizeof(g_err));
  if (st == EAGLE_OK) g_err[0] = 0;
  return st;
}

eagle_status eagle_verify_check_tree_rerank(const eagle_verify_desc* desc, const eagle_tree_rerank_args* a) {
  eagle_status st = ev::check_tree_rerank(desc, a, g_err, sizeof(g_err));
  if (st == EAGLE_OK) g_err[0] = 0;
  return st;
}

}  // extern "C"
