// Host-side argument validation and launch planning for libeagle_verify.
// Pure C++: no HIP call is made here, so everything in this file runs (and is
// tested) without a GPU.
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "ev_internal.h"

static_assert(sizeof(eagle_dtype) == sizeof(int32_t), "dtype fields are 32-bit in the C ABI");

namespace ev {
namespace {

eagle_status fail(eagle_status st, char* err, size_t errlen, const char* fmt, ...) {
  if (err && errlen) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(err, errlen, fmt, ap);
    va_end(ap);
  }
  return st;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int env_int(const char* name, int dflt) {
  const char* s = std::getenv(name);
  if (!s || !*s) return dflt;
  int v = std::atoi(s);
  return v > 0 ? v : dflt;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

int vocab_chunks(int V) { return static_cast<int>(ceil_div(V, kVocabChunk)); }

eagle_status check_desc(const eagle_verify_desc* d, char* err, size_t errlen) {
  if (!d) return fail(EAGLE_ERR_ARG, err, errlen, "descriptor is NULL");
  if (d->max_batch < 1 || d->max_batch > kMaxBatch)
    return fail(EAGLE_ERR_ARG, err, errlen, "max_batch=%d outside [1, %d]", d->max_batch, kMaxBatch);
  if (d->num_q_heads < 1 || d->num_kv_heads < 1 || d->num_q_heads % d->num_kv_heads != 0)
    return fail(EAGLE_ERR_ARG, err, errlen, "num_q_heads=%d must be a positive multiple of num_kv_heads=%d",
                d->num_q_heads, d->num_kv_heads);
  if (d->num_q_heads > 4096)
    return fail(EAGLE_ERR_ARG, err, errlen, "num_q_heads=%d above 4096", d->num_q_heads);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(EAGLE_ERR_UNSUPPORTED, err, errlen, "head_dim=%d (supported: 64, 128)", d->head_dim);
  if (d->max_tree_rows < 1 || d->max_tree_rows > kMaxTree)
    return fail(EAGLE_ERR_ARG, err, errlen, "max_tree_rows=%d outside [1, %d]", d->max_tree_rows, kMaxTree);
  if (d->vocab_size < 2 || d->vocab_size > (1 << 30))
    return fail(EAGLE_ERR_ARG, err, errlen, "vocab_size=%d outside [2, 2^30]", d->vocab_size);
  // a C caller may store any integer in the enum fields: read their bits
  int32_t kvd, lgd;
  std::memcpy(&kvd, &d->kv_dtype, sizeof(kvd));
  std::memcpy(&lgd, &d->logits_dtype, sizeof(lgd));
  if ((kvd != EAGLE_F32 && kvd != EAGLE_BF16) || (lgd != EAGLE_F32 && lgd != EAGLE_BF16))
    return fail(EAGLE_ERR_ARG, err, errlen, "unknown dtype");
  return EAGLE_OK;
}

// Paged K/V layout (page_size > 0): page size a multiple of 64 dividing the
// row count, and a table row long enough for every sequence's L_b + T rows.
static eagle_status check_paging(const int32_t* table, int32_t page_size, int32_t pages_per_seq,
                                 int64_t num_kv_rows, const int32_t* lens, int B, int T, char* err,
                                 size_t errlen) {
  if (page_size == 0) return EAGLE_OK;
  if (page_size < 0 || page_size % 64 != 0 || page_size > (1 << 20))
    return fail(EAGLE_ERR_ARG, err, errlen, "page_size=%d: 0 or a multiple of 64 up to 2^20", page_size);
  if (!table) return fail(EAGLE_ERR_ARG, err, errlen, "page_table is NULL with page_size > 0");
  if (!aligned(table, 4)) return fail(EAGLE_ERR_ARG, err, errlen, "page_table misaligned");
  if (num_kv_rows > static_cast<int64_t>(UINT32_MAX))
    return fail(EAGLE_ERR_CAPACITY, err, errlen, "paged K/V holds more than 2^32 - 1 rows");
  if (num_kv_rows % page_size != 0)
    return fail(EAGLE_ERR_ARG, err, errlen, "num_kv_rows=%lld not a multiple of page_size=%d",
                static_cast<long long>(num_kv_rows), page_size);
  if (pages_per_seq < 1) return fail(EAGLE_ERR_ARG, err, errlen, "pages_per_seq=%d < 1", pages_per_seq);
  if (static_cast<int64_t>(B) * pages_per_seq > INT32_MAX)
    return fail(EAGLE_ERR_CAPACITY, err, errlen, "batch * pages_per_seq above 2^31 - 1");
  for (int b = 0; b < B; ++b) {
    const int64_t need = (static_cast<int64_t>(lens[b]) + T + page_size - 1) / page_size;
    if (need > pages_per_seq)
      return fail(EAGLE_ERR_ARG, err, errlen, "sequence %d needs %lld pages, pages_per_seq=%d", b,
                  static_cast<long long>(need), pages_per_seq);
  }
  return EAGLE_OK;
}

eagle_status plan_tree_attention(const eagle_verify_desc* d, const eagle_tree_attention_args* a,
                                 int num_cus, AttnPlan* plan, char* err, size_t errlen) {
  eagle_status st = check_desc(d, err, errlen);
  if (st != EAGLE_OK) return st;
  if (!a) return fail(EAGLE_ERR_ARG, err, errlen, "args is NULL");
  if (!plan) return fail(EAGLE_ERR_ARG, err, errlen, "plan is NULL");
  if (a->batch < 1) return fail(EAGLE_ERR_ARG, err, errlen, "batch=%d < 1", a->batch);
  if (a->batch > d->max_batch)
    return fail(EAGLE_ERR_CAPACITY, err, errlen, "batch=%d above max_batch=%d", a->batch, d->max_batch);
  if (a->tree_rows < 1) return fail(EAGLE_ERR_ARG, err, errlen, "tree_rows=%d < 1", a->tree_rows);
  if (a->tree_rows > d->max_tree_rows)
    return fail(EAGLE_ERR_CAPACITY, err, errlen, "tree_rows=%d above max_tree_rows=%d", a->tree_rows,
                d->max_tree_rows);
  if (a->num_kv_rows < 0) return fail(EAGLE_ERR_ARG, err, errlen, "num_kv_rows < 0");
  const bool paged = a->page_size != 0;
  if (!a->q || !a->k || !a->v || (!paged && !a->kv_indptr) || !a->prefix_lens_host || !a->parents || !a->out ||
      !a->flags)
    return fail(EAGLE_ERR_ARG, err, errlen, "a required pointer is NULL");
  if (!aligned(a->q, 16) || !aligned(a->k, 16) || !aligned(a->v, 16) || !aligned(a->out, 16))
    return fail(EAGLE_ERR_ARG, err, errlen, "q, k, v and out must be 16-byte aligned");
  if ((!paged && !aligned(a->kv_indptr, 8)) || !aligned(a->parents, 4) || !aligned(a->flags, 4))
    return fail(EAGLE_ERR_ARG, err, errlen, "kv_indptr/parents/flags misaligned");
  if (!std::isfinite(a->sm_scale) || a->sm_scale <= 0.f)
    return fail(EAGLE_ERR_ARG, err, errlen, "sm_scale must be finite and > 0");

  const int B = a->batch, T = a->tree_rows;
  const int Hkv = d->num_kv_heads, g = d->num_q_heads / d->num_kv_heads, D = d->head_dim;
  int64_t total_keys = 0;
  for (int b = 0; b < B; ++b) {
    const int32_t L = a->prefix_lens_host[b];
    if (L < 0) return fail(EAGLE_ERR_ARG, err, errlen, "prefix_lens_host[%d]=%d < 0", b, L);
    if (static_cast<int64_t>(L) + T > a->num_kv_rows)
      return fail(EAGLE_ERR_CAPACITY, err, errlen, "sequence %d needs %lld KV rows, only %lld allocated",
                  b, static_cast<long long>(L) + T, static_cast<long long>(a->num_kv_rows));
    total_keys += L;
  }
  st = check_paging(a->page_table, a->page_size, a->pages_per_seq, a->num_kv_rows, a->prefix_lens_host, B, T, err,
                    errlen);
  if (st != EAGLE_OK) return st;

  std::memset(plan, 0, sizeof(*plan));
  const int R = T * g;
  plan->R = R;
  plan->path = (d->kv_dtype == EAGLE_BF16 && R >= 16) ? 1 : 0;
  int target_wgs;
  int min_chunk;
  if (plan->path == 1) {
    // rows per workgroup: 64 * mb, mb <= 4 (tuning override EAGLE_VERIFY_ATTN_MB).
    // One 16-row block per wave keeps the kernel at two waves per SIMD; the
    // row tiles of one KV chunk then share its K/V tiles through L2.
    const int mb_env = env_int("EAGLE_VERIFY_ATTN_MB", 1);
    const int max_mb = mb_env > 2 ? 2 : (mb_env < 1 ? 1 : mb_env);
    plan->stages = 2;
    if (R <= 32) {
      // at most two 16-row blocks per KV head: wave pairs split the keys of
      // each tile instead of padding the workgroup to 64 rows
      plan->row_tiles = 1;
      plan->rows_per_tile = 32;
      plan->mb = 1;
      plan->kg = 2;
    } else {
      int rt = static_cast<int>(ceil_div(R, 64 * max_mb));
      int rows = static_cast<int>(ceil_div(ceil_div(R, rt), 64) * 64);
      plan->row_tiles = rt;
      plan->rows_per_tile = rows;
      plan->mb = rows / 64;
      plan->kg = 1;
    }
    // two row blocks per wave run one workgroup per CU (512 registers a wave)
    target_wgs = num_cus * env_int("EAGLE_VERIFY_ATTN_WG_PER_CU", plan->mb > 1 ? 1 : 2);
    min_chunk = 2 * kTileKeys;
  } else {
    plan->row_tiles = R;
    plan->rows_per_tile = 1;
    plan->mb = 0;
    target_wgs = num_cus * env_int("EAGLE_VERIFY_FMA_WG_PER_CU", 8);
    min_chunk = kTileKeys;
  }
  const int64_t units = static_cast<int64_t>(Hkv) * plan->row_tiles;
  int64_t chunk = ceil_div(total_keys * units, target_wgs);
  chunk = ceil_div(chunk, kTileKeys) * kTileKeys;
  if (chunk < min_chunk) chunk = min_chunk;
  if (const char* f = std::getenv("EAGLE_VERIFY_ATTN_CHUNK")) {   // tuning override
    int v = std::atoi(f);
    if (v >= kTileKeys) chunk = ceil_div(v, kTileKeys) * kTileKeys;
  }
  for (;;) {
    int64_t splits = 0, part = 0;
    bool any_multi = false;
    for (int b = 0; b < B; ++b) {
      const int64_t L = a->prefix_lens_host[b];
      const int64_t S = L > 0 ? ceil_div(L, chunk) : 1;
      plan->splits[b] = static_cast<int32_t>(S);
      plan->split_base[b] = static_cast<int32_t>(splits);
      splits += S;
      if (S > 1) any_multi = true;
    }
    plan->split_base[B] = static_cast<int32_t>(splits);
    // partial slots are indexed by workgroup, so all of them are reserved
    if (any_multi) part = splits * units * plan->rows_per_tile * (D + 6);
    if (part <= kAttnPartFloats && splits < (1ll << 30)) {
      plan->total_splits = static_cast<int>(splits);
      plan->part_floats = part;
      plan->chunk = static_cast<int>(chunk);
      plan->workgroups = splits * units;
      // measured: pays from 4 prefix tiles per workgroup (tuning override
      // EAGLE_VERIFY_ATTN_LATE_PRIORITY = 1 on, 2 off)
      const int lp = env_int("EAGLE_VERIFY_ATTN_LATE_PRIORITY", 0);
      plan->late_priority = (plan->path == 1 && (lp == 1 || (lp != 2 && chunk >= 4 * kTileKeys))) ? 1 : 0;
      plan->merge_workgroups = any_multi ? static_cast<int64_t>(B) * units : 0;
      break;
    }
    chunk *= 2;
  }
  return EAGLE_OK;
}

eagle_status check_spec_accept(const eagle_verify_desc* d, const eagle_spec_accept_args* a,
                               char* err, size_t errlen) {
  eagle_status st = check_desc(d, err, errlen);
  if (st != EAGLE_OK) return st;
  if (!a) return fail(EAGLE_ERR_ARG, err, errlen, "args is NULL");
  if (a->batch < 1) return fail(EAGLE_ERR_ARG, err, errlen, "batch=%d < 1", a->batch);
  if (a->batch > d->max_batch)
    return fail(EAGLE_ERR_CAPACITY, err, errlen, "batch=%d above max_batch=%d", a->batch, d->max_batch);
  if (a->tree_rows < 1) return fail(EAGLE_ERR_ARG, err, errlen, "tree_rows=%d < 1", a->tree_rows);
  if (a->tree_rows > d->max_tree_rows)
    return fail(EAGLE_ERR_CAPACITY, err, errlen, "tree_rows=%d above max_tree_rows=%d", a->tree_rows,
                d->max_tree_rows);
  if (!std::isfinite(a->temperature) || a->temperature < 0.f)
    return fail(EAGLE_ERR_ARG, err, errlen, "temperature must be finite and >= 0");
  if (a->without_replacement != 0 && a->without_replacement != 1)
    return fail(EAGLE_ERR_ARG, err, errlen, "without_replacement=%d: 0 or 1", a->without_replacement);
  if (a->top_k < 0) return fail(EAGLE_ERR_ARG, err, errlen, "top_k=%d < 0", a->top_k);
  if (!(a->top_p >= 0.f && a->top_p <= 1.f))
    return fail(EAGLE_ERR_ARG, err, errlen, "top_p must lie in [0, 1] (0 or 1: no nucleus filter)");
  if (!a->target_logits || !a->parents || !a->tokens || !a->accept_len || !a->accepted_nodes ||
      !a->out_tokens || !a->flags || !a->near_ties)
    return fail(EAGLE_ERR_ARG, err, errlen, "a required pointer is NULL");
  if (a->temperature > 0.f && !a->draft_logits)
    return fail(EAGLE_ERR_ARG, err, errlen, "draft_logits is NULL with temperature > 0");
  if (!aligned(a->target_logits, 16) || (a->draft_logits && !aligned(a->draft_logits, 16)))
    return fail(EAGLE_ERR_ARG, err, errlen, "logits must be 16-byte aligned");
  if (!aligned(a->parents, 4) || !aligned(a->tokens, 4) || !aligned(a->accept_len, 4) ||
      !aligned(a->accepted_nodes, 4) || !aligned(a->out_tokens, 4) || !aligned(a->flags, 4) ||
      !aligned(a->near_ties, 4))
    return fail(EAGLE_ERR_ARG, err, errlen, "integer buffers must be 4-byte aligned");
  return EAGLE_OK;
}

eagle_status check_kv_commit(const eagle_verify_desc* d, const eagle_kv_commit_args* a, char* err, size_t errlen) {
  eagle_status st = check_desc(d, err, errlen);
  if (st != EAGLE_OK) return st;
  if (!a) return fail(EAGLE_ERR_ARG, err, errlen, "args is NULL");
  if (a->batch < 1) return fail(EAGLE_ERR_ARG, err, errlen, "batch=%d < 1", a->batch);
  if (a->batch > d->max_batch)
    return fail(EAGLE_ERR_CAPACITY, err, errlen, "batch=%d above max_batch=%d", a->batch, d->max_batch);
  if (a->tree_rows < 1) return fail(EAGLE_ERR_ARG, err, errlen, "tree_rows=%d < 1", a->tree_rows);
  if (a->tree_rows > d->max_tree_rows)
    return fail(EAGLE_ERR_CAPACITY, err, errlen, "tree_rows=%d above max_tree_rows=%d", a->tree_rows,
                d->max_tree_rows);
  if (a->num_kv_rows < 0) return fail(EAGLE_ERR_ARG, err, errlen, "num_kv_rows < 0");
  const bool paged = a->page_size != 0;
  if (!a->k || !a->v || (!paged && !a->kv_indptr) || !a->prefix_lens_host || !a->accept_len || !a->accepted_nodes ||
      !a->new_lens || !a->flags)
    return fail(EAGLE_ERR_ARG, err, errlen, "a required pointer is NULL");
  if (!aligned(a->k, 16) || !aligned(a->v, 16))
    return fail(EAGLE_ERR_ARG, err, errlen, "k and v must be 16-byte aligned");
  if ((!paged && !aligned(a->kv_indptr, 8)) || !aligned(a->accept_len, 4) || !aligned(a->accepted_nodes, 4) ||
      !aligned(a->new_lens, 4) || !aligned(a->flags, 4))
    return fail(EAGLE_ERR_ARG, err, errlen, "integer buffers misaligned");
  for (int b = 0; b < a->batch; ++b)
    if (a->prefix_lens_host[b] < 0)
      return fail(EAGLE_ERR_ARG, err, errlen, "prefix_lens_host[%d]=%d < 0", b, a->prefix_lens_host[b]);
  st = check_paging(a->page_table, a->page_size, a->pages_per_seq, a->num_kv_rows, a->prefix_lens_host, a->batch,
                    a->tree_rows, err, errlen);
  if (st != EAGLE_OK) return st;
  if (a->num_layers < 1 || a->num_layers > 4096)
    return fail(EAGLE_ERR_ARG, err, errlen, "num_layers=%d outside [1, 4096]", a->num_layers);
  if (static_cast<int64_t>(a->num_layers) * a->batch * d->num_kv_heads > INT32_MAX)
    return fail(EAGLE_ERR_CAPACITY, err, errlen, "num_layers * batch * num_kv_heads above 2^31 - 1");
  const int64_t layer_elems = a->num_kv_rows * d->num_kv_heads * d->head_dim;
  if (a->num_layers > 1 && a->layer_stride < layer_elems)
    return fail(EAGLE_ERR_ARG, err, errlen, "layer_stride=%lld below one layer's %lld elements",
                static_cast<long long>(a->layer_stride), static_cast<long long>(layer_elems));
  const int esize = d->kv_dtype == EAGLE_BF16 ? 2 : 4;
  if ((a->layer_stride * esize) % 16 != 0)
    return fail(EAGLE_ERR_ARG, err, errlen, "layer_stride must keep every layer 16-byte aligned");
  return EAGLE_OK;
}

eagle_status check_tree_expand(const eagle_verify_desc* d, const eagle_tree_expand_args* a, char* err,
                               size_t errlen) {
  eagle_status st = check_desc(d, err, errlen);
  if (st != EAGLE_OK) return st;
  if (!a) return fail(EAGLE_ERR_ARG, err, errlen, "args is NULL");
  if (a->batch < 1) return fail(EAGLE_ERR_ARG, err, errlen, "batch=%d < 1", a->batch);
  if (a->batch > d->max_batch)
    return fail(EAGLE_ERR_CAPACITY, err, errlen, "batch=%d above max_batch=%d", a->batch, d->max_batch);
  if (a->frontier < 1) return fail(EAGLE_ERR_ARG, err, errlen, "frontier=%d < 1", a->frontier);
  if (a->frontier > d->max_tree_rows)
    return fail(EAGLE_ERR_CAPACITY, err, errlen, "frontier=%d above max_tree_rows=%d", a->frontier,
                d->max_tree_rows);
  if (a->top_k < 1 || a->top_k > kMaxTopK)
    return fail(EAGLE_ERR_ARG, err, errlen, "top_k=%d outside [1, %d]", a->top_k, kMaxTopK);
  if (a->keep < 1 || a->keep > kMaxKeep)
    return fail(EAGLE_ERR_ARG, err, errlen, "keep=%d outside [1, %d]", a->keep, kMaxKeep);
  if (expand_chunks(d->vocab_size) > kMaxChunksExpand)
    return fail(EAGLE_ERR_UNSUPPORTED, err, errlen, "vocab_size=%d above %d for tree expansion", d->vocab_size,
                kMaxChunksExpand * kVocabChunk);
  if (!(a->temperature > 0.f) || !std::isfinite(a->temperature))
    return fail(EAGLE_ERR_ARG, err, errlen, "temperature must be finite and > 0");
  if (!a->draft_logits || !a->scores || !a->parent || !a->token || !a->value || !a->flags || !a->near_ties)
    return fail(EAGLE_ERR_ARG, err, errlen, "a required pointer is NULL");
  if (!aligned(a->draft_logits, 4) || !aligned(a->scores, 4) || !aligned(a->parent, 4) || !aligned(a->token, 4) ||
      !aligned(a->value, 4) || !aligned(a->flags, 4) || !aligned(a->near_ties, 4))
    return fail(EAGLE_ERR_ARG, err, errlen, "buffers must be 4-byte aligned");
  return EAGLE_OK;
}

eagle_status check_tree_rerank(const eagle_verify_desc* d, const eagle_tree_rerank_args* a, char* err,
                               size_t errlen) {
  eagle_status st = check_desc(d, err, errlen);
  if (st != EAGLE_OK) return st;
  if (!a) return fail(EAGLE_ERR_ARG, err, errlen, "args is NULL");
  if (a->batch < 1) return fail(EAGLE_ERR_ARG, err, errlen, "batch=%d < 1", a->batch);
  if (a->batch > d->max_batch)
    return fail(EAGLE_ERR_CAPACITY, err, errlen, "batch=%d above max_batch=%d", a->batch, d->max_batch);
  if (a->steps < 1 || a->steps > kMaxSteps)
    return fail(EAGLE_ERR_ARG, err, errlen, "steps=%d outside [1, %d]", a->steps, kMaxSteps);
  if (a->keep < 1 || a->keep > kMaxKeep)
    return fail(EAGLE_ERR_ARG, err, errlen, "keep=%d outside [1, %d]", a->keep, kMaxKeep);
  if (a->nodes < 0) return fail(EAGLE_ERR_ARG, err, errlen, "nodes=%d < 0", a->nodes);
  if (a->nodes + 1 > d->max_tree_rows)
    return fail(EAGLE_ERR_CAPACITY, err, errlen, "nodes + 1 = %d above max_tree_rows=%d", a->nodes + 1,
                d->max_tree_rows);
  if (!a->parent || !a->token || !a->value || !a->root_tokens || !a->parents || !a->tokens || !a->rows)
    return fail(EAGLE_ERR_ARG, err, errlen, "a required pointer is NULL");
  if (!aligned(a->parent, 4) || !aligned(a->token, 4) || !aligned(a->value, 4) || !aligned(a->root_tokens, 4) ||
      !aligned(a->parents, 4) || !aligned(a->tokens, 4) || !aligned(a->rows, 4))
    return fail(EAGLE_ERR_ARG, err, errlen, "buffers must be 4-byte aligned");
  return EAGLE_OK;
}

}  // namespace ev
