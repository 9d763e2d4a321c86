/*
 * eagle_verify.h — C ABI of the EAGLE draft-tree verification step, one
 * target layer at a time, for AMD Instinct MI355X (gfx950).
 *
 * The verification step of EAGLE speculative decoding (EAGLE notes page,
 * core mechanism §5 and the GPU data-path steps ⑥–⑦; speculative-decoding
 * lesson page, "Concept" and build steps 1–3) has two parts, each one call:
 *
 *   eagle_verify_tree_attention  every draft-tree node attends to the whole
 *       prefix KV cache plus only its own ancestors and itself (the "tree
 *       attention" term on the EAGLE notes page; the lesson page's glossary
 *       calls it attention under a non-causal mask that follows the tree).
 *   eagle_verify_spec_accept     multi-round speculative sampling over the
 *       vocabulary: softmax of target (q) and draft (p) logits, a walk of the
 *       tree from the root in which the children of a node are tried in
 *       ascending index, a child with token t is accepted if r < q(t)/p(t),
 *       otherwise q <- norm(max(0, q - p)) and the next child is tried; if
 *       every child is rejected the token is sampled from that residual, and
 *       at a node without children a bonus token is sampled from q.
 *
 * Conventions shared by every entry point
 *  - Every tensor pointer is DEVICE memory owned by the caller, 16-byte
 *    aligned, row-major with the innermost dimension last, and must stay
 *    alive until the work enqueued on `hip_stream` has completed.  Pointers
 *    named *_host are host memory read synchronously during the call.
 *  - Calls enqueue asynchronously on `hip_stream` (a hipStream_t, NULL = the
 *    null stream) and return; nothing is allocated per call and there is no
 *    device-wide synchronisation.  The library owns only its workspace,
 *    allocated by eagle_verify_create and freed by eagle_verify_destroy.
 *  - Argument errors are detected before any launch and returned as an
 *    eagle_status; eagle_verify_last_error() then describes the problem.
 *    Problems in device-resident contents (a parent array that is not a tree
 *    in topological order, a token outside the vocabulary, a logits row that
 *    holds NaN or +inf or is entirely -inf, a KV range that does not fit)
 *    set bits in the per-sequence `flags` output; that sequence's outputs
 *    are poisoned (NaN floats, -1 integers).  Kernels never trap.
 *  - A handle is not thread-safe and keeps per-call scratch state: use one
 *    handle per stream and do not run two calls of one handle concurrently.
 *  - Same inputs and the same (seed, offset) give bit-identical outputs.
 *  - No exception crosses this ABI.
 */
#ifndef EAGLE_VERIFY_H_
#define EAGLE_VERIFY_H_

#include <stdint.h>

#ifndef EAGLE_API
#define EAGLE_API __attribute__((visibility("default")))
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef struct eagle_verify eagle_verify; /* opaque handle */

typedef enum {
  EAGLE_OK = 0,
  EAGLE_ERR_ARG = 1,         /* null/misaligned pointer, value out of range       */
  EAGLE_ERR_UNSUPPORTED = 2, /* shape/dtype combination the library does not run  */
  EAGLE_ERR_CAPACITY = 3,    /* above the maxima given to eagle_verify_create      */
  EAGLE_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed         */
  EAGLE_ERR_OOM = 5          /* workspace allocation failed                        */
} eagle_status;

typedef enum { EAGLE_F32 = 0, EAGLE_BF16 = 1 } eagle_dtype;

/* Per-sequence `flags` bits.  Bits 0-2 and 5 poison the sequence's outputs;
 * bits 3-4 report events on the accepted walk (outputs stay valid). */
#define EAGLE_FLAG_BAD_TREE 1u          /* parents[b,0] != -1 or !(0 <= parents[b,i] < i) */
#define EAGLE_FLAG_BAD_TOKEN 2u         /* tokens[b,i] outside [0, V), i >= 1, not padding */
#define EAGLE_FLAG_NONFINITE 4u         /* a target row, or a draft row of a node with
                                           children, holds NaN/+inf or is all -inf      */
#define EAGLE_FLAG_P_ZERO 8u            /* a tested child had draft probability 0: it was
                                           accepted iff its residual target mass > 0     */
#define EAGLE_FLAG_DEGENERATE_RESIDUAL 16u /* residual mass was 0: fell back to q        */
#define EAGLE_FLAG_BAD_KV_RANGE 32u     /* kv_indptr[b..b+1] does not hold L_b + T rows
                                           inside [0, num_kv_rows)                       */
#define EAGLE_FLAG_INTERNAL 64u         /* a bounded device-side wait expired (workgroups
                                           not co-resident, e.g. other kernels occupied
                                           the device): the sequence's outputs are
                                           poisoned (-1 / NaN rows); retry the call     */

#define EAGLE_MAX_TREE_ROWS 64 /* T = root + up to 63 draft nodes */

/* Create-time maxima; the workspace is sized from them. */
typedef struct {
  int32_t max_batch;      /* B <= max_batch, 1..256                                */
  int32_t num_q_heads;    /* Hq                                                    */
  int32_t num_kv_heads;   /* Hkv, Hq % Hkv == 0                                    */
  int32_t head_dim;       /* D in {64, 128}                                        */
  int32_t max_tree_rows;  /* T = N + 1 <= 64                                       */
  int32_t vocab_size;     /* V >= 2                                                */
  eagle_dtype kv_dtype;     /* dtype of q, k and v                                 */
  eagle_dtype logits_dtype; /* dtype of target and draft logits                    */
} eagle_verify_desc;

/* Tree attention (one layer).
 *   q         [B, T, Hq, D]             queries of the tree nodes (kv_dtype)
 *   k, v      [num_kv_rows, Hkv, D]     keys/values (kv_dtype); sequence b uses
 *             rows kv_indptr[b] .. kv_indptr[b] + L_b + T - 1: its L_b prefix
 *             rows followed by the T tree-node rows in node order (the tree's
 *             own K/V, appended by the verification forward before the cache
 *             is truncated to the accepted path)
 *   kv_indptr [B+1] int64 (device)      first KV row of each sequence
 *   prefix_lens_host [B] int32 (host)   L_b >= 0, used to plan the launch
 *   parents   [B, T] int32 (device)     parents[b,0] = -1, 0 <= parents[b,i] < i
 *   sm_scale  softmax scale (1/sqrt(D) by convention)
 *   out       [B, T, Hq, D] float32     O[b,i,h] = sum_j softmax_j(scale q.k_j) v_j over
 *             prefix rows and the tree rows of the nodes on the root path of i
 *             (i included); query head h reads KV head h / (Hq/Hkv)
 *   flags     [B] uint32 (device)       EAGLE_FLAG_BAD_TREE | EAGLE_FLAG_BAD_KV_RANGE
 * Paged K/V (page_size > 0; a serving engine's block tables): k and v hold
 * num_kv_rows / page_size pages of page_size rows each, and sequence b's
 * logical row x (its L_b prefix rows, then its T tree rows) is physical row
 *   page_table[b * pages_per_seq + x / page_size] * page_size + x % page_size.
 * kv_indptr is then not read (may be NULL).  page_size must be a multiple of
 * 64 (one 64-key tile never spans two pages) dividing num_kv_rows, and
 * pages_per_seq >= ceil((L_b + T) / page_size) for every b (EAGLE_ERR_ARG
 * otherwise); a table entry outside [0, num_kv_rows / page_size) flags the
 * sequence EAGLE_FLAG_BAD_KV_RANGE (poisoned, nothing read out of bounds).
 * page_size == 0: the contiguous layout above.
 * Inputs are not modified.  Keys/values are read once from HBM per launch.
 * Long prefixes are split into key chunks whose partial results are merged by
 * log-sum-exp; on the bf16 path the merge runs inside the attention kernel
 * when all of its workgroups fit on the device at once (they then wait for
 * each other), otherwise as a second kernel.  Calls on one handle must not
 * overlap: they share the workspace. */
typedef struct {
  int32_t batch;           /* B <= max_batch            */
  int32_t tree_rows;       /* T <= max_tree_rows, >= 1  */
  int64_t num_kv_rows;     /* rows allocated in k and v */
  const void* q;
  const void* k;
  const void* v;
  const int64_t* kv_indptr;
  const int32_t* prefix_lens_host;
  const int32_t* parents;
  float sm_scale;
  float* out;
  uint32_t* flags;
  const int32_t* page_table; /* [B, pages_per_seq] int32 (device), paged K/V only */
  int32_t page_size;         /* 0: contiguous K/V; else rows per page, a multiple of 64 */
  int32_t pages_per_seq;     /* row stride of page_table */
} eagle_tree_attention_args;

/* Multi-round speculative sampling over the vocabulary.
 *   target_logits [B, T, V]  row n: the target's next-token logits after node n
 *   draft_logits  [B, T, V]  row n: the draft logits that proposed n's children
 *                            (rows of nodes without children are never read;
 *                            not read at all when temperature == 0)
 *   parents [B, T] int32, tokens [B, T] int32 (tokens[b,0] = the already
 *            committed root token, unused)
 *   Trees of different sizes share a batch by padding: rows i >= 1 whose
 *   token is -1 are padding.  They must form a suffix of the T rows (else
 *   EAGLE_FLAG_BAD_TREE), keep a valid parent, are never children and their
 *   logits rows are never read; the result is that of the tree without them.
 *   temperature  > 0: q = softmax(target/t), p = softmax(draft/t);
 *                == 0: greedy — accept the first child whose token is the
 *                target argmax (lowest id on ties), else emit that argmax.
 *   without_replacement  1: the siblings of a node were drawn from its draft
 *                distribution without replacement (the k sampled children of
 *                the EAGLE notes page, core mechanism), so sibling i is tested
 *                against that distribution with the earlier siblings' tokens
 *                removed and renormalised, and the residual update uses the
 *                same distribution (a repeated token has probability 0 there:
 *                accepted iff the residual keeps mass on it); 0: i.i.d.
 *                siblings, every sibling against the parent's draft row.
 *                Ignored when temperature == 0.
 *   top_k, top_p filtered distributions (the request's sampling filters):
 *                with temperature > 0, q and p are both replaced by their
 *                filtered and renormalised versions before the walk, and the
 *                children must have been drawn from the filtered draft.
 *                top_k > 0 keeps the tokens whose logit is at least the
 *                top_k-th largest of the row (ties at that value all kept;
 *                top_k = 0 or >= V keeps everything).  top_p in (0, 1) then
 *                keeps, among those, every token whose strictly larger
 *                logits hold less than top_p of their mass (0 or 1: off).
 *                A row whose nucleus boundary lies within 1e-6 of its mass
 *                target adds a near tie to its node's decisions.  The
 *                result is lossless for the filtered target (a rejection
 *                never emits a filtered-out token).  Ignored when
 *                temperature == 0 (the argmax is never filtered out).
 *   seed, offset Philox4x32-10 key / per-step counter word: the uniform for the
 *                test of the i-th child (0-based) of node n in sequence b uses
 *                counter (i, n | b << 8, offset_lo, offset_hi), key (seed_lo,
 *                seed_hi), and u = (x0 >> 8) * 2^-24; the terminal sample of
 *                node n uses slot i = 0xffffffff.  Samples are inverse-CDF over
 *                ascending token ids.
 * Outputs (device):
 *   accept_len [B]        number of accepted draft nodes (-1 if poisoned)
 *   accepted_nodes [B, T] accepted node indices along the root path, -1 padded
 *   out_tokens [B, T]     tokens of the accepted nodes, then one final token
 *                         (residual sample or bonus), -1 padded
 *   flags [B]             EAGLE_FLAG_* bits
 *   near_ties [B]         decisions on the walk within 1e-6 of their threshold
 *                         (|r - q_res(t)/p(t)| or |running sum - u*total|/total) */
typedef struct {
  int32_t batch;
  int32_t tree_rows;
  const void* target_logits;
  const void* draft_logits;
  const int32_t* parents;
  const int32_t* tokens;
  float temperature;
  uint64_t seed;
  uint64_t offset;
  int32_t* accept_len;
  int32_t* accepted_nodes;
  int32_t* out_tokens;
  uint32_t* flags;
  int32_t* near_ties;
  int32_t without_replacement; /* 0 or 1, see above */
  int32_t top_k;               /* >= 0, 0 = off, see above */
  float top_p;                 /* [0, 1], 0 or 1 = off, see above */
} eagle_spec_accept_args;

/* Commit the accepted path into the KV cache, in place (lesson page, the
 * "KV cache rollback" section and build step 4, KV accounting).  For
 * sequence b with n = accept_len[b] (spec_accept's outputs):
 *   row kv_indptr[b] + L_b + i receives what row kv_indptr[b] + L_b + path_i
 *   held before the call, i = 0 .. n, with path_0 = 0 (the root: the token
 *   the previous step emitted, whose K/V this step computed) and
 *   path_i = accepted_nodes[b, i-1]; rows of rejected nodes are left as
 *   they are (rolled back by the length alone)
 *   new_lens[b] = L_b + n + 1, the rows that now hold committed tokens (the
 *   step's final token gets its row from the next forward, as its root)
 * accept_len < 0 (a poisoned sequence) commits the root only.  A path that is
 * not strictly increasing inside [1, T) moves nothing: new_lens[b] = L_b + 1,
 * flags[b] = EAGLE_FLAG_BAD_TREE.  kv_indptr[b..b+1] not holding L_b + T rows
 * inside [0, num_kv_rows): nothing moves, new_lens[b] = -1, flags[b] =
 * EAGLE_FLAG_BAD_KV_RANGE.  Otherwise flags[b] = 0.
 *   k, v             [num_kv_rows, Hkv, D] (kv_dtype), device, modified
 *   kv_indptr        [B+1] int64 (device)
 *   prefix_lens_host [B] int32 (host), L_b >= 0
 *   accept_len       [B] int32 (device)
 *   accepted_nodes   [B, T] int32 (device)
 *   new_lens         [B] int32 (device, written)
 *   flags            [B] uint32 (device, written)
 *   num_layers       >= 1: the same commit is applied to every layer's cache
 *   layer_stride     elements from one layer's k (and v) to the next's;
 *                    >= num_kv_rows * Hkv * D when num_layers > 1
 * One launch covers every layer.  Every moving row is read before any is
 * written, so a path whose sources and destinations overlap is safe.
 * Paged K/V (page_size > 0): rows are logical rows of the sequence, mapped
 * through page_table exactly as for eagle_verify_tree_attention (kv_indptr
 * not read); the moves happen between the physical rows.
 * Nothing else may touch k or v while the call runs. */
typedef struct {
  int32_t batch;           /* B <= max_batch            */
  int32_t tree_rows;       /* T <= max_tree_rows, >= 1  */
  int64_t num_kv_rows;     /* rows allocated in k and v */
  void* k;
  void* v;
  const int64_t* kv_indptr;
  const int32_t* prefix_lens_host;
  const int32_t* accept_len;
  const int32_t* accepted_nodes;
  int32_t* new_lens;
  uint32_t* flags;
  int32_t num_layers;
  int64_t layer_stride;
  const int32_t* page_table; /* [B, pages_per_seq] int32 (device), paged K/V only */
  int32_t page_size;         /* 0: contiguous K/V; else rows per page, a multiple of 64 */
  int32_t pages_per_seq;
} eagle_kv_commit_args;

/* One expansion step of a dynamic draft tree (EAGLE notes page, the EAGLE-2
 * section: the draft's confidence tracks the acceptance rate, so the tree
 * grows where a path's cumulative confidence is high; the tree-drafting
 * section: greedy drafting takes each node's top-k children).  For sequence b:
 *   frontier node f has value s_f = scores[b, f] (log-probability of its
 *   path; not > -inf (including NaN): inactive) and draft logits
 *   draft_logits[b, f, :]; p_f = softmax(logits / temperature)
 *   candidates: each active node's top_k most probable tokens (largest logit
 *   first, ties to the lower id), valued s_f + log p_f(token)
 *   kept: the `keep` candidates of largest value, in that order, ties to the
 *   lower frontier index, then the lower token id
 * Outputs (device): parent/token/value [B, keep] (frontier index, token id,
 * value as float32; -1, -1, -inf past the last candidate), flags [B]
 * (EAGLE_FLAG_NONFINITE when an active row holds NaN/+inf or is all -inf:
 * that node is skipped), near_ties [B] (ranking decisions, up to the boundary
 * between kept and dropped, between values less than 1e-6 apart; equal
 * logits of one row are exact ties and not counted).  Values are computed in
 * fp64 from fp32 exponentials summed in fp64.
 * Limits: frontier <= max_tree_rows, 1 <= top_k <= 16, 1 <= keep <= 64,
 * vocab_size <= 64 * 8192. */
typedef struct {
  int32_t batch;           /* B <= max_batch                 */
  int32_t frontier;        /* F rows per sequence            */
  const void* draft_logits;/* [B, F, V] logits_dtype         */
  const float* scores;     /* [B, F] float32                 */
  float temperature;       /* > 0                            */
  int32_t top_k;
  int32_t keep;
  int32_t* parent;
  int32_t* token;
  float* value;
  uint32_t* flags;
  int32_t* near_ties;
} eagle_tree_expand_args;

/* The final draft tree from chained expansion steps (EAGLE notes page, the
 * EAGLE-2 section: nodes are kept by the cumulative confidence of their
 * paths).  parent/token/value [steps, B, keep] hold the outputs of `steps`
 * calls of eagle_verify_tree_expand: step 0 expanded the root (its parents
 * are 0), step d > 0 expanded step d-1's kept list (its parents index that
 * list); parent -1 = no candidate.  The `nodes` candidates of largest value
 * are kept, ties to the earlier step, then the better rank; a node's value
 * never exceeds its parent's, so every kept node's parent is kept.
 * Outputs (device): parents/tokens [B, nodes + 1]: row 0 the root (parent -1,
 * token root_tokens[b]), then the kept nodes in (step, rank) order, parents
 * before children (the layout tree_attention and spec_accept read); rows
 * past the last kept node are padding rows (parent 0, token -1), which both
 * calls accept as a tree of rows[b] rows; rows [B] = 1 + kept nodes.
 * Limits: steps <= 64, keep <= 64, nodes + 1 <= max_tree_rows. */
typedef struct {
  int32_t batch;
  int32_t steps;
  int32_t keep;
  int32_t nodes;
  const int32_t* parent;
  const int32_t* token;
  const float* value;
  const int32_t* root_tokens;
  int32_t* parents;
  int32_t* tokens;
  int32_t* rows;
} eagle_tree_rerank_args;

/* Launch plan of one tree-attention call (what eagle_verify_tree_attention
 * will launch for these arguments). */
typedef struct {
  int32_t path;            /* 0 = fp32/FMA kernel, 1 = bf16 MFMA kernel          */
  int32_t rows_per_kv_head;/* R = T * Hq / Hkv                                   */
  int32_t row_tiles;       /* workgroups along R per (sequence, split, KV head)  */
  int32_t rows_per_tile;   /* rows one workgroup covers                          */
  int32_t chunk_keys;      /* prefix keys per split                              */
  int32_t total_splits;    /* sum over sequences of the split counts             */
  int32_t workgroups;      /* attention workgroups launched                      */
  int32_t merge_workgroups;/* workgroups of a separate LSE merge (0 = one split  *
                            * per sequence); not launched when the merge runs   *
                            * inside the attention kernel                       */
  int32_t merge_in_kernel; /* 1: the splits merge inside the attention kernel.  *
                            * Decided per call from the device's capacity, so   *
                            * it is only known for a handle's last call; the    *
                            * descriptor-only check reports 0                   */
} eagle_attention_plan;

/* Multi-round speculative sampling without a handle and without any device
 * allocation, for callers that cannot allocate: code that is captured into a
 * HIP graph, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, kernels and results as eagle_verify_spec_accept (bit-identical
 * outputs for the same inputs), with the create-time descriptor passed per
 * call (`desc` maxima are checked, V and the logits dtype are read; the q/kv
 * fields are validated but unused).  The kernels' scratch lives in a fixed
 * 8 MiB array in device memory that the library holds on every GPU it runs
 * on until the process ends; each call first clears the part it uses with a
 * kernel on `hip_stream`.  A call whose scratch does not fit (it grows with
 * batch x tree_rows x ceil(V / 8192): e.g. 64 sequences of 64 rows fit at
 * V = 32000, 32 at V = 128256) returns EAGLE_ERR_CAPACITY before any launch.
 * Calls that overlap on one GPU share that array and race: serialise them.
 * Errors: as eagle_verify_spec_accept; the message is read with
 * eagle_verify_last_error(NULL). */
EAGLE_API eagle_status eagle_verify_spec_accept_noalloc(const eagle_verify_desc* desc,
                                                        const eagle_spec_accept_args* a, void* hip_stream);

/* Allocate a handle and its workspace on the current HIP device.
 * Errors: EAGLE_ERR_ARG (bad descriptor), EAGLE_ERR_HIP, EAGLE_ERR_OOM.
 * On error *out is set to NULL. */
EAGLE_API eagle_status eagle_verify_create(const eagle_verify_desc* desc, eagle_verify** out);

/* Tree-masked attention, see eagle_tree_attention_args. */
EAGLE_API eagle_status eagle_verify_tree_attention(eagle_verify* h, const eagle_tree_attention_args* a,
                                         void* hip_stream);

/* Multi-round speculative sampling, see eagle_spec_accept_args. */
EAGLE_API eagle_status eagle_verify_spec_accept(eagle_verify* h, const eagle_spec_accept_args* a,
                                      void* hip_stream);

/* Commit of the accepted path into the KV cache, see eagle_kv_commit_args.
 * Errors: EAGLE_ERR_ARG / EAGLE_ERR_CAPACITY (bad arguments, nothing
 * launched), EAGLE_ERR_HIP (launch failed). */
EAGLE_API eagle_status eagle_verify_kv_commit(eagle_verify* h, const eagle_kv_commit_args* a, void* hip_stream);

/* One dynamic draft-tree expansion step, see eagle_tree_expand_args.
 * Errors: EAGLE_ERR_ARG / EAGLE_ERR_CAPACITY / EAGLE_ERR_UNSUPPORTED (nothing
 * launched), EAGLE_ERR_HIP (launch failed).  Shares the handle's workspace:
 * calls on one handle must not overlap. */
EAGLE_API eagle_status eagle_verify_tree_expand(eagle_verify* h, const eagle_tree_expand_args* a, void* hip_stream);

/* Final draft tree from chained expansion steps, see eagle_tree_rerank_args. */
EAGLE_API eagle_status eagle_verify_tree_rerank(eagle_verify* h, const eagle_tree_rerank_args* a, void* hip_stream);

/* Synchronise the last stream the handle used, free the workspace and the
 * handle.  NULL is accepted. */
EAGLE_API eagle_status eagle_verify_destroy(eagle_verify* h);

/* Text of the last error on this handle ("" if none); a thread-local
 * message is returned for h == NULL (e.g. after a failed create). */
EAGLE_API const char* eagle_verify_last_error(const eagle_verify* h);

/* Validate arguments exactly as the calls above do and report the launch
 * plan, without touching the device (no HIP call is made).  `desc` is the
 * descriptor the handle was (or would be) created with. */
EAGLE_API eagle_status eagle_verify_check_tree_attention(const eagle_verify_desc* desc,
                                               const eagle_tree_attention_args* a,
                                               eagle_attention_plan* plan);
EAGLE_API eagle_status eagle_verify_check_spec_accept(const eagle_verify_desc* desc,
                                            const eagle_spec_accept_args* a);
EAGLE_API eagle_status eagle_verify_check_kv_commit(const eagle_verify_desc* desc, const eagle_kv_commit_args* a);
EAGLE_API eagle_status eagle_verify_check_tree_expand(const eagle_verify_desc* desc, const eagle_tree_expand_args* a);
EAGLE_API eagle_status eagle_verify_check_tree_rerank(const eagle_verify_desc* desc, const eagle_tree_rerank_args* a);

/* Kernels of the last successful eagle_verify_spec_accept call on h, as a
 * bitwise OR of the values below (a batch larger than the fused kernel's
 * co-resident capacity runs in slices, and a slice that cannot be made
 * resident falls back to the three-kernel path, so a call can use both):
 *   EAGLE_ACCEPT_PATH_THREE_KERNEL  statistics, pass and final kernels;
 *   EAGLE_ACCEPT_PATH_FUSED         one co-resident kernel per slice;
 *   EAGLE_ACCEPT_PATH_NODE_PARALLEL one workgroup per node, then one per
 *                                   sequence (vocabularies up to 32768).
 * Every path applies the same rule; their sums run in different orders, so
 * their results can differ only where a near tie is reported (near_ties).
 * No HIP call is made.
 * Errors: EAGLE_ERR_ARG when h or paths is NULL or h has made no such call. */
enum {
  EAGLE_ACCEPT_PATH_THREE_KERNEL = 1,
  EAGLE_ACCEPT_PATH_FUSED = 2,
  EAGLE_ACCEPT_PATH_NODE_PARALLEL = 4
};
EAGLE_API eagle_status eagle_verify_last_accept_paths(const eagle_verify* h, int* paths);

/* Launch plan of the last successful eagle_verify_tree_attention call on h
 * (merge_in_kernel included).  No HIP call is made.
 * Errors: EAGLE_ERR_ARG when h or plan is NULL or h has made no such call. */
EAGLE_API eagle_status eagle_verify_last_attention_plan(const eagle_verify* h, eagle_attention_plan* plan);

/* Diagnostic phase timeline of the two step kernels (for profiling; the
 * results of every call are the same with or without it).
 *
 * device_words: caller-owned device memory of num_words 64-bit words, kept
 * alive while calls on h may use it; NULL (or num_words 0) switches the
 * timeline off.  While it is set, every MFMA tree-attention launch and every
 * fused acceptance launch on h whose workgroups need at most num_words words
 * (32 per workgroup) records: thread 0 of workgroup w writes word w * 32 + k
 * at phase k, as a reading of the device's constant-rate real-time counter
 * (100 MHz on MI355X).  Nothing is cleared: a phase a workgroup does not
 * reach keeps the word's old value, so the caller clears the buffer before a
 * call.  A call of several fused launches (a batch cut into slices) leaves
 * the last launch's words.  Other kernels record nothing.
 *   tree attention (workgroup = (KV head, key split, row tile)):
 *     0 start, 1 parent array and query rows landed (the first K/V tile
 *     may still be in flight), 2 ancestor words built, 3 tile loop done, 4 partial (or final) rows stored, 5 row
 *     statistics published (in-kernel merge only), 6 every split of the rows
 *     it merges has arrived, 7 merged rows written; word 30 = tiles of the
 *     workgroup, 31 = split | KV head << 16 | row tile << 32 | sequence << 48
 *   acceptance (workgroup = (sequence, node, vocabulary chunk)):
 *     0 start, 1 chunk in LDS, 2 chunk statistics, 3 row statistics
 *     combined, 4 first decision, 5 + i end of residual round i (i < 12),
 *     17 node decided, 18 terminal preparation starts, 19 the chunk holding
 *     the terminal sample is known, 20 the walk ends at this node, 21
 *     outputs written; word 30 = residual rounds, 31 = node | chunk << 8 |
 *     node state << 16 | sequence << 24
 * Errors: EAGLE_ERR_ARG when h is NULL, num_words < 0, or device_words is
 * not 8-byte aligned. */
EAGLE_API eagle_status eagle_verify_set_timeline(eagle_verify* h, uint64_t* device_words, int64_t num_words);

#ifdef __cplusplus
}
#endif

#endif /* EAGLE_VERIFY_H_ */
