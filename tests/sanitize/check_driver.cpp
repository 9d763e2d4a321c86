// Host-side argument validation and launch planning (plan.cpp) under
// AddressSanitizer and UndefinedBehaviorSanitizer: every check entry point
// is called with seeded random descriptors and arguments (valid, borderline
// and invalid: null and misaligned pointers, out-of-range sizes, huge
// prefixes, paged layouts), and the plans it accepts are checked for
// internal consistency.  Exit status 0 = no finding and every plan sound.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "../../eagle_draft_tree_attention_amd/csrc/ev_internal.h"

namespace {

std::mt19937_64 rng(12345);
int pick(int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); }
bool coin(double p) { return std::uniform_real_distribution<double>(0, 1)(rng) < p; }

const void* ptr(bool aligned = true) {
  static char buf[64];
  uintptr_t a = (reinterpret_cast<uintptr_t>(buf) + 31) & ~uintptr_t(31);
  if (coin(0.03)) return nullptr;
  return reinterpret_cast<const void*>(aligned && !coin(0.03) ? a : a + 2);
}

int failures = 0;
void expect(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "plan inconsistency: %s\n", what);
    ++failures;
  }
}

}  // namespace

int main() {
  char err[512];
  for (int it = 0; it < 20000; ++it) {
    eagle_verify_desc d;
    d.max_batch = coin(0.05) ? pick(-2, 300) : pick(1, 64);
    d.num_kv_heads = pick(1, 16);
    d.num_q_heads = d.num_kv_heads * (coin(0.05) ? pick(0, 3) : pick(1, 8)) + (coin(0.03) ? 1 : 0);
    d.head_dim = coin(0.9) ? (coin(0.5) ? 64 : 128) : pick(0, 256);
    d.max_tree_rows = coin(0.05) ? pick(-1, 70) : pick(1, 64);
    d.vocab_size = coin(0.05) ? pick(-5, 3) : pick(2, 600000);
    d.kv_dtype = static_cast<eagle_dtype>(coin(0.97) ? pick(0, 1) : 7);
    d.logits_dtype = static_cast<eagle_dtype>(coin(0.97) ? pick(0, 1) : 9);
    (void)ev::check_desc(&d, err, sizeof(err));

    const int B = coin(0.05) ? pick(-1, 300) : pick(1, std::max(1, std::min(d.max_batch, 64)));
    const int T = coin(0.05) ? pick(-1, 70) : pick(1, std::max(1, std::min(d.max_tree_rows, 64)));
    std::vector<int32_t> lens(B > 0 ? B : 1);
    int64_t total = 0;
    for (auto& L : lens) {
      L = coin(0.02) ? -pick(1, 5) : (coin(0.1) ? pick(0, 300000) : pick(0, 9000));
      total += L > 0 ? L : 0;
    }
    eagle_tree_attention_args a{};
    a.batch = B;
    a.tree_rows = T;
    a.num_kv_rows = coin(0.05) ? pick(-3, 1000) : total + static_cast<int64_t>(B > 0 ? B : 0) * (T > 0 ? T : 0) +
                                                     pick(0, 100);
    a.q = ptr();
    a.k = ptr();
    a.v = ptr();
    a.kv_indptr = static_cast<const int64_t*>(ptr());
    a.prefix_lens_host = coin(0.02) ? nullptr : lens.data();
    a.parents = static_cast<const int32_t*>(ptr());
    a.sm_scale = coin(0.03) ? -1.0f : 0.088f;
    a.out = static_cast<float*>(const_cast<void*>(ptr()));
    a.flags = static_cast<uint32_t*>(const_cast<void*>(ptr()));
    std::vector<int32_t> table;
    if (coin(0.3)) {
      a.page_size = coin(0.9) ? 64 * pick(1, 8) : pick(-64, 200);
      a.pages_per_seq = pick(0, 400);
      if (a.page_size > 0) a.num_kv_rows = (a.num_kv_rows / a.page_size + 1) * a.page_size;
      table.resize(static_cast<size_t>(B > 0 ? B : 1) * (a.pages_per_seq > 0 ? a.pages_per_seq : 1));
      a.page_table = coin(0.03) ? nullptr : table.data();
    }
    ev::AttnPlan plan;
    if (ev::plan_tree_attention(&d, &a, ev::kDefaultCUs, &plan, err, sizeof(err)) == EAGLE_OK) {
      expect(plan.total_splits >= a.batch, "a split per sequence at least");
      expect(plan.split_base[a.batch] == plan.total_splits, "split bases end at the total");
      expect(plan.workgroups >= plan.total_splits, "workgroups cover the splits");
      expect(plan.chunk % ev::kTileKeys == 0 && plan.chunk > 0, "chunk is whole tiles");
      expect(plan.rows_per_tile * plan.row_tiles >= plan.R, "row tiles cover the rows");
      for (int b = 0; b < a.batch; ++b) {
        const int64_t S = plan.split_base[b + 1] - plan.split_base[b];
        expect(S >= 1 && S * plan.chunk >= lens[b], "splits cover the prefix");
      }
    }
    eagle_spec_accept_args s{};
    s.batch = B;
    s.tree_rows = T;
    s.target_logits = ptr();
    s.draft_logits = ptr();
    s.parents = static_cast<const int32_t*>(ptr());
    s.tokens = static_cast<const int32_t*>(ptr());
    s.temperature = coin(0.05) ? -0.5f : (coin(0.2) ? 0.f : 0.7f);
    s.accept_len = static_cast<int32_t*>(const_cast<void*>(ptr()));
    s.accepted_nodes = static_cast<int32_t*>(const_cast<void*>(ptr()));
    s.out_tokens = static_cast<int32_t*>(const_cast<void*>(ptr()));
    s.flags = static_cast<uint32_t*>(const_cast<void*>(ptr()));
    s.near_ties = static_cast<int32_t*>(const_cast<void*>(ptr()));
    s.without_replacement = coin(0.03) ? 2 : pick(0, 1);
    s.top_k = coin(0.03) ? -1 : pick(0, 100);
    s.top_p = coin(0.03) ? 1.5f : static_cast<float>(pick(0, 10)) / 10.f;
    (void)ev::check_spec_accept(&d, &s, err, sizeof(err));

    eagle_kv_commit_args c{};
    c.batch = B;
    c.tree_rows = T;
    c.num_kv_rows = a.num_kv_rows;
    c.k = const_cast<void*>(ptr());
    c.v = const_cast<void*>(ptr());
    c.kv_indptr = a.kv_indptr;
    c.prefix_lens_host = a.prefix_lens_host;
    c.accept_len = static_cast<const int32_t*>(ptr());
    c.accepted_nodes = static_cast<const int32_t*>(ptr());
    c.new_lens = static_cast<int32_t*>(const_cast<void*>(ptr()));
    c.flags = static_cast<uint32_t*>(const_cast<void*>(ptr()));
    c.num_layers = coin(0.05) ? pick(-1, 0) : pick(1, 80);
    c.layer_stride = coin(0.05) ? 1 : (c.num_kv_rows + 1) * d.num_kv_heads * d.head_dim;
    c.page_table = a.page_table;
    c.page_size = a.page_size;
    c.pages_per_seq = a.pages_per_seq;
    (void)ev::check_kv_commit(&d, &c, err, sizeof(err));

    eagle_tree_expand_args e{};
    e.batch = B;
    e.frontier = coin(0.05) ? pick(-1, 80) : pick(1, 64);
    e.draft_logits = ptr();
    e.scores = static_cast<const float*>(ptr());
    e.temperature = coin(0.05) ? 0.f : 1.f;
    e.top_k = pick(-1, 20);
    e.keep = pick(-1, 70);
    e.parent = static_cast<int32_t*>(const_cast<void*>(ptr()));
    e.token = static_cast<int32_t*>(const_cast<void*>(ptr()));
    e.value = static_cast<float*>(const_cast<void*>(ptr()));
    e.flags = static_cast<uint32_t*>(const_cast<void*>(ptr()));
    e.near_ties = static_cast<int32_t*>(const_cast<void*>(ptr()));
    (void)ev::check_tree_expand(&d, &e, err, sizeof(err));

    eagle_tree_rerank_args r{};
    r.batch = B;
    r.steps = pick(-1, 70);
    r.keep = pick(-1, 70);
    r.nodes = pick(-1, 70);
    r.parent = static_cast<const int32_t*>(ptr());
    r.token = static_cast<const int32_t*>(ptr());
    r.value = static_cast<const float*>(ptr());
    r.root_tokens = static_cast<const int32_t*>(ptr());
    r.parents = static_cast<int32_t*>(const_cast<void*>(ptr()));
    r.tokens = static_cast<int32_t*>(const_cast<void*>(ptr()));
    r.rows = static_cast<int32_t*>(const_cast<void*>(ptr()));
    (void)ev::check_tree_rerank(&d, &r, err, sizeof(err));
  }
  std::printf("20000 rounds, %d plan inconsistencies\n", failures);
  return failures ? 1 : 0;
}
