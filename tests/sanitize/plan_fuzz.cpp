// plan_fuzz.cpp -- randomized driver of the host planner, built with the address
// and undefined-behaviour sanitizers by tests/test_plan_sanitize.py (host code
// only: the planner has no HIP dependency).
//
// Each case draws a configuration (heads, head dim, page size, dtype switches,
// causal, window, grid per kernel kind) and a batch of block rows (single format
// or a shared-prefix composition), plans it, and checks the blob's structure:
// offsets inside the blob, queues that partition the items and merge tasks,
// merge sources that name written partial rows, and chunks inside their rows.
// Any sanitizer report or failed check ends the process with a non-zero status.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <string>
#include <vector>

#include "bsr_attn.h"
#include "plan.h"

using namespace bsr;

#define CHECK(cond)                                                              \
  do {                                                                           \
    if (!(cond)) {                                                               \
      std::fprintf(stderr, "case %d: check failed: %s (line %d)\n", c, #cond, __LINE__); \
      return 1;                                                                  \
    }                                                                            \
  } while (0)

int main(int argc, char** argv) {
  const int cases = argc > 1 ? std::atoi(argv[1]) : 2000;
  const unsigned seed = argc > 2 ? static_cast<unsigned>(std::atoi(argv[2])) : 1u;
  std::mt19937 rng(seed);
  auto pick = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
  int planned = 0;
  for (int c = 0; c < cases; ++c) {
    PlanConfig cfg;
    const int hkv_opts[] = {1, 2, 4, 8};
    const int g_opts[] = {1, 2, 4, 8, 16};
    const int d_opts[] = {64, 128, 256};
    const int p_opts[] = {1, 2, 3, 5, 16, 64};
    cfg.h_kv = hkv_opts[pick(0, 3)];
    cfg.group = g_opts[pick(0, 4)];
    cfg.h_qo = cfg.h_kv * cfg.group;
    cfg.head_dim = d_opts[pick(0, 2)];
    cfg.page_size = p_opts[pick(0, 5)];
    cfg.bf16 = pick(0, 3) != 0;
    cfg.kv8 = cfg.bf16 && pick(0, 4) == 0;
    cfg.cap = pick(0, 1) == 1;
    const bool composable = pick(0, 4) == 0;
    cfg.causal = !composable && pick(0, 1) == 1;
    cfg.window = (!composable && pick(0, 3) == 0) ? pick(1, 3000) : 0;
    const int nwg = pick(1, 96);
    for (int k = 0; k < 4; ++k)
      for (int r = 0; r < 2; ++r) cfg.num_wg[k][r][0] = cfg.num_wg[k][r][1] = nwg;
    if (!composable && pick(0, 3) == 0) {
      cfg.alibi_raw.resize(cfg.h_qo);
      for (float& a : cfg.alibi_raw) a = 0.01f * pick(-100, 100);
    }
    cfg.cus = pick(0, 1) ? nwg / 2 : 0;
    cfg.slot2_speed16 = pick(8, 16);
    cfg.static_queues = pick(0, 1) == 1;
    cfg.mfma_w16 = pick(16, 400);
    cfg.gamma = pick(0, 1024);
    cfg.min_chunk = 64 * pick(1, 4);
    cfg.max_batch = 1 << 20;
    cfg.max_total_qo = 1 << 24;
    cfg.max_total_kv = int64_t(1) << 34;
    cfg.max_partial_rows = int64_t(1) << 30;
    cfg.blob_capacity = int64_t(1) << 30;

    std::vector<BlockRow> rows;
    int32_t total_qo = 0;
    if (!composable) {
      const int batch = pick(0, 24);
      int32_t page = 0;
      for (int r = 0; r < batch; ++r) {
        BlockRow b;
        b.qo_begin = total_qo;
        b.qo_len = pick(0, 4) == 0 ? pick(0, 300) : pick(0, 3);
        b.kv_len = pick(0, 3) == 0 ? pick(0, 20000) : pick(0, 900);
        if (cfg.causal && b.kv_len < b.qo_len) b.kv_len = b.qo_len;
        b.page_begin = page;
        page += (b.kv_len + cfg.page_size - 1) / cfg.page_size;
        total_qo += b.qo_len;
        rows.push_back(b);
      }
    } else {
      const int branches = pick(1, 40);
      const int prefix = cfg.page_size * pick(0, 200);
      total_qo = branches;
      BlockRow p;
      p.qo_begin = 0;
      p.qo_len = branches;
      p.kv_len = prefix;
      p.page_begin = 0;
      p.format = 0;
      rows.push_back(p);
      int32_t page = prefix / cfg.page_size;
      for (int b = 0; b < branches; ++b) {
        BlockRow s;
        s.qo_begin = b;
        s.qo_len = 1;
        s.kv_len = pick(0, 700);
        s.page_begin = page;
        s.format = 1;
        page += (s.kv_len + cfg.page_size - 1) / cfg.page_size;
        rows.push_back(s);
      }
    }
    // tree masks on some single-format batches (rows of at most 64 tokens)
    std::vector<uint64_t> tree;
    bool use_tree = !composable && pick(0, 3) == 0;
    for (const BlockRow& b : rows) use_tree = use_tree && b.qo_len <= kMaxTreeTokens && b.qo_len <= b.kv_len;
    if (use_tree) {
      tree.assign(total_qo, 0);
      for (BlockRow& b : rows) {
        b.tree = b.qo_len > 0;
        for (int t = 0; t < b.qo_len; ++t)
          tree[b.qo_begin + t] = (uint64_t(rng()) << 32 | rng()) | (uint64_t(1) << t);
      }
    }
    PlanResult res;
    std::string err;
    // every other case scores its candidates on threads whatever their time; the
    // plan must be the same bytes as the sequential one
    cfg.parallel_plan_us = 1e12;
    const int rc = make_plan(cfg, rows, total_qo, composable, &res, &err, use_tree ? &tree : nullptr);
    CHECK(rc == BSR_OK || rc == BSR_ERR_UNSUPPORTED || rc == BSR_ERR_CAPACITY);
    if (c % 2 == 0) {
      PlanResult par;
      std::string perr;
      cfg.parallel_plan_us = 0.0;
      const int prc = make_plan(cfg, rows, total_qo, composable, &par, &perr, use_tree ? &tree : nullptr);
      CHECK(prc == rc);
      CHECK(rc != BSR_OK || par.blob == res.blob);
    }
    if (rc != BSR_OK) continue;
    ++planned;
    CHECK(res.blob.size() >= sizeof(PlanHeader));
    PlanHeader h;
    std::memcpy(&h, res.blob.data(), sizeof(h));
    const int64_t n = static_cast<int64_t>(res.blob.size());
    CHECK(h.magic == kPlanMagic && h.blob_bytes == n);
    CHECK(h.num_wg > 0 && h.num_wg <= nwg);
    CHECK(h.spin_limit > 0);
    const int32_t offs[] = {h.off_status, h.off_claim, h.off_epochs, h.off_flags, h.off_item_ptr,
                            h.off_items, h.off_merge_ptr, h.off_merge, h.off_srcs};
    for (int32_t o : offs) CHECK(o >= static_cast<int32_t>(sizeof(PlanHeader)) && o <= n && o % 16 == 0);
    CHECK(h.off_claim + 8 <= n);
    {
      int32_t claim[2];
      std::memcpy(claim, res.blob.data() + h.off_claim, sizeof(claim));
      CHECK(claim[0] == 0 && claim[1] == 0);
    }
    CHECK(h.off_items + int64_t(h.num_items) * int64_t(sizeof(WorkItem)) <= n);
    CHECK(h.off_srcs + int64_t(h.num_srcs) * int64_t(sizeof(MergeSrc)) <= n);
    const uint8_t* base = res.blob.data();
    std::vector<int32_t> iptr(h.num_wg + 1), mptr(h.num_wg + 1);
    std::memcpy(iptr.data(), base + h.off_item_ptr, 4 * (h.num_wg + 1));
    std::memcpy(mptr.data(), base + h.off_merge_ptr, 4 * (h.num_wg + 1));
    CHECK(h.pool_begin >= 0 && h.pool_begin <= h.num_items);
    CHECK(iptr[0] == 0 && iptr[h.num_wg] == h.pool_begin);
    CHECK(!cfg.static_queues || h.pool_begin == h.num_items);
    // only tile-grid plans claim items; every queue keeps its first item
    if (h.kernel != kKindMfma) CHECK(h.pool_begin == h.num_items);
    if (h.pool_begin < h.num_items) {
      int busy = 0;
      for (int w = 0; w < h.num_wg; ++w) busy += iptr[w + 1] > iptr[w];
      CHECK(busy > 0);
    }
    CHECK(mptr[0] == 0 && mptr[h.num_wg] == h.num_merge);
    for (int w = 0; w < h.num_wg; ++w) CHECK(iptr[w] <= iptr[w + 1] && mptr[w] <= mptr[w + 1]);
    std::vector<char> flag_written(h.num_flags, 0);
    int64_t max_partial = 0;
    for (int32_t i = 0; i < h.num_items; ++i) {
      WorkItem it;
      std::memcpy(&it, base + h.off_items + int64_t(i) * sizeof(WorkItem), sizeof(it));
      CHECK(it.kv_begin >= 0 && it.kv_begin <= it.kv_end);
      CHECK(it.qo_count >= 1 && it.qo_begin >= 0 && it.qo_begin + it.qo_count <= total_qo);
      CHECK(it.kv_head >= 0 && it.kv_head < cfg.h_kv);
      if (it.tree_lo != kNoTree) CHECK(use_tree && it.tree_lo >= 0 && it.kv_end - it.tree_lo <= kMaxTreeTokens);
      if (it.flags & kItemPartial) {
        CHECK(it.flag_id >= 0 && it.flag_id < h.num_flags && it.partial_row >= 0);
        flag_written[it.flag_id] = 1;
        max_partial = std::max<int64_t>(max_partial, int64_t(it.partial_row) + int64_t(it.qo_count) * cfg.group);
      }
    }
    CHECK(max_partial == res.num_partial_rows);
    CHECK((h.off_alibi != 0) == !cfg.alibi_raw.empty());
    CHECK((h.off_tree != 0) == use_tree);
    if (h.off_alibi != 0) CHECK(h.off_alibi + 4 * int64_t(cfg.h_qo) <= n);
    if (h.off_tree != 0) CHECK(h.off_tree + 8 * int64_t(total_qo) <= n && h.off_tree % 8 == 0);
    for (int32_t t = 0; t < h.num_merge; ++t) {
      MergeTask m;
      std::memcpy(&m, base + h.off_merge + int64_t(t) * sizeof(MergeTask), sizeof(m));
      CHECK(m.src_begin >= 0 && m.src_count >= 0 && m.src_begin + m.src_count <= h.num_srcs);
      CHECK(m.qo_row >= 0 && m.qo_row < total_qo && m.kv_head >= 0 && m.kv_head < cfg.h_kv);
      for (int32_t s = 0; s < m.src_count; ++s) {
        MergeSrc src;
        std::memcpy(&src, base + h.off_srcs + int64_t(m.src_begin + s) * sizeof(MergeSrc), sizeof(src));
        CHECK(src.flag_id >= 0 && src.flag_id < h.num_flags && flag_written[src.flag_id]);
        CHECK(src.partial_row >= 0 && src.partial_row + cfg.group <= res.num_partial_rows);
      }
    }
  }
  std::printf("planned %d of %d cases\n", planned, cases);
  return planned > 0 ? 0 : 1;
}
