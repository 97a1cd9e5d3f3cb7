// plan.cpp -- deterministic host planner.
//
// Follows Core mechanism 6 of the FlashInfer explainer page (paper Algorithm 1,
// section 3.3.1, Figure 6), the query-tile rule of Core mechanism 4 (paper
// section 3.2.2), and the direct-write rule of Core mechanism 7 (paper
// Appendix D.2):
//   1. pick the query tile: the decode body when every block row folds into at
//      most 8 rows (GQA heads folded into the query dimension), otherwise the
//      smallest MFMA tile that is at least the mean folded query length;
//   2. one work unit per (block row, KV head, query tile), with the KV length it
//      actually reads (causally clipped);
//   3. L_kv = ceil(sum of unit KV lengths / #workgroups), rounded up to the KV
//      granule and at least the minimum chunk;
//   4. units longer than L_kv are cut into equal chunks of at most L_kv; only
//      those write partial states, the rest write O/LSE directly;
//   5. cost = alpha * rows + beta * KV tokens (+ gamma, a fixed per-item cost
//      that models pipeline fill and drain; an extension of the pages' model;
//      when one grid runs both bodies, an MFMA unit's tokens are weighted by the
//      measured ratio of the two bodies' time per token, and L_kv is counted in
//      weighted tokens);
//      items sorted by cost, longest first, each given to the least-loaded
//      workgroup (min-heap on (load, workgroup id)), so the plan depends on the
//      lengths only;
//   6. partial states get fixed slots; every query token whose result is split
//      gets a merge task listing its partial states in KV order (format order
//      first for composed formats), and merge tasks are spread the same way.
// Steps 4-6 are evaluated for L_kv, for L_kv / k (k <= kChunkCandidates) and as fills
// at L_kv and L_kv / 2; the
// plan with the smallest predicted makespan is kept, the pages' L_kv unless a
// finer cut is better by more than 3 % (finer cuts help when indivisible short
// units leave some workgroups over-full).  Ties are broken by creation order, so
// equal lengths give identical bytes.
#include "plan.h"

#include <algorithm>
#include <chrono>
#include <climits>
#include <cstdint>
#include <cstring>
#include <functional>
#include <new>
#include <queue>
#include <thread>
#include <utility>

#include "bsr_attn.h"

namespace bsr {

namespace {

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }
inline int32_t align16(int64_t x) { return static_cast<int32_t>(round_up(x, 16)); }

struct Unit {
  int32_t row;
  int32_t head;
  int32_t t0, nt;
  int32_t kv_lo;  // first key the unit reads (0 unless a sliding window cuts keys off)
  int32_t l_eff;  // keys the unit reads: kv_lo .. kv_lo + l_eff - 1
  int32_t causal_limit;
  int32_t window_lo;
  int32_t q_pos;    // position of the unit's first token (l_kv - l_qo + t0)
  int32_t tree_lo;  // first key of the row's tree-masked tokens, or kNoTree
  bool mfma;
  int32_t w16;  // cost of one KV token in sixteenths (16 except MFMA units of a mixed grid)
};

// KV tokens weighted by the unit's token cost.
inline int64_t weighted(const Unit& u, int64_t keys) { return (keys * u.w16 + 15) / 16; }
// Longest piece of a unit that stays within `chunk` weighted tokens.
inline int64_t unit_chunk(const Unit& u, int64_t chunk) {
  return std::max<int64_t>(kChunkGranule, chunk * 16 / u.w16 / kChunkGranule * kChunkGranule);
}

struct Item {
  WorkItem w;
  int64_t cost;
  int32_t unit;
  int32_t nchunks;
};

// Longest-first assignment: each entry, longest first, goes to the workgroup where
// it would finish first, i.e. the least-loaded one when all workgroups run at the
// same speed.  speed16[w] is workgroup w's speed in sixteenths (a workgroup of
// speed s finishes a cost c in 16 c / s); workgroups of one speed form one
// min-heap on (load, id), and the heads of the heaps are compared.  Returns the
// workgroup of each entry (indexed like costs).
void assign_longest_first(const std::vector<int64_t>& costs, const std::vector<int32_t>& speed16,
                          std::vector<int64_t>* load, std::vector<int32_t>* owner, std::vector<int32_t>* order) {
  const int32_t n = static_cast<int32_t>(costs.size());
  // longest first, ties in index order: sorted as contiguous (-cost, index) pairs
  {
    std::vector<std::pair<int64_t, int32_t>> keyed(n);
    for (int32_t i = 0; i < n; ++i) keyed[i] = {-costs[i], i};
    std::sort(keyed.begin(), keyed.end());
    order->resize(n);
    for (int32_t i = 0; i < n; ++i) (*order)[i] = keyed[i].second;
  }
  using Slot = std::pair<int64_t, int32_t>;  // (load, workgroup)
  std::vector<int32_t> speeds;  // distinct speeds, in first-seen order
  std::vector<std::vector<Slot>> heaps;  // binary min-heaps on (load, workgroup)
  for (int32_t w = 0; w < static_cast<int32_t>(load->size()); ++w) {
    size_t k = 0;
    while (k < speeds.size() && speeds[k] != speed16[w]) ++k;
    if (k == speeds.size()) {
      speeds.push_back(speed16[w]);
      heaps.emplace_back();
    }
    heaps[k].push_back({(*load)[w], w});
  }
  for (auto& h : heaps) std::make_heap(h.begin(), h.end(), std::greater<Slot>());
  // the top's load grows: move it down to its place (one pass instead of a pop
  // and a push)
  auto sift_down = [](std::vector<Slot>& h) {
    const size_t m = h.size();
    size_t i = 0;
    const Slot v = h[0];
    while (true) {
      size_t c = 2 * i + 1;
      if (c >= m) break;
      if (c + 1 < m && h[c + 1] < h[c]) ++c;
      if (!(h[c] < v)) break;
      h[i] = h[c];
      i = c;
    }
    h[i] = v;
  };
  owner->assign(n, -1);
  for (int32_t j = 0; j < n; ++j) {
    const int32_t i = (*order)[j];
    size_t best = 0;
    int64_t best_f = INT64_MAX;
    for (size_t k = 0; k < heaps.size(); ++k) {
      const Slot& top = heaps[k].front();
      const int64_t f = (top.first + costs[i]) * 16 / speeds[k];
      if (f < best_f || (f == best_f && top.second < heaps[best].front().second)) {
        best_f = f;
        best = k;
      }
    }
    Slot& s = heaps[best].front();
    (*owner)[i] = s.second;
    s.first += costs[i];
    (*load)[s.second] = s.first;
    sift_down(heaps[best]);
  }
}

// Time a workgroup needs for its load, in cost units at speed 16.
inline int64_t finish_time(int64_t load, int32_t speed16) { return load * 16 / speed16; }

struct Schedule {
  int64_t chunk = 0;
  std::vector<Item> items;
  std::vector<MergeTask> tasks;
  std::vector<MergeSrc> srcs;
  std::vector<int32_t> owner, order, mowner, morder;
  std::vector<int64_t> att_load;  // attention cost per workgroup
  int64_t partial_rows = 0;
  int32_t num_flags = 0, num_partial_items = 0;
  int64_t makespan = 0, total = 0;
};

// Steps 4-7 for one chunk length: items, direct/partial, merge map, assignment.
// fill = false: the pages' rule -- units longer than `chunk` are cut into equal
// chunks of at most `chunk`, then every item goes longest-first to the least
// loaded workgroup.  fill = true: units of at most `chunk` keys (the ones the
// pages leave whole) go longest-first to the least-loaded workgroup first; then
// each longer unit, longest first, is cut into pieces that fill the least-loaded
// workgroup up to the mean load (Stream-K-like filling, no piece below the
// minimum chunk), so indivisible short units no longer leave some workgroups
// over-full.
int schedule(const PlanConfig& cfg, const std::vector<BlockRow>& rows, const std::vector<Unit>& units,
             int64_t chunk, bool fill, int32_t nwg, const std::vector<int32_t>& speed16, int32_t total_qo,
             bool composable, Schedule* out, std::string* err) {
  (void)err;
  const int32_t g = cfg.group;
  const int32_t h_kv = cfg.h_kv;
  const int64_t min_piece = round_up(std::max(cfg.min_chunk, 1), kChunkGranule);
  auto template_of = [&](int32_t ui) {
    const Unit& u = units[ui];
    const BlockRow& r = rows[u.row];
    WorkItem w;
    std::memset(&w, 0, sizeof(w));
    w.flags = u.mfma ? kItemMfma : 0;
    w.qo_begin = r.qo_begin + u.t0;
    w.qo_count = u.nt;
    w.kv_head = u.head;
    w.page_begin = r.page_begin;
    w.causal_limit = u.causal_limit;
    w.window_lo = u.window_lo;
    w.q_pos = u.q_pos;
    w.tree_lo = u.tree_lo;
    w.partial_row = -1;
    w.flag_id = -1;
    return w;
  };
  auto item_cost = [&](int32_t ui, int64_t keys) {
    return cfg.alpha * static_cast<int64_t>(units[ui].nt) * g + cfg.beta * weighted(units[ui], keys) + cfg.gamma;
  };

  // ---- 4. chunks -> items, and 7a. their assignment --------------------------
  std::vector<Item> items;
  items.reserve(units.size() + 2 * nwg);
  std::vector<int64_t> load(nwg, 0);
  std::vector<int32_t> owner, order;
  if (!fill) {
    for (int32_t ui = 0; ui < static_cast<int32_t>(units.size()); ++ui) {
      const Unit& u = units[ui];
      WorkItem w = template_of(ui);
      if (u.l_eff == 0) {
        if (composable) continue;  // contributes no keys to the composed result
        items.push_back({w, item_cost(ui, 0), ui, 1});
        continue;
      }
      const int64_t n = ceil_div(u.l_eff, unit_chunk(u, chunk));
      const int64_t csz = n == 1 ? u.l_eff : round_up(ceil_div(u.l_eff, n), kChunkGranule);
      for (int64_t b = 0; b < u.l_eff; b += csz) {
        w.kv_begin = static_cast<int32_t>(u.kv_lo + b);
        w.kv_end = static_cast<int32_t>(u.kv_lo + std::min<int64_t>(b + csz, u.l_eff));
        items.push_back({w, item_cost(ui, w.kv_end - w.kv_begin), ui, 0});
      }
    }
    std::vector<int64_t> costs(items.size());
    for (size_t i = 0; i < items.size(); ++i) costs[i] = items[i].cost;
    assign_longest_first(costs, speed16, &load, &owner, &order);
  } else {
    std::vector<int32_t> short_u, long_u;
    int64_t total = 0;
    for (int32_t ui = 0; ui < static_cast<int32_t>(units.size()); ++ui) {
      const Unit& u = units[ui];
      if (u.l_eff == 0 && composable) continue;
      (u.l_eff <= unit_chunk(u, chunk) ? short_u : long_u).push_back(ui);
      total += item_cost(ui, u.l_eff);
    }
    // filling cuts about one piece per workgroup beyond one per long unit
    if (!long_u.empty()) total += cfg.gamma * nwg;
    auto longer = [&](int32_t a, int32_t b) {
      return weighted(units[a], units[a].l_eff) > weighted(units[b], units[b].l_eff);
    };
    std::stable_sort(short_u.begin(), short_u.end(), longer);
    std::stable_sort(long_u.begin(), long_u.end(), longer);
    // each workgroup is filled to its share of the total at its speed (all equal
    // unless the grid's workgroups run at different speeds); the heap holds
    // (load - target, workgroup), so its top is the workgroup with the most room
    int64_t sum_speed = 0;
    for (int32_t w = 0; w < nwg; ++w) sum_speed += speed16[w];
    auto target_of = [&](int32_t w) { return ceil_div(total * speed16[w], std::max<int64_t>(sum_speed, 1)); };
    using Slot = std::pair<int64_t, int32_t>;
    std::priority_queue<Slot, std::vector<Slot>, std::greater<Slot>> heap;
    for (int32_t w = 0; w < nwg; ++w) heap.push({-target_of(w), w});
    auto place = [&](int32_t ui, int64_t b, int64_t e) {
      Slot s = heap.top();
      heap.pop();
      WorkItem w = template_of(ui);
      w.kv_begin = static_cast<int32_t>(units[ui].kv_lo + b);
      w.kv_end = static_cast<int32_t>(units[ui].kv_lo + e);
      const int64_t c = item_cost(ui, e - b);
      order.push_back(static_cast<int32_t>(items.size()));
      owner.push_back(s.second);
      items.push_back({w, c, ui, 0});
      s.first += c;
      load[s.second] += c;
      heap.push(s);
    };
    for (int32_t ui : short_u) place(ui, 0, units[ui].l_eff);
    for (int32_t ui : long_u) {
      const int64_t len = units[ui].l_eff;
      int64_t pos = 0;
      while (pos < len) {
        const int64_t rem = len - pos;
        const int64_t fixed = item_cost(ui, 0);
        // room left in the least-loaded workgroup, in this unit's KV tokens
        const int64_t space =
            (-heap.top().first - fixed) * 16 / (static_cast<int64_t>(units[ui].w16) * std::max<int64_t>(cfg.beta, 1));
        // pieces round up to the granule (the rounding overshoot is absorbed by
        // workgroups that end up with no long piece) and are never tiny
        const int64_t floor_piece = std::max<int64_t>(min_piece, 4 * kChunkGranule);
        // and at most twice L_kv (the fixed item cost makes a full workgroup hold
        // a little more than L_kv keys)
        const int64_t cap = 2 * unit_chunk(units[ui], chunk);
        int64_t piece = std::min(rem, cap);
        if (piece > space) {
          piece = std::min(cap, std::max(floor_piece, round_up(std::max<int64_t>(space, 0), kChunkGranule)));
          if (rem - piece < floor_piece && rem <= cap) piece = rem;
        }
        place(ui, pos, pos + piece);
        pos += piece;
      }
    }
    // queues run in assignment order: owner/order already follow it
  }
  {
    std::vector<int32_t> count(units.size(), 0);
    for (const Item& it : items) count[it.unit] += 1;
    for (Item& it : items) it.nchunks = count[it.unit];
  }

  // ---- 5. direct write versus partial ----------------------------------------
  // (token, head) coverage counts; an item writes O/LSE directly when its unit is
  // not split and it is the only contributor for every token it covers.
  // In a single format the units partition (token, head), so only composed
  // formats need the coverage counts.
  std::vector<int32_t> cover;
  if (composable) {
    cover.assign(static_cast<size_t>(total_qo) * h_kv, 0);
    for (const Item& it : items)
      for (int32_t t = 0; t < it.w.qo_count; ++t)
        cover[static_cast<size_t>(it.w.qo_begin + t) * h_kv + it.w.kv_head] += 1;
  }
  int64_t partial_rows = 0;
  int32_t num_flags = 0, num_partial_items = 0;
  for (Item& it : items) {
    bool direct = it.nchunks == 1;
    for (int32_t t = 0; composable && direct && t < it.w.qo_count; ++t)
      direct = cover[static_cast<size_t>(it.w.qo_begin + t) * h_kv + it.w.kv_head] == 1;
    if (!direct) {
      it.w.flags |= kItemPartial;
      it.w.partial_row = static_cast<int32_t>(partial_rows);
      it.w.flag_id = num_flags++;
      partial_rows += static_cast<int64_t>(it.w.qo_count) * g;
      ++num_partial_items;
    }
  }

  // ---- 6. merge map ----------------------------------------------------------
  // A (token, head) needs a merge task unless a direct item wrote it; its sources
  // are the partial states covering it, in item creation order (format, then KV
  // order).  Built as a flat CSR over (token, head).
  const size_t nkeys = (num_partial_items > 0 || composable) ? static_cast<size_t>(total_qo) * h_kv : 0;
  std::vector<int32_t> src_ptr(nkeys + 1, 0);
  std::vector<char> state(nkeys, 0);  // 1 = written directly, 2 = needs a task
  for (const Item& it : (nkeys > 0 ? items : std::vector<Item>())) {
    for (int32_t t = 0; t < it.w.qo_count; ++t) {
      const size_t key = static_cast<size_t>(it.w.qo_begin + t) * h_kv + it.w.kv_head;
      if (it.w.flags & kItemPartial) {
        src_ptr[key + 1] += 1;
        if (state[key] == 0) state[key] = 2;
      } else {
        state[key] = 1;
      }
    }
  }
  if (composable) {
    // tokens a format lists must end up with a result even if no key covers them
    for (const BlockRow& r : rows)
      for (int32_t t = 0; t < r.qo_len; ++t)
        for (int32_t h = 0; h < h_kv; ++h) {
          const size_t key = static_cast<size_t>(r.qo_begin + t) * h_kv + h;
          if (state[key] == 0) state[key] = 2;
        }
  }
  for (size_t k = 0; k < nkeys; ++k) src_ptr[k + 1] += src_ptr[k];
  if (nkeys == 0) src_ptr.assign(1, 0);
  std::vector<MergeSrc> srcs(src_ptr[nkeys]);
  {
    std::vector<int32_t> fill(src_ptr.begin(), src_ptr.end() - 1);
    for (const Item& it : items) {
      if (!(it.w.flags & kItemPartial)) continue;
      for (int32_t t = 0; t < it.w.qo_count; ++t) {
        const size_t key = static_cast<size_t>(it.w.qo_begin + t) * h_kv + it.w.kv_head;
        srcs[fill[key]++] = {it.w.partial_row + t * g, it.w.flag_id};
      }
    }
  }
  std::vector<MergeTask> tasks;
  for (size_t key = 0; key < nkeys; ++key) {
    if (state[key] != 2) continue;
    MergeTask m;
    m.qo_row = static_cast<int32_t>(key / h_kv);
    m.kv_head = static_cast<int32_t>(key % h_kv);
    m.src_begin = src_ptr[key];
    m.src_count = src_ptr[key + 1] - src_ptr[key];
    tasks.push_back(m);
  }

  // ---- 7b. merge tasks, longest first, on top of the attention loads ---------
  // (a quick estimate to compare candidates; the chosen plan's tasks are then
  // placed with their ready times, see assign_merges)
  std::vector<int64_t> mcosts(tasks.size());
  for (size_t i = 0; i < tasks.size(); ++i)
    mcosts[i] = cfg.gamma + cfg.beta * static_cast<int64_t>(tasks[i].src_count) * g;
  std::vector<int32_t> mowner, morder;
  out->att_load = load;
  assign_longest_first(mcosts, speed16, &load, &mowner, &morder);
  out->makespan = 0;
  out->total = 0;
  for (int32_t w = 0; w < nwg; ++w) {
    out->makespan = std::max(out->makespan, finish_time(load[w], speed16[w]));
    out->total += load[w];
  }
  // the longest chunk actually cut (L_kv for the pages' rule; filling may cut more;
  // with weighted units L_kv is not in tokens, so only the pieces count)
  bool weighted_units = false;
  for (const Unit& u : units) weighted_units |= u.w16 != 16;
  out->chunk = weighted_units ? 0 : chunk;
  for (const Item& it : items)
    if (it.nchunks > 1) out->chunk = std::max<int64_t>(out->chunk, it.w.kv_end - it.w.kv_begin);
  out->partial_rows = partial_rows;
  out->num_flags = num_flags;
  out->num_partial_items = num_partial_items;
  out->items = std::move(items);
  out->tasks = std::move(tasks);
  out->srcs = std::move(srcs);
  out->owner = std::move(owner);
  out->order = std::move(order);
  out->mowner = std::move(mowner);
  out->morder = std::move(morder);
  return BSR_OK;

}

}  // namespace

#ifndef BSR_EARLY_RELEASE
#define BSR_EARLY_RELEASE 1
#endif

// Each workgroup runs its items that write partial states first (its load is
// unchanged), and those that are not the last of its queue are stamped right after
// the item (kItemRelease), so that their merges can start while the queue's direct
// items run on: in a batch with one long request, the long request's chunks end
// well before the short requests that share their workgroups (skewed decode batch:
// 123-125 -> 120-121 us).  Composed formats keep one stamp pass per queue: their
// workgroups write partial states only, and each early release waits for the
// item's stores.  Tile grids keep theirs too: their queue tails are claimed at run
// time, and the reordering cost the FP8 prefill 1.5 %.
static void mark_releases(int32_t nwg, Schedule* s) {
  if (!BSR_EARLY_RELEASE) return;
  std::stable_partition(s->order.begin(), s->order.end(),
                        [&](int32_t i) { return (s->items[i].w.flags & kItemPartial) != 0; });
  std::vector<int32_t> last(nwg, -1);
  for (int32_t i : s->order) last[s->owner[i]] = i;
  for (int32_t i : s->order) {
    Item& it = s->items[i];
    if ((it.w.flags & kItemPartial) && last[s->owner[i]] != i) it.w.flags |= kItemRelease;
  }
}

// Merge tasks of the chosen schedule.  A task can start only when every
// workgroup holding one of its sources has finished its attention items (its
// release follows all of them), and a workgroup merges after its own attention
// and after the sources of all its tasks are ready.  Tasks go longest first to the
// workgroup where they would finish first, so tasks that become ready together at
// the end of the attention phase are spread instead of stacked on the
// least-loaded workgroups.  A workgroup without tasks whose attention ends by the
// task's ready time is always a best choice; among those the least loaded (then
// lowest id) is taken.
static void assign_merges(const PlanConfig& cfg, int32_t nwg, const std::vector<int32_t>& speed16, Schedule* s) {
  const int32_t g = cfg.group;
  const size_t nt = s->tasks.size();
  std::vector<int64_t> mcosts(nt);
  for (size_t i = 0; i < nt; ++i)
    mcosts[i] = cfg.gamma + cfg.beta * static_cast<int64_t>(s->tasks[i].src_count) * g;
  // a partial state is ready when its workgroup's queue is done, or, released
  // early, when its own item is
  std::vector<int64_t> flag_ready(s->num_flags, 0), done(nwg, 0);
  for (int32_t i : s->order) {
    const Item& it = s->items[i];
    const int32_t w = s->owner[i];
    done[w] += it.cost;
    if (it.w.flag_id >= 0) flag_ready[it.w.flag_id] = (it.w.flags & kItemRelease) ? done[w] : s->att_load[w];
  }
  std::vector<int64_t> ready(nt, 0);
  for (size_t i = 0; i < nt; ++i)
    for (int32_t k = 0; k < s->tasks[i].src_count; ++k)
      ready[i] = std::max(ready[i], flag_ready[s->srcs[s->tasks[i].src_begin + k].flag_id]);
  s->morder.resize(nt);
  for (size_t i = 0; i < nt; ++i) s->morder[i] = static_cast<int32_t>(i);
  std::stable_sort(s->morder.begin(), s->morder.end(), [&](int32_t a, int32_t b) { return mcosts[a] > mcosts[b]; });
  s->mowner.assign(nt, -1);
  const std::vector<int64_t>& att = s->att_load;
  std::vector<int64_t> mready(nwg, 0), msum(nwg, 0);
  std::vector<int32_t> busy;  // workgroups holding tasks
  using Slot = std::pair<int64_t, int32_t>;
  std::priority_queue<Slot, std::vector<Slot>, std::greater<Slot>> idle;  // (attention load, wg)
  for (int32_t w = 0; w < nwg; ++w) idle.push({att[w], w});
  for (int32_t i : s->morder) {
    int32_t best_w = -1;
    int64_t best_f = INT64_MAX;
    if (!idle.empty()) {
      best_w = idle.top().second;
      best_f = std::max(att[best_w], ready[i]) + mcosts[i];
    }
    if (idle.empty() || att[best_w] > ready[i]) {
      for (int32_t w : busy) {
        const int64_t f = std::max(att[w], std::max(mready[w], ready[i])) + msum[w] + mcosts[i];
        if (f < best_f || (f == best_f && w < best_w)) {
          best_f = f;
          best_w = w;
        }
      }
    }
    if (msum[best_w] == 0) {
      idle.pop();  // best_w was the idle top (busy workgroups have msum > 0)
      busy.push_back(best_w);
    }
    s->mowner[i] = best_w;
    mready[best_w] = std::max(mready[best_w], ready[i]);
    msum[best_w] += mcosts[i];
  }
  s->makespan = 0;
  s->total = 0;
  for (int32_t w = 0; w < nwg; ++w) {
    const int64_t l = msum[w] > 0 ? std::max(att[w], mready[w]) + msum[w] : att[w];
    s->makespan = std::max(s->makespan, finish_time(l, speed16[w]));
    s->total += l;
  }
}

int make_plan(const PlanConfig& cfg, const std::vector<BlockRow>& rows, int32_t total_qo,
              bool composable, PlanResult* out, std::string* err, const std::vector<uint64_t>* tree_rows) {
  const int32_t g = cfg.group;
  const int32_t h_kv = cfg.h_kv;

  // ---- 1. kernel kind and query tile -----------------------------------------
  const bool var = !cfg.alibi_raw.empty() || tree_rows != nullptr;
  bool any_decode = false, any_wide = false;
  int64_t max_decode_rows = 0;
  // KV tokens streamed by decode-sized rows and by tiles (once per query tile)
  int64_t decode_kv = 0, tile_kv = 0;
  // folded rows and count of the rows that need tiles
  int64_t wide_rows = 0, num_wide = 0;
  const int64_t tile_rows = mfma_tile(cfg.head_dim);
  for (const BlockRow& r : rows) {
    if (r.qo_len == 0) continue;
    const int64_t fr = static_cast<int64_t>(r.qo_len) * g;
    if (fr <= kMaxDecodeRows) {
      any_decode = true;
      max_decode_rows = std::max(max_decode_rows, fr);
      decode_kv += r.kv_len;
    } else {
      any_wide = true;
      tile_kv += ceil_div(fr, tile_rows) * r.kv_len;
      wide_rows += fr;
      ++num_wide;
    }
  }
  int32_t kernel = kKindDecode;
  int32_t decode_rows = max_decode_rows <= 4 ? 4 : 8;
  int32_t q_tile = decode_rows;
  bool short_tile = false;
  // the MFMA bodies take bf16 K/V, and FP8 K/V up to head dim 128
  const bool mfma_ok = cfg.bf16 && !(cfg.kv8 && cfg.head_dim > 128);
  if (any_wide) {
    if (!mfma_ok) {
      // fp32, and an FP8 K/V cache at head dim 256, have no MFMA body here: long
      // query rows run as tiles of 8 folded rows
      if (g > kMaxDecodeRows) {
        *err = "fp32 or FP8 K/V with more than 8 query heads per KV head is not supported";
        return BSR_ERR_UNSUPPORTED;
      }
      kernel = kKindDecode;
      decode_rows = kMaxDecodeRows;
      q_tile = decode_rows;
    } else {
      // Decode-sized rows next to tiles: the mixed grid (decode body for them, one
      // workgroup per CU) only when they stream at least a quarter of the KV
      // tokens; otherwise every row runs as a tile on the two-per-CU tile grid,
      // where a tile runs several times faster per CU than in the mixed grid's one
      // wavefront per SIMD (tree-masked speculative decode, 8 % decode-row tokens:
      // 457 -> 175 us; shared-prefix batch, 35 %: mixed 91 us, tiles 97 us).
      kernel = any_decode && decode_kv * 4 >= decode_kv + tile_kv ? kKindMixed : kKindMfma;
      // Tile height: the smallest tile of the menu at least the mean folded length
      // of the rows that need tiles.  The tile kernel at head dim 128 with bf16 K/V
      // has two, 64 and 128 rows; every other kernel has one.  The 64-row tile
      // (16 rows per wavefront, three workgroups per CU) halves the padding of
      // short rows, such as speculative drafts of 16 tokens at 4 query heads per
      // KV head (tree-masked decode batch: 176 -> 147 us), and loses to the
      // 128-row tile on long prefill rows (ragged causal prefill: 1630 ->
      // 2280 us), whose mean is far above 64.
      int32_t tile = mfma_tile(cfg.head_dim);
      if (kernel == kKindMfma && cfg.head_dim == 128 && !cfg.kv8 && g <= kShortTile &&
          wide_rows <= kShortTile * num_wide && cfg.num_wg[kKindMfma][1][var ? 1 : 0] > 0) {
        tile = kShortTile;
        short_tile = true;
      }
      if (g > tile) {
        *err = "query heads per KV head exceed the MFMA tile height";
        return BSR_ERR_UNSUPPORTED;
      }
      q_tile = tile;
    }
  }
  const int32_t nwg =
      cfg.num_wg[kernel][(kernel != kKindMfma && decode_rows == 8) || short_tile ? 1 : 0][var ? 1 : 0];
  if (nwg <= 0) {
    *err = "the kernel this plan needs (kind " + std::to_string(kernel) + ") is not built for this handle";
    return BSR_ERR_UNSUPPORTED;
  }

  // Workgroup speeds.  In a grid of two workgroups per CU (the MFMA kernel) the
  // hardware dispatches workgroups 0 .. #CU-1 first, one per CU, and #CU .. 2 #CU-1
  // into the second slots; while both run, the older wavefronts win the SIMD's
  // issue arbitration, so the second workgroup of a CU progresses more slowly and,
  // with equal loads, finishes its last stretch alone (a per-workgroup timeline of
  // the ragged causal prefill: 1360 us for the first slots, 1720 us for the
  // second).  Loads are then balanced in time: a second-slot workgroup runs at
  // slot2_speed16 / 16 of a first-slot one.
  std::vector<int32_t> speed16(nwg, 16);
  if (kernel == kKindMfma && cfg.cus > 0 && nwg == 2 * cfg.cus && cfg.slot2_speed16 > 0)
    for (int32_t w = cfg.cus; w < nwg; ++w) speed16[w] = cfg.slot2_speed16;

  // ---- 2. work units ---------------------------------------------------------
  std::vector<Unit> units;
  for (int32_t ri = 0; ri < static_cast<int32_t>(rows.size()); ++ri) {
    const BlockRow& r = rows[ri];
    if (r.qo_len == 0) continue;
    const bool wide = static_cast<int64_t>(r.qo_len) * g > kMaxDecodeRows;
    const bool mfma = mfma_ok && (kernel == kKindMfma || (kernel == kKindMixed && wide));
    const int32_t tile_tokens = (mfma ? q_tile : decode_rows) / g;
    // a row with per-head pages serves its own KV head only
    const int32_t h_first = r.head < 0 ? 0 : r.head;
    const int32_t h_last = r.head < 0 ? h_kv : r.head + 1;
    for (int32_t h = h_first; h < h_last; ++h) {
      for (int32_t t0 = 0; t0 < r.qo_len; t0 += tile_tokens) {
        Unit u;
        u.row = ri;
        u.head = h;
        u.t0 = t0;
        u.nt = std::min(tile_tokens, r.qo_len - t0);
        u.mfma = mfma;
        // the two bodies differ in time per KV token; only a grid that runs both
        // needs the weight (single-body plans keep the pages' key counts)
        u.w16 = kernel == kKindMixed && mfma ? std::max(cfg.mfma_w16, 1) : 16;
        int32_t end;
        if (cfg.causal) {
          u.causal_limit = r.kv_len - r.qo_len + t0;
          end = std::min<int32_t>(r.kv_len, u.causal_limit + u.nt);
        } else {
          u.causal_limit = kNoCausal;
          end = r.kv_len;
        }
        u.q_pos = r.kv_len - r.qo_len + t0;
        u.tree_lo = r.tree ? r.kv_len - r.qo_len : kNoTree;
        // a sliding window hides keys below window_lo + t from token t: the unit
        // starts at its first token's window, rounded down to the chunk granule so
        // chunk starts stay where the bodies expect them
        u.window_lo = kNoWindow;
        u.kv_lo = 0;
        if (cfg.window > 0) {
          // (in 64 bits: a window longer than every row reaches below kNoWindow)
          const int64_t lo = static_cast<int64_t>(r.kv_len) - r.qo_len + t0 - cfg.window + 1;
          u.window_lo = static_cast<int32_t>(std::max<int64_t>(lo, kNoWindow));
          u.kv_lo = std::min(std::max(u.window_lo, 0), std::max(end - 1, 0)) / kChunkGranule * kChunkGranule;
        }
        u.l_eff = std::max(end - u.kv_lo, 0);
        units.push_back(u);
      }
    }
  }

  // ---- 3. maximum KV chunk (the pages' L_kv) and its refinements -------------
  // (in weighted KV tokens: plain tokens unless a mixed grid weights MFMA units)
  int64_t total_kv = 0, max_leff = 0;
  for (const Unit& u : units) {
    total_kv += weighted(u, u.l_eff);
    max_leff = std::max<int64_t>(max_leff, weighted(u, u.l_eff));
  }
  const int64_t min_chunk = round_up(std::max(cfg.min_chunk, 1), kChunkGranule);
  const int64_t base_chunk =
      std::max<int64_t>(round_up(std::max<int64_t>(ceil_div(total_kv, nwg), 1), kChunkGranule), min_chunk);
  // A lower bound on every candidate's makespan: each candidate's loads sum to at
  // least the units' unsplit costs (cutting adds the fixed item cost, merges add
  // theirs), and the busiest workgroup finishes no earlier than that sum spread
  // over all workgroups at their speeds.  A candidate replaces the best only if it
  // is 3 % shorter, so once the best is within 3 % of the bound no later candidate
  // can: the remaining ones are not scored (the plan is the same).
  int64_t lb_total = 0, sum_speed16 = 0;
  for (const Unit& u : units)
    if (!(composable && u.l_eff == 0))
      lb_total += cfg.alpha * static_cast<int64_t>(u.nt) * g + cfg.beta * weighted(u, u.l_eff) + cfg.gamma;
  for (int32_t w = 0; w < nwg; ++w) sum_speed16 += speed16[w];
  const int64_t lower_bound = lb_total * 16 / std::max<int64_t>(sum_speed16, 1);
  // The candidates (chunk length, filling), in scoring order.  The first always
  // exists; the later ones skip repeats of a chunk length and lengths that cut
  // nothing (the same plan as the first).
  struct Candidate {
    int64_t chunk;
    bool fill;
  };
  std::vector<Candidate> cands;
  {
    int64_t last_chunk = -1;
    for (int k = 1; k <= kChunkCandidates + 2; ++k) {
      // candidates: the pages' L_kv, L_kv / k (k = 2..), then filling at L_kv and
      // at L_kv / 2 (the latter cuts units of more than half of L_kv only where a
      // workgroup's room ends: when more units than workgroups are a little over
      // L_kv / 2 long, as under a sliding window, whole units cannot balance and
      // halving every one costs an item and a merge each)
      const bool fill = k > kChunkCandidates;
      const int64_t fill_chunk =
          k == kChunkCandidates + 1 ? base_chunk
                                    : std::max<int64_t>(round_up(ceil_div(base_chunk, 2), kChunkGranule), min_chunk);
      int64_t chunk =
          fill ? fill_chunk : std::max<int64_t>(round_up(ceil_div(base_chunk, k), kChunkGranule), min_chunk);
      // chunks at least as long as every unit cut nothing: all such candidates,
      // and filling without long units, are the same plan
      if (chunk >= max_leff) {
        if (!cands.empty()) continue;
        chunk = std::max<int64_t>(round_up(std::max<int64_t>(max_leff, 1), kChunkGranule), base_chunk);
      }
      if (!fill && chunk == last_chunk) continue;
      last_chunk = chunk;
      cands.push_back({chunk, fill});
    }
  }
  // The first candidate is scored alone: it often ends the search (within 3 % of
  // the bound).  When it does not and it took long enough to pay for threads, the
  // others are scored in parallel; either way they are then taken in order with the
  // same rule, so the plan does not depend on the path.
  const size_t nc = cands.size();
  std::vector<Schedule> scored(nc);
  std::vector<int> rcs(nc, BSR_OK);
  std::vector<std::string> errs(nc);
  const auto t_first = std::chrono::steady_clock::now();
  rcs[0] = schedule(cfg, rows, units, cands[0].chunk, cands[0].fill, nwg, speed16, total_qo, composable, &scored[0],
                    &errs[0]);
  const double first_us =
      std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t_first).count();
  const bool done_early = rcs[0] != BSR_OK || scored[0].makespan * 97 <= lower_bound * 100;
  if (!done_early && nc > 1) {
    // (an allocation failure inside a worker becomes that candidate's error)
    auto score = [&](size_t c) {
      try {
        rcs[c] = schedule(cfg, rows, units, cands[c].chunk, cands[c].fill, nwg, speed16, total_qo, composable,
                          &scored[c], &errs[c]);
      } catch (const std::bad_alloc&) {
        rcs[c] = BSR_ERR_CAPACITY;
        errs[c] = "host memory exhausted while scoring a plan";
      }
    };
    size_t threaded = 1;  // candidates 1 .. threaded - 1 run on threads
    std::vector<std::thread> pool;
    if (first_us >= cfg.parallel_plan_us && std::thread::hardware_concurrency() > 1) {
      try {
        pool.reserve(nc - 1);
        for (size_t c = 1; c < nc; ++c) {
          pool.emplace_back(score, c);
          threaded = c + 1;
        }
      } catch (const std::exception&) {
        // no more threads: the remaining candidates are scored here
      }
    }
    for (size_t c = threaded; c < nc; ++c) {
      score(c);
      if (rcs[c] != BSR_OK) break;
    }
    for (std::thread& t : pool) t.join();
  }
  Schedule best;
  bool have = false;
  for (size_t c = 0; c < nc; ++c) {
    if (rcs[c] != BSR_OK) {
      *err = errs[c];
      return rcs[c];
    }
    Schedule& cand = scored[c];
    if (!have || cand.makespan * 100 < best.makespan * 97) {
      best = std::move(cand);
      have = true;
    }
    if (best.makespan * 97 <= lower_bound * 100) break;
  }
  if (!composable && kernel != kKindMfma) mark_releases(nwg, &best);
  assign_merges(cfg, nwg, speed16, &best);
  if (best.partial_rows > cfg.max_partial_rows) {
    *err = "plan needs " + std::to_string(best.partial_rows) + " partial rows, capacity is " +
           std::to_string(cfg.max_partial_rows);
    return BSR_ERR_CAPACITY;
  }
  const std::vector<Item>& items = best.items;
  const std::vector<MergeTask>& tasks = best.tasks;
  const std::vector<MergeSrc>& srcs = best.srcs;
  const std::vector<int32_t>& owner = best.owner;
  const std::vector<int32_t>& order = best.order;
  const std::vector<int32_t>& mowner = best.mowner;
  const std::vector<int32_t>& morder = best.morder;
  const int64_t chunk = best.chunk;
  const int64_t partial_rows = best.partial_rows;
  const int32_t num_flags = best.num_flags;
  const int32_t num_partial_items = best.num_partial_items;
  const int64_t max_load = best.makespan;
  const int64_t total_cost = best.total;

  // ---- 8. blob ---------------------------------------------------------------
  PlanHeader hdr;
  std::memset(&hdr, 0, sizeof(hdr));
  hdr.magic = kPlanMagic;
  hdr.kernel = kernel;
  hdr.num_wg = nwg;
  hdr.num_items = static_cast<int32_t>(items.size());
  hdr.num_merge = static_cast<int32_t>(tasks.size());
  hdr.num_srcs = static_cast<int32_t>(srcs.size());
  hdr.num_flags = num_flags;
  hdr.instance = instance_key(kernel, kernel == kKindMfma ? (short_tile ? 1 : 0) : decode_rows, cfg.head_dim, cfg.bf16, cfg.cap,
                              kernel == kKindMfma && cfg.page_size == 1, cfg.kv8, var);
  hdr.spin_limit = kDefaultSpinLimit;
  // Claimed items (MFMA tile grids): the tail of each workgroup's queue, the items
  // that start after (16 - kPoolTail16) / 16 of its planned load (never its first
  // item), go to a pool that free workgroups claim at run time, longest first.
  // Only the tail: items as large as a workgroup's whole load are balanced better
  // by the plan than by first-come claims, which hand an early finisher a whole
  // second item.  Decode and mixed grids keep their queues: their workgroups end
  // together, and the claims they would all issue at the end, on one counter in
  // the memory-side cache, serialize (measured: batch decode 215 -> 232 us with 88
  // claimed items), while a tile grid's claims spread over the run (ragged causal
  // prefill 1613 -> 1581 us).
  std::vector<char> pooled(items.size(), 0);
  std::vector<int32_t> pool_order;
  int32_t num_static = static_cast<int32_t>(items.size());
  if (!cfg.static_queues && kernel == kKindMfma) {
    std::vector<int64_t> wg_load(nwg, 0), wg_at(nwg, 0);
    std::vector<int32_t> wg_count(nwg, 0);
    for (size_t i = 0; i < items.size(); ++i) wg_load[owner[i]] += items[i].cost;
    for (int32_t i : order) {
      const int32_t w = owner[i];
      if (wg_count[w] > 0 && wg_at[w] * 16 >= wg_load[w] * (16 - kPoolTail16)) {
        pooled[i] = 1;
        pool_order.push_back(i);
        --num_static;
      }
      wg_at[w] += items[i].cost;
      wg_count[w] += 1;
    }
    // (longest-first assignments already list the pool in that order)
    auto longer = [&](int32_t a, int32_t b) { return items[a].cost > items[b].cost; };
    if (!std::is_sorted(pool_order.begin(), pool_order.end(), longer))
      std::stable_sort(pool_order.begin(), pool_order.end(), longer);
  }
  hdr.pool_begin = num_static;
  int64_t off = sizeof(PlanHeader);
  hdr.off_status = align16(off);
  off = hdr.off_status + 16;
  hdr.off_claim = align16(off);
  off = hdr.off_claim + 16;
  hdr.off_epochs = align16(off);
  off = hdr.off_epochs + 4LL * nwg;
  hdr.off_flags = align16(off);
  off = hdr.off_flags + 4LL * num_flags;
  hdr.off_item_ptr = align16(off);
  off = hdr.off_item_ptr + 4LL * (nwg + 1);
  hdr.off_items = align16(off);
  off = hdr.off_items + static_cast<int64_t>(sizeof(WorkItem)) * items.size();
  hdr.off_merge_ptr = align16(off);
  off = hdr.off_merge_ptr + 4LL * (nwg + 1);
  hdr.off_merge = align16(off);
  off = hdr.off_merge + static_cast<int64_t>(sizeof(MergeTask)) * tasks.size();
  hdr.off_srcs = align16(off);
  off = hdr.off_srcs + static_cast<int64_t>(sizeof(MergeSrc)) * srcs.size();
  if (!cfg.alibi_raw.empty()) {
    hdr.off_alibi = align16(off);
    off = hdr.off_alibi + 4LL * static_cast<int64_t>(cfg.alibi_raw.size());
  }
  if (tree_rows != nullptr) {
    hdr.off_tree = align16(off);
    off = hdr.off_tree + 8LL * total_qo;
  }
  const int64_t bytes = align16(off);
  if (bytes > cfg.blob_capacity) {
    *err = "plan of " + std::to_string(bytes) + " bytes exceeds the plan segment (" +
           std::to_string(cfg.blob_capacity) + " bytes); raise the maxima at create";
    return BSR_ERR_CAPACITY;
  }
  hdr.blob_bytes = static_cast<int32_t>(bytes);

  out->blob.assign(bytes, 0);
  uint8_t* base = out->blob.data();
  std::memcpy(base, &hdr, sizeof(hdr));
  // work queues: items of workgroup w in the order they were assigned, then the
  // pool in assignment order
  {
    std::vector<int32_t> count(nwg + 1, 0);
    for (size_t i = 0; i < items.size(); ++i)
      if (!pooled[i]) count[owner[i] + 1] += 1;
    for (int32_t w = 0; w < nwg; ++w) count[w + 1] += count[w];
    std::memcpy(base + hdr.off_item_ptr, count.data(), 4 * (nwg + 1));
    std::vector<int32_t> fill(count.begin(), count.end() - 1);
    WorkItem* dst = reinterpret_cast<WorkItem*>(base + hdr.off_items);
    for (int32_t i : order)
      if (!pooled[i]) dst[fill[owner[i]]++] = items[i].w;
    // Composed formats in a mixed grid: every queue holds tile items (the shared
    // prefix) first, then decode items (the suffixes), so all CUs would multiply
    // and then all stream.  Odd workgroups run their queue backwards, so that at
    // any time about half the CUs do each (the order within a queue does not
    // change any result; shared-prefix batch 96 -> 93 us).
    if (kernel == kKindMixed && composable)
      for (int32_t w = 1; w < nwg; w += 2) std::reverse(dst + count[w], dst + count[w + 1]);
    int32_t next_pool = num_static;
    for (int32_t i : pool_order) dst[next_pool++] = items[i].w;
  }
  {
    std::vector<int32_t> count(nwg + 1, 0);
    for (size_t i = 0; i < tasks.size(); ++i) count[mowner[i] + 1] += 1;
    for (int32_t w = 0; w < nwg; ++w) count[w + 1] += count[w];
    std::memcpy(base + hdr.off_merge_ptr, count.data(), 4 * (nwg + 1));
    std::vector<int32_t> fill(count.begin(), count.end() - 1);
    MergeTask* dst = reinterpret_cast<MergeTask*>(base + hdr.off_merge);
    for (int32_t i : morder) dst[fill[mowner[i]]++] = tasks[i];
    if (!srcs.empty()) std::memcpy(base + hdr.off_srcs, srcs.data(), sizeof(MergeSrc) * srcs.size());
  }
  if (hdr.off_alibi != 0)
    std::memcpy(base + hdr.off_alibi, cfg.alibi_raw.data(), 4 * cfg.alibi_raw.size());
  if (hdr.off_tree != 0 && total_qo > 0)
    std::memcpy(base + hdr.off_tree, tree_rows->data(), 8LL * total_qo);

  out->kernel = kernel;
  out->num_wg = nwg;
  out->var = var;
  out->q_tile = q_tile;
  out->short_tile = short_tile;
  out->decode_rows = decode_rows;
  out->num_items = hdr.num_items;
  out->num_partial_items = num_partial_items;
  out->num_partial_rows = partial_rows;
  out->num_merge = hdr.num_merge;
  out->num_srcs = hdr.num_srcs;
  out->kv_chunk = chunk;
  out->max_wg_cost = max_load;
  out->total_cost = total_cost;
  return BSR_OK;
}

}  // namespace bsr
