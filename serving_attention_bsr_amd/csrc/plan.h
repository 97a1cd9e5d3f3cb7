// plan.h -- host planner: from sequence lengths to a work queue and merge map.
//
// Core mechanism 6 of the FlashInfer explainer page (paper Algorithm 1, section
// 3.3.1, Figure 6) and the tile heuristic of Core mechanism 4 (paper section
// 3.2.2).  Pure host C++: no HIP calls, so it is exercised on machines without a
// GPU through a host-only handle.
#pragma once

#include <stdint.h>

#include <string>
#include <vector>

#include "layout.h"

namespace bsr {

struct PlanConfig {
  int32_t h_qo = 0, h_kv = 0, group = 0, head_dim = 0, page_size = 0;
  bool causal = false;
  bool bf16 = false;
  bool cap = false;  // logits soft-cap on (selects the kernel instance)
  // grid per kernel instance: [KernelKind][decode rows 4 -> 0, 8 -> 1; tile
  // kernel: 128-row tile -> 0, 64-row tile -> 1][variant data]
  int32_t num_wg[4][2][2] = {};
  int64_t alpha = 1, beta = 1;
  int64_t gamma = 512;       // fixed cost of a work item or merge task (KV-token units)
  int32_t min_chunk = 64;
  // cost of one KV token of an MFMA item in a mixed grid, in sixteenths of a
  // decode item's token (16 = equal)
  int32_t mfma_w16 = 16;
  // CUs of the device (0 for host-only handles) and the speed of the second
  // workgroup of each CU in a two-per-CU MFMA grid, in sixteenths of the first's
  int32_t cus = 0;
  bool kv8 = false;  // K/V are FP8 codes: decode body only (no MFMA tiles)
  int32_t slot2_speed16 = 16;
  int32_t window = 0;  // sliding window in keys (0: none)
  // every item on the workgroup it is assigned to (no run-time claiming)
  bool static_queues = false;
  // a plan whose first chunking candidate took at least this long (microseconds)
  // scores the others on threads of their own (the plan is the same either way)
  double parallel_plan_us = 150.0;
  // ALiBi: per query head, slope / sm_scale (empty: no ALiBi)
  std::vector<float> alibi_raw;
  // capacities (plan rejected beyond them)
  int32_t max_batch = 0, max_total_qo = 0;
  int64_t max_total_kv = 0;
  int64_t max_partial_rows = 0;
  int64_t blob_capacity = 0;
};

// One block row of one format.
struct BlockRow {
  int32_t qo_begin = 0, qo_len = 0;
  int32_t page_begin = 0;  // absolute index into kv_indices
  int32_t kv_len = 0;
  int32_t format = 0;
  bool tree = false;  // the row's new tokens carry tree-mask rows
  int32_t head = -1;  // the KV head this row's pages belong to, or -1 for every head
};

struct PlanResult {
  std::vector<uint8_t> blob;  // the bytes to upload
  int32_t kernel = 0, num_wg = 0, q_tile = 0, decode_rows = 0;
  bool var = false;  // the plan carries variant data (ALiBi slopes, tree masks)
  bool short_tile = false;  // tile kernel with 64-row tiles at head dim 128
  int32_t num_items = 0, num_partial_items = 0, num_merge = 0, num_srcs = 0;
  int64_t num_partial_rows = 0;
  int64_t kv_chunk = 0, max_wg_cost = 0, total_cost = 0;
};

// Decode body handles up to this many folded rows per item.
constexpr int kMaxDecodeRows = 8;
// KV granularity that chunk lengths are rounded to (tokens).
constexpr int kChunkGranule = 64;
// Share of each workgroup's planned load, in sixteenths, whose items are claimed
// at run time instead of queued (the tail of the queue; measured on the ragged
// causal prefill: 2 -> 1543 us, 4 -> 1556, 6 -> 1574, 8 -> 1607).
#ifndef BSR_POOL_TAIL16
#define BSR_POOL_TAIL16 2
#endif
constexpr int kPoolTail16 = BSR_POOL_TAIL16;
// The planner also tries L_kv / k for k up to this and keeps the smallest
// predicted makespan (the pages' L_kv unless another is clearly better).
constexpr int kChunkCandidates = 4;
// MFMA tile height (folded rows) of the kernels: 32 rows per wavefront up to
// D = 128, 16 rows per wavefront at D = 256.
inline int32_t mfma_tile(int32_t head_dim) { return head_dim == 256 ? 64 : 128; }
// The second tile of the tile kernel at D = 128: 16 rows per wavefront.
constexpr int32_t kShortTile = 64;

// Returns 0 and fills out, or a bsr_status code with a message in err.
// tree_rows: null, or one 64-bit tree-mask row per query token (rows of block
// rows whose `tree` is set; bit u: the token sees key l_kv - l_qo + u).
int make_plan(const PlanConfig& cfg, const std::vector<BlockRow>& rows, int32_t total_qo,
              bool composable, PlanResult* out, std::string* err,
              const std::vector<uint64_t>* tree_rows = nullptr);

}  // namespace bsr
