// layout.h -- the plan blob and workspace layout shared by the host planner and
// the persistent kernel.  Plain structs of int32 so that host and device agree
// byte for byte.
//
// The workspace follows Core mechanism 7 of the FlashInfer explainer page
// (paper section 3.3.1 and Appendix D.1): it is sized once for the maxima given
// at set-up, its segments sit at constant offsets, and each plan is staged in
// host memory and copied into the plan segment with one asynchronous copy.  The
// kernel receives only the workspace base pointer, so a captured launch stays
// valid across plans.
//
// Workspace (byte offsets fixed at create time):
//   [0, plan_capacity)                 plan blob, rewritten by every plan upload
//   [partial_o_offset, ...)            fp32 [max_partial_rows, D] partial outputs
//   [partial_lse_offset, ...)          fp32 [max_partial_rows] partial log2-sum-exp
//
// Plan blob (offsets inside the blob are in the header; all 16-byte aligned):
//   PlanHeader       magic, kernel instance, counts, offsets, wait bound
//   status[4]        device error words, zeroed by each upload
//   epochs[num_wg]   per-workgroup run counters (all equal between runs)
//   flags[num_flags] per-partial ready stamps (the epoch of the run that wrote it)
//   item_ptr[num_wg + 1]   work queue of workgroup w: items[item_ptr[w] .. item_ptr[w+1])
//   items[num_items]       WorkItem
//   merge_ptr[num_wg + 1]  merge tasks of workgroup w
//   merge[num_merge]       MergeTask
//   srcs[num_srcs]         MergeSrc, grouped per task
//   alibi[H_qo]            (ALiBi plans) slope / sm_scale of each query head
//   tree[total_qo]         (tree-masked plans) uint64 per query token: bit u set iff
//                          the token sees its block row's key tree_lo + u
#pragma once

#include <stdint.h>

namespace bsr {

constexpr int32_t kPlanMagic = 0x41525342;  // "BSRA"
constexpr int kWgThreads = 256;             // 4 wavefronts of 64
constexpr int kWaves = 4;
constexpr int32_t kNoCausal = 0x3fffffff;   // causal_limit meaning "every key visible"
constexpr int32_t kNoWindow = -0x3fffffff;  // window_lo meaning "no lower bound"
constexpr int32_t kNoTree = 0x3fffffff;     // tree_lo meaning "no tree mask"
constexpr int kMaxTreeTokens = 64;          // new tokens of a tree-masked request (one 64-bit row each)

enum KernelKind : int32_t { kKindDecode = 1, kKindMfma = 2, kKindMixed = 3 };

enum ItemFlags : int32_t {
  kItemMfma = 1,     // run the MFMA tile body (else the VALU decode body)
  kItemPartial = 2,  // write a partial state to the workspace (else O/LSE directly)
  kItemRelease = 4,  // stamp the partial state right after the item, not at the end of the queue
};

enum StatusWord : int32_t {
  kStatusWaitTimeout = 0,    // a merge gave up waiting for a partial
  kStatusWrongKernel = 1,    // the plan was made for another kernel instance or grid
};

// Identity of the persistent-kernel instance a plan is made for: the kernel kind,
// the decode body's folded rows (for the MFMA-only kind: 0 for 128-row tiles, 1
// for 64-row tiles at head dim 128), the head dim, the
// handle-level switches that select an instance, and whether the plan carries
// variant data (ALiBi slopes, tree masks).  The planner writes it into the
// header and the kernel compares it with its own template arguments, so a launch
// captured for one instance never runs a later plan made for another (for
// example a decode graph captured at 4 folded rows replaying an 8-row plan).
constexpr int32_t instance_key(int kind, int rows, int head_dim, bool bf16, bool cap, bool page1, bool kv8,
                               bool var) {
  return kind | (rows << 4) | ((head_dim / 64) << 8) | (bf16 ? 1 << 12 : 0) | (cap ? 1 << 13 : 0) |
         (page1 ? 1 << 14 : 0) | (kv8 ? 1 << 15 : 0) | (var ? 1 << 16 : 0);
}

// Default bound of a merge's wait for one ready stamp, in polls (each poll sleeps
// briefly); the planner writes it into the header.
constexpr int32_t kDefaultSpinLimit = 1 << 21;

struct WorkItem {  // 64 bytes
  int32_t flags;
  int32_t qo_begin;      // first query token (row of Q/O) of the tile
  int32_t qo_count;      // query tokens in the tile (folded rows = qo_count * g)
  int32_t kv_head;
  int32_t page_begin;    // index into kv_indices of the block row's first page
  int32_t kv_begin;      // first key of the chunk, counted within the block row
  int32_t kv_end;        // one past the last key of the chunk
  int32_t causal_limit;  // token i of the tile sees keys j <= causal_limit + i
  int32_t partial_row;   // first folded row of the partial state, or -1
  int32_t flag_id;       // ready-flag slot of the partial state, or -1
  int32_t window_lo;     // token i of the tile sees keys j >= window_lo + i
  int32_t q_pos;         // position of the tile's first token (l_kv - l_qo + t0; ALiBi)
  int32_t tree_lo;       // first key of the block row's tree-masked new tokens, or kNoTree
  int32_t pad[3];
};

struct MergeTask {  // 16 bytes: combine the states of g folded rows of one token
  int32_t qo_row;     // query token
  int32_t kv_head;    // rows kv_head*g .. kv_head*g+g-1 of O
  int32_t src_begin;  // first MergeSrc of this task
  int32_t src_count;  // 0 writes the empty state (O = 0, LSE = -inf)
};

struct MergeSrc {  // 8 bytes
  int32_t partial_row;  // folded row holding this token's first head of the group
  int32_t flag_id;      // ready flag of the item that wrote it
};

struct PlanHeader {  // 88 bytes
  int32_t magic;
  int32_t kernel;
  int32_t num_wg;
  int32_t num_items;
  int32_t num_merge;
  int32_t num_srcs;
  int32_t num_flags;
  int32_t off_status;
  int32_t off_epochs;
  int32_t off_flags;
  int32_t off_item_ptr;
  int32_t off_items;
  int32_t off_merge_ptr;
  int32_t off_merge;
  int32_t off_srcs;
  int32_t blob_bytes;
  int32_t instance;    // instance_key() of the kernel this plan is made for
  int32_t spin_limit;  // polls before a merge gives up on a ready stamp
  int32_t off_alibi;   // float [H_qo] ALiBi slopes / sm_scale, or 0 without ALiBi
  int32_t off_tree;    // uint64 [total_qo] tree-mask rows, or 0 without tree masks
  // Items pool_begin .. num_items - 1 are claimed at run time, in array order, by
  // whichever workgroup is free (items 0 .. pool_begin - 1 are the per-workgroup
  // queues); off_claim holds two int32 claim counters, used by alternate runs
  // (epoch parity), each run clearing the other one for the next.
  int32_t pool_begin;
  int32_t off_claim;
};

static_assert(sizeof(WorkItem) == 64, "WorkItem layout");
static_assert(sizeof(MergeTask) == 16, "MergeTask layout");
static_assert(sizeof(MergeSrc) == 8, "MergeSrc layout");
static_assert(sizeof(PlanHeader) == 88, "PlanHeader layout");

}  // namespace bsr
