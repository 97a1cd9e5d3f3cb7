/*
 * bsr_attn.h -- C ABI of an MI355X (gfx950) library for attention over a KV cache
 * stored as a block-sparse-row (BSR) matrix.
 *
 * Sources: the FlashInfer explainer page on zenmind.me ("FlashInfer：面向 LLM 推理
 * 服务的高效可定制注意力引擎", restating the MLSys 2025 paper), cited below by
 * its section names:
 *   - Terms "BSR" and Core mechanism 1 (paper section 3.1.1, Figure 2): the KV
 *     cache is a BSR matrix; block row r of the matrix reads the physical pages
 *     kv_indices[kv_indptr[r] .. kv_indptr[r+1]); any page size is allowed.
 *   - Terms "ragged tensor": Q and O of all requests packed without padding and
 *     addressed by qo_indptr.
 *   - Terms "Attention State and ⊕" (paper section 2.2): the result of attention is
 *     the state (O, LSE); partial states of key chunks are combined with ⊕.
 *   - Terms "plan()/run()" and Core mechanism 6 (paper Algorithm 1, section
 *     3.3.1, Figure 6): a host planner runs once per generation step from the
 *     sequence lengths only, balances work over a fixed number of workgroups
 *     with cost alpha*l_q + beta*l_kv, caps KV chunks at
 *     L_kv = sum(ceil(l_qo/T_q) * l_kv) / #workgroups, assigns the longest work
 *     first through a priority queue, and merges partial states without atomic
 *     aggregation in an order fixed by the lengths.
 *   - Core mechanism 7 (paper section 3.3.1, Appendix D): the run kernel is
 *     persistent with a fixed grid; the workspace is sized for the maxima given at
 *     set-up and its segments sit at constant offsets; the plan is staged in host
 *     memory and copied asynchronously; only long requests are split, short ones
 *     write the final output directly; partial outputs are bounded by
 *     2 * #workgroups * T_q * H_qo * (D + 1) values.
 *   - Core mechanism 8 (paper Appendix E): the caller may set the number of
 *     workgroups attention uses.
 *   - Terms "composable formats" and Core mechanism 2 (paper section 3.1.2,
 *     Figure 3): the KV matrix may be split into several BSR sub-matrices (for
 *     example a shared prefix read by many query rows and per-request suffixes);
 *     only index arrays differ, no KV data moves.
 *   - Terms "GQA head-group fusion" (paper Appendix A, Figure 11): query head h
 *     reads KV head h / g with g = H_qo / H_kv; the g heads of a group are folded
 *     into the query-length dimension of one work item.
 *
 * Layouts (all row-major, last index contiguous):
 *   Q, O           [sum l_qo, H_qo, D]    dtype of the handle (fp32 or bf16)
 *   LSE            [sum l_qo, H_qo]       fp32, natural logarithm
 *   K pool, V pool [num_pages, H_kv, P, D] dtype of the handle
 *   qo_indptr      int32 [B + 1]   query tokens of block row r: [qo_indptr[r], qo_indptr[r+1])
 *   kv_indptr      int32 [B + 1]   pages of block row r: kv_indices[kv_indptr[r] .. kv_indptr[r+1])
 *   kv_indices     int32 [nnz]     physical page ids (device memory)
 *   last_page_len  int32 [B]       valid slots in the last page, 1..P (ignored for empty rows)
 * Block row r holds l_kv = (n_pages - 1) * P + last_page_len[r] tokens; token tau
 * is slot tau % P of page kv_indices[kv_indptr[r] + tau / P].
 *
 * Semantics: O = softmax(S) V and LSE = log(sum exp(S)) per query row and head,
 * where S = sm_scale * q.k, then S = cap * tanh(S / cap) when a soft-cap is set,
 * then, for causal handles, key j of a block row is hidden from its t-th query
 * token (0-based) when j > l_kv - l_qo + t, and, with a sliding window of W keys,
 * when j <= l_kv - l_qo + t - W (a window is one of the mask variants of the
 * FlashInfer explainer page's Background and paper section 3.2.3; the window ends
 * at the same bottom-right aligned position as the causal mask).  A row that sees
 * no key gives O = 0 and LSE = -inf.
 *
 * Ownership: the library allocates no device memory.  The caller allocates the
 * workspace (device) and the staging buffer (host; page-locked for an
 * asynchronous upload) with the sizes bsr_attn_workspace_size() reports, and keeps
 * both alive and unchanged in address while plans and runs use them.  Host arrays
 * passed to the plan calls are read during the call only.
 *
 * Errors: every call returns a bsr_status; on failure nothing is launched and
 * bsr_attn_last_error() returns a message for the calling thread.  A handle is
 * not thread-safe.  Streams are hipStream_t passed as void* (NULL = null stream).
 */
#ifndef BSR_ATTN_H
#define BSR_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BSR_ATTN_ABI_VERSION 4

typedef enum bsr_status {
  BSR_OK = 0,
  BSR_ERR_INVALID_ARG = 1, /* malformed arguments or index arrays */
  BSR_ERR_CAPACITY = 2,    /* a plan exceeds the maxima given at create time */
  BSR_ERR_UNSUPPORTED = 3, /* shape or option the library does not implement */
  BSR_ERR_HIP = 4,         /* a HIP runtime call failed */
  BSR_ERR_DEVICE = 5       /* the device reported an error (see bsr_attn_check) */
} bsr_status;

/* BSR_DTYPE_BF16_KV_FP8: Q and O bf16, K and V pools (and appended K/V rows) OCP
 * FP8 E4M3 codes, one byte per element (Core mechanism 8 of the explainer page,
 * paper Appendix F), converted exactly to bf16 on chip; decode rows on the VALU
 * body, wide rows (prefill) on the MFMA tile body up to head dim 128 (at 256 they
 * run as 8-row decode tiles).  Scales are the caller's: a K scale folds into
 * sm_scale, a V scale multiplies O. */
typedef enum bsr_dtype { BSR_DTYPE_F32 = 0, BSR_DTYPE_BF16 = 1, BSR_DTYPE_BF16_KV_FP8 = 2 } bsr_dtype;

typedef struct bsr_attn_config {
  int32_t num_qo_heads;    /* H_qo */
  int32_t num_kv_heads;    /* H_kv; must divide H_qo */
  int32_t head_dim;        /* D in {64, 128, 256} */
  int32_t page_size;       /* P >= 1 (Bc of the BSR matrix) */
  int32_t dtype;           /* bsr_dtype of Q, K, V and O */
  int32_t causal;          /* 0 or 1; bottom-right aligned mask */
  float sm_scale;          /* <= 0 selects 1 / sqrt(D) */
  float logits_soft_cap;   /* 0 disables; otherwise S = cap * tanh(S / cap) */
  int32_t max_batch;       /* most block rows of one plan (all formats together) */
  int32_t max_total_qo;    /* most query tokens (rows of Q) of one plan */
  int64_t max_total_kv;    /* most KV tokens summed over the block rows of one plan */
  int32_t num_workgroups;  /* persistent grid budget; each kernel uses at most what the
                              device keeps resident; 0 = the kernel's default per CU */
  int32_t cost_alpha;      /* work-item cost weights alpha, beta; 0 selects 1 */
  int32_t cost_beta;
  int32_t min_kv_chunk;    /* smallest KV chunk the planner cuts, tokens; 0 selects 64 */
  int32_t max_partial_rows;/* partial-state capacity in folded rows; 0 = derived bound */
  int32_t cost_item;       /* fixed cost of one work item, in KV-token units (pipeline
                              fill and drain); 0 selects the default, < 0 selects none */
  int32_t cost_mfma;       /* cost of one KV token of an MFMA (tile) work item relative
                              to one of a decode work item, in sixteenths; used when one
                              grid runs both bodies (composed formats, mixed batches);
                              0 selects the measured default for the head dim */
  int32_t slot2_speed;     /* in a grid of two workgroups per CU (MFMA tile body), the
                              rate of each CU's second workgroup relative to its first,
                              in sixteenths; the planner balances their loads in time
                              (Core mechanism 6 balances in cost).  0 selects the
                              measured default, 16 treats them as equal */
  int32_t sliding_window;  /* 0: no window.  W >= 1: each query sees only keys inside
                              the window of W keys described above; bsr_attn_plan only
                              (bsr_attn_plan_composable rejects it).  The planner gives
                              each query tile only the keys its window can reach */
  int32_t static_queues;   /* 0 (default): in plans for the MFMA tile kernel, the tail
                              of each workgroup's queue (items starting after 7/8 of its
                              planned load) is claimed at run time, one item at a time,
                              longest first, from a counter in the workspace, by
                              whichever workgroup is free, so that faster CUs (the chip's
                              XCDs run at measurably different rates) take more of it.
                              1: every item runs on the workgroup the plan assigns.  The
                              items, partial states and merges are the same either way,
                              so results are bitwise identical between the two */
  const float* alibi_slopes; /* NULL: no ALiBi.  Otherwise host array [num_qo_heads],
                              read at create: query head h adds m_h * (j - p) to the
                              scaled logit of key j before the soft-cap, p being the
                              query's bottom-right aligned position l_kv - l_qo + t
                              (ALiBi, one of the variants of the explainer page's
                              Background and paper section 3.2.3); bsr_attn_plan and
                              bsr_attn_plan_tree_mask only */
} bsr_attn_config;

/* One BSR sub-matrix for bsr_attn_plan_composable().  Arrays are host memory. */
typedef struct bsr_format {
  int32_t num_block_rows;
  const int32_t* qo_indptr;     /* [num_block_rows + 1] query-token ranges into Q/O */
  const int32_t* kv_indptr;     /* [num_block_rows + 1] page ranges, relative to the offset */
  const int32_t* last_page_len; /* [num_block_rows] */
  int32_t kv_indices_offset;    /* first entry of this format inside kv_indices */
} bsr_format;

typedef struct bsr_plan_info {
  int32_t kernel;          /* 1 = VALU decode body, 2 = MFMA tile body, 3 = both */
  int32_t num_workgroups;  /* grid of the kernel this plan runs */
  int32_t num_items;       /* attention work items */
  int32_t num_partial_items;
  int32_t num_partial_rows;
  int32_t num_merge_tasks;
  int32_t num_merge_sources;
  int32_t q_tile;          /* folded query rows per work item (T_q) */
  int64_t kv_chunk;        /* L_kv: longest KV chunk of a work item, tokens */
  int64_t max_wg_cost;     /* largest per-workgroup cost after assignment */
  int64_t total_cost;
  int32_t blob_bytes;      /* bytes of plan uploaded to the workspace */
  int32_t instance;        /* kernel instance the plan runs on (kind, decode rows, head dim,
                              switches); plans with equal values and num_workgroups replay
                              under one captured run */
} bsr_plan_info;

typedef struct bsr_attn* bsr_attn_t;

/* Create a handle.  device >= 0 selects a HIP device (made current during calls);
 * device = -1 creates a host-only handle that can plan (into the staging buffer,
 * nothing uploaded) but not run; it then needs num_workgroups > 0.  The handle
 * holds host state only. */
int bsr_attn_create(const bsr_attn_config* cfg, int device, bsr_attn_t* out);

/* Workspace (device) and staging (host) bytes a plan/run pair needs, fixed at create. */
int bsr_attn_workspace_size(bsr_attn_t h, size_t* device_bytes, size_t* host_bytes);

/* Plan one generation step from the lengths (Core mechanism 6): validate the index
 * arrays, choose the tile and L_kv, cut chunks, assign work longest-first, build
 * the merge map, write the plan into host_staging and enqueue its copy into
 * workspace on stream.  Before rewriting host_staging it waits for the previous
 * copy from it.  Deterministic: the same lengths give the same plan bytes.
 * When scoring the first chunking takes long (large batches), the other chunkings
 * are scored on up to five short-lived host threads, joined before the call
 * returns; the plan is the same either way.
 * Not capturable in a HIP graph.  workspace may be NULL (then nothing is uploaded,
 * and bsr_attn_run keeps launching the last plan that was; required for host-only
 * handles).  Returns BSR_ERR_CAPACITY beyond the maxima,
 * BSR_ERR_INVALID_ARG for non-monotone indptrs, last_page_len outside [1, P] for a
 * non-empty row, or (causal) a row with l_qo > l_kv. */
int bsr_attn_plan(bsr_attn_t h, const int32_t* qo_indptr, const int32_t* kv_indptr,
                  const int32_t* last_page_len, int32_t batch, void* workspace,
                  void* host_staging, void* stream);

/* bsr_attn_plan with a tree mask over each block row's new tokens, for
 * speculative decoding with a token tree (custom masks, Quick read item 1 and
 * Background of the explainer page; paper section 3.2.3).  The l_qo query tokens
 * of block row r are its last l_qo keys; token t sees key l_kv - l_qo + u only if
 * bit (t, u) of the row's mask is set, and every earlier key as usual (the causal
 * and window masks of the handle still apply).  tree_mask is a host bit array:
 * block row r's l_qo x l_qo bits, row-major (bit t * l_qo + u), start at bit
 * offset sum over r' < r of l_qo(r')^2, least significant bit first within each
 * byte.  Returns BSR_ERR_UNSUPPORTED for a block row with more than 64 query
 * tokens, BSR_ERR_INVALID_ARG for one with l_qo > l_kv or a null tree_mask, and
 * otherwise behaves as bsr_attn_plan. */
int bsr_attn_plan_tree_mask(bsr_attn_t h, const int32_t* qo_indptr, const int32_t* kv_indptr,
                            const int32_t* last_page_len, int32_t batch, const uint8_t* tree_mask,
                            void* workspace, void* host_staging, void* stream);

/* bsr_attn_plan with one page list per request and KV head (Core mechanism 1 with
 * the page table per KV head): KV head h of block row r reads the pages
 * kv_indices[kv_indptr[r * H_kv + h] .. kv_indptr[r * H_kv + h + 1]), whose last
 * page holds last_page_len[r] valid slots.  This is the plan of the pages kept
 * by bsr_attn_quest_select (kv_indptr is then its out_indptr).  kv_indptr has
 * batch * H_kv + 1 entries; max_total_kv bounds the keys of one KV head.  Same
 * validation and staging/upload contract as bsr_attn_plan. */
int bsr_attn_plan_head_pages(bsr_attn_t h, const int32_t* qo_indptr, const int32_t* kv_indptr,
                             const int32_t* last_page_len, int32_t batch, void* workspace,
                             void* host_staging, void* stream);

/* Plan over several BSR sub-matrices of one KV matrix (Core mechanism 2).  A query
 * token's keys are the union of the keys of the block rows that cover it, in format
 * order; the formats must not overlap in keys (caller contract).  Causal, windowed
 * and ALiBi handles are not supported here.  Same staging/upload contract as
 * bsr_attn_plan. */
int bsr_attn_plan_composable(bsr_attn_t h, int32_t num_formats, const bsr_format* formats,
                             int32_t total_qo, void* workspace, void* host_staging,
                             void* stream);

/* Statistics of the last plan made on this handle. */
int bsr_attn_plan_get_info(bsr_attn_t h, bsr_plan_info* info);

/* Run the last plan uploaded to a workspace: one launch of the persistent kernel on
 * stream (asynchronous).  q, k_pool, v_pool, kv_indices, o, lse (nullable) and
 * workspace are device pointers in the layouts above; kv_indices must be the array
 * the plan's kv_indptr (and format offsets) index, with page ids < the pool's page
 * count (caller contract, not checked).  No allocation, no synchronisation,
 * constant grid: capturable in a HIP graph.  A captured run replays any later plan
 * uploaded to the same workspace whose bsr_plan_info.instance and num_workgroups
 * equal those of the plan it was captured with (same pointers).  The instance
 * changes with the kernel kind and, for the decode and mixed kinds, with the
 * decode body's folded rows: 4 when every block row folds into at most 4 rows
 * (l_qo * g <= 4), else 8.  A replay that meets a plan made for another instance
 * or grid computes nothing and writes no output; bsr_attn_check then returns
 * BSR_ERR_DEVICE. */
int bsr_attn_run(bsr_attn_t h, const void* q, const void* k_pool, const void* v_pool,
                 const int32_t* kv_indices, void* o, float* lse, void* workspace,
                 void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): bsr_attn_run without a
 * workspace argument.  The workspace is a static device array of the library,
 * 64 MiB per device, held until the process ends; a handle whose
 * bsr_attn_workspace_size device bytes exceed it is rejected with
 * BSR_ERR_CAPACITY (lower max_partial_rows or the other maxima).  Each call copies
 * the plan that the handle's last plan call wrote to host_staging (which must be
 * that buffer; plan with a null workspace to skip the ordinary upload) into the
 * array, which also clears every word that must start at zero, and launches the
 * kernel on it: asynchronous on stream; no allocation.  All calls on one device
 * share its array: calls that overlap on one device (several streams or handles)
 * race.  bsr_attn_check with a null workspace reports the errors of these runs.
 * Under graph capture each replay copies host_staging's contents at replay time. */
int bsr_attn_run_static(bsr_attn_t h, const void* q, const void* k_pool, const void* v_pool,
                        const int32_t* kv_indices, void* o, float* lse, const void* host_staging,
                        void* stream);

/* Synchronise stream and report whether the device flagged an error during the
 * runs since the last upload: a bounded wait for a partial state that expired, or
 * a launch that met a plan made for another kernel instance or grid
 * (BSR_ERR_DEVICE).  BSR_OK if none.  A null workspace checks the runs of
 * bsr_attn_run_static instead. */
int bsr_attn_check(bsr_attn_t h, void* workspace, void* stream);

/* Stand-alone ⊕ of two sets of attention states (Terms "Attention State and ⊕"):
 * o_a, o_b, o: fp32 [rows, D]; lse_a, lse_b, lse: fp32 [rows] natural log.
 * (0, -inf) is the identity.  Device pointers; o/lse may alias an input. */
int bsr_attn_merge_states(const float* o_a, const float* lse_a, const float* o_b,
                          const float* lse_b, float* o, float* lse, int64_t rows,
                          int32_t head_dim, void* stream);

/* Write new K/V rows into the paged cache (Core mechanism 1, paper section
 * 3.1.1: new K/V rows are packed like the queries, then written into the BSR
 * cache).  k_new, v_new: [total_new, H_kv, D] in dtype, rows packed by
 * append_indptr (int32 [batch + 1], like qo_indptr).  The page table
 * (kv_indptr, kv_indices, last_page_len; int32, as for bsr_attn_run) describes
 * each request's KV AFTER the write: the n_r new rows of request r become its
 * last n_r tokens, row j at position tau = l_kv - n_r + j, i.e. slot tau % P of
 * page kv_indices[kv_indptr[r] + tau / P] in every head plane of k_pool / v_pool
 * ([num_pages, H_kv, P, D], dtype).  Rows without a position (n_r > l_kv) and
 * rows whose page id lies outside [0, num_pages) are not written; nothing else in
 * the pools changes.  All arrays are device memory owned by the caller.  No
 * allocation, no synchronisation: asynchronous on `stream` and capturable.
 * Returns BSR_ERR_INVALID_ARG for negative sizes, null pointers or an unknown
 * dtype, BSR_ERR_UNSUPPORTED when D times the element size is not a multiple of
 * 16 bytes. */
int bsr_attn_append_kv(const void* k_new, const void* v_new, const int32_t* append_indptr,
                       const int32_t* kv_indptr, const int32_t* kv_indices,
                       const int32_t* last_page_len, int32_t batch, int64_t total_new,
                       int32_t num_kv_heads, int32_t head_dim, int32_t page_size, int32_t dtype,
                       void* k_pool, void* v_pool, int64_t num_pages, void* stream);

/* Quest-style page-budget sparse decode (Applicable scenarios item 5 of the
 * explainer page; paper Appendix G.5): long-context decode keeps a budget of KV
 * pages per step and attends over the kept pages only.  The page choice follows
 * Quest's criterion (the pages name the method, not the rule):
 *
 * bsr_attn_page_summary writes, for every page of the page table (kv_indptr,
 * kv_indices, last_page_len as for bsr_attn_run, kv_indptr[0] = 0, num_entries =
 * kv_indptr[batch]) and every KV head, the elementwise minimum and maximum of the
 * page's valid keys: k_min, k_max [num_pages, H_kv, D] in the pool's dtype (F32
 * or BF16; exact).  Pages outside [0, num_pages) are skipped.  Run it when pages
 * fill, not every step.
 *
 * bsr_attn_quest_select chooses the pages of one decode step.  q: [batch, H_qo,
 * D] (one token per request).  A page's score for query head h is
 * sum_d max(q_d min_d, q_d max_d), an upper bound of q.k over its keys; a KV head
 * takes the largest score of its H_qo / H_kv query heads.  Per request and KV
 * head the last page is always kept and the page_budget - 1 best other pages join
 * it (ties to the earlier page); their page ids go, in logical order with the last
 * page last, to out_indices[out_indptr[r * H_kv + h] ..], a list of
 * min(n_pages(r), page_budget) ids that the caller sizes in out_indptr ([batch *
 * H_kv + 1], device).  scores: caller scratch of H_kv * num_entries floats.
 * max_pages bounds the pages of one request (at most 16385, else
 * BSR_ERR_UNSUPPORTED).  Asynchronous, no allocation, capturable.  The kept pages
 * then run through bsr_attn_plan_head_pages and bsr_attn_run. */
int bsr_attn_page_summary(const void* k_pool, const int32_t* kv_indptr, const int32_t* kv_indices,
                          const int32_t* last_page_len, int32_t batch, int64_t num_entries,
                          int32_t num_kv_heads, int32_t head_dim, int32_t page_size, int32_t dtype,
                          int64_t num_pages, void* k_min, void* k_max, void* stream);
int bsr_attn_quest_select(const void* q, const void* k_min, const void* k_max, const int32_t* kv_indptr,
                          const int32_t* kv_indices, int32_t batch, int64_t num_entries, int32_t max_pages,
                          int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                          int64_t num_pages, int32_t page_budget, const int32_t* out_indptr,
                          int32_t* out_indices, float* scores, void* stream);

void bsr_attn_destroy(bsr_attn_t h);
const char* bsr_attn_last_error(void);
int bsr_attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BSR_ATTN_H */
