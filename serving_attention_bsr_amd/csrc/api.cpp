// api.cpp -- the C ABI declared in include/bsr_attn.h.
//
// Handles hold host state only: configuration, the workspace layout fixed at
// create time (Core mechanism 7 of the FlashInfer explainer page, paper
// Appendix D.1), the last plan, and one event that guards the host staging
// buffer against being rewritten while its previous upload is in flight.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "bsr_attn.h"
#include "handle.h"
#include "kernels/registry.h"
#include "layout.h"
#include "params.h"
#include "plan.h"

using bsr::BlockRow;
using bsr::align_up;
using bsr::DeviceGuard;
using bsr::fail;
using bsr::hip_fail;
using bsr::KernelKey;
using bsr::PlanConfig;
using bsr::PlanResult;

// Default rate of the second workgroup of a CU in the two-per-CU MFMA grid, in
// sixteenths of the first's (from a sweep on MI355X; see the planner).
constexpr int32_t kSlot2Speed16 = 11;


namespace bsr {

thread_local std::string g_error;

int fail(int code, const std::string& msg) {
  g_error = msg;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  g_error = std::string(what) + ": " + hipGetErrorString(e);
  return BSR_ERR_HIP;
}

const void* find_kernel(const KernelKey& key, int* wg_per_cu) {
  static std::vector<KernelEntry> table;
  static std::once_flag once;
  std::call_once(once, [] {
    register_d64(&table);
    register_d128(&table);
    register_d256(&table);
    register_d64_var(&table);
    register_d128_var(&table);
    register_d256_var(&table);
  });
  for (const KernelEntry& e : table) {
    const KernelKey& k = e.key;
    if (k.kind == key.kind && k.bf16 == key.bf16 && k.head_dim == key.head_dim &&
        k.rows == key.rows && k.cap == key.cap && k.page1 == key.page1 && k.kv8 == key.kv8 && k.var == key.var) {
      if (wg_per_cu != nullptr) *wg_per_cu = e.wg_per_cu;
      return e.fn;
    }
  }
  return nullptr;
}

}  // namespace bsr


namespace {

int validate_config(const bsr_attn_config* c) {
  if (c == nullptr) return fail(BSR_ERR_INVALID_ARG, "config is null");
  if (c->num_qo_heads <= 0 || c->num_kv_heads <= 0 || c->num_qo_heads % c->num_kv_heads != 0)
    return fail(BSR_ERR_INVALID_ARG, "num_qo_heads must be a positive multiple of num_kv_heads");
  if (c->num_qo_heads / c->num_kv_heads > 16)
    return fail(BSR_ERR_UNSUPPORTED, "at most 16 query heads per KV head are supported");
  if (c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256)
    return fail(BSR_ERR_UNSUPPORTED, "head_dim must be 64, 128 or 256");
  if (c->page_size < 1 || c->page_size > (1 << 16))
    return fail(BSR_ERR_INVALID_ARG, "page_size must be in [1, 65536]");
  if (c->dtype != BSR_DTYPE_F32 && c->dtype != BSR_DTYPE_BF16 && c->dtype != BSR_DTYPE_BF16_KV_FP8)
    return fail(BSR_ERR_INVALID_ARG, "dtype must be BSR_DTYPE_F32, BSR_DTYPE_BF16 or BSR_DTYPE_BF16_KV_FP8");
  if (c->causal != 0 && c->causal != 1) return fail(BSR_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (!(c->logits_soft_cap >= 0.0f) || !std::isfinite(c->logits_soft_cap))
    return fail(BSR_ERR_INVALID_ARG, "logits_soft_cap must be finite and >= 0");
  if (!std::isfinite(c->sm_scale)) return fail(BSR_ERR_INVALID_ARG, "sm_scale must be finite");
  if (c->max_batch <= 0 || c->max_total_qo <= 0 || c->max_total_kv <= 0)
    return fail(BSR_ERR_INVALID_ARG, "max_batch, max_total_qo and max_total_kv must be positive");
  if (c->max_total_kv >= (int64_t(1) << 40)) return fail(BSR_ERR_INVALID_ARG, "max_total_kv too large");
  if (c->num_workgroups < 0 || c->cost_alpha < 0 || c->cost_beta < 0 || c->min_kv_chunk < 0 ||
      c->max_partial_rows < 0 || c->cost_mfma < 0 || c->slot2_speed < 0)
    return fail(BSR_ERR_INVALID_ARG, "negative tuning parameter");
  if (c->cost_mfma > 16 * 256) return fail(BSR_ERR_INVALID_ARG, "cost_mfma too large");
  if (c->slot2_speed > 64) return fail(BSR_ERR_INVALID_ARG, "slot2_speed too large");
  if (c->sliding_window < 0) return fail(BSR_ERR_INVALID_ARG, "sliding_window must be >= 0");
  if (c->static_queues != 0 && c->static_queues != 1) return fail(BSR_ERR_INVALID_ARG, "static_queues must be 0 or 1");
  if (c->alibi_slopes != nullptr)
    for (int32_t hq = 0; hq < c->num_qo_heads; ++hq)
      if (!std::isfinite(c->alibi_slopes[hq])) return fail(BSR_ERR_INVALID_ARG, "ALiBi slopes must be finite");
  return BSR_OK;
}

// Granlund-Montgomery magic for division by d (n < 2^31): q = (mulhi(m, n) + n) >> l.
void div_magic_for(uint32_t d, uint32_t* magic, int32_t* shift) {
  int l = 0;
  while ((uint64_t(1) << l) < d) ++l;
  const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1;
  *magic = static_cast<uint32_t>(m);
  *shift = l;
}

}  // namespace

extern "C" {

int bsr_attn_abi_version(void) { return BSR_ATTN_ABI_VERSION; }

const char* bsr_attn_last_error(void) { return bsr::g_error.c_str(); }

int bsr_attn_create(const bsr_attn_config* cfg, int device, bsr_attn_t* out) {
  if (out == nullptr) return fail(BSR_ERR_INVALID_ARG, "out is null");
  *out = nullptr;
  if (int rc = validate_config(cfg)) return rc;
  if (device < -1) return fail(BSR_ERR_INVALID_ARG, "device must be >= -1");
  if (device == -1 && cfg->num_workgroups <= 0)
    return fail(BSR_ERR_INVALID_ARG, "a host-only handle needs num_workgroups > 0");

  bsr_attn* h = new bsr_attn();
  h->cfg = *cfg;
  h->device = device;
  const bool bf16 = cfg->dtype != BSR_DTYPE_F32;      // Q and O
  const bool kv8 = cfg->dtype == BSR_DTYPE_BF16_KV_FP8;  // K and V as FP8 codes
  const bool cap = cfg->logits_soft_cap > 0.0f;
  const int g = cfg->num_qo_heads / cfg->num_kv_heads;

  // persistent grid per kernel kind: the resident capacity of the device, or the
  // caller's budget when it fits (Core mechanism 8, paper Appendix E)
  if (device >= 0) {
    DeviceGuard guard(device);
    if (guard.err != hipSuccess) {
      delete h;
      return hip_fail(guard.err, "hipSetDevice");
    }
    hipDeviceProp_t prop;
    hipError_t e = hipGetDeviceProperties(&prop, device);
    if (e != hipSuccess) {
      delete h;
      return hip_fail(e, "hipGetDeviceProperties");
    }
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
      delete h;
      return fail(BSR_ERR_UNSUPPORTED, std::string("kernels are built for gfx950, device is ") + prop.gcnArchName);
    }
    const int cus = prop.multiProcessorCount;
    h->cus = cus;
    for (int kind = bsr::kKindDecode; kind <= bsr::kKindMixed; ++kind) {
      for (int ri = 0; ri < 4; ++ri) {
        const bool var = ri >= 2;
        KernelKey key{kind, bf16, cfg->head_dim, kind == bsr::kKindMfma ? ri % 2 : (ri % 2 == 0 ? 4 : 8), cap,
                      kind == bsr::kKindMfma && cfg->page_size == 1, kv8, var};
        int preferred = 1;
        const void* fn = bsr::find_kernel(key, &preferred);
        if (fn == nullptr) continue;  // instance not built for this configuration
        int per_cu = 0;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, bsr::kWgThreads, 0);
        if (e != hipSuccess) {
          delete h;
          return hip_fail(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
        }
        // the merge phase waits on other workgroups, so the grid never exceeds
        // what stays resident; a caller's budget is capped per instance
        const int resident = per_cu * cus;
        if (resident <= 0) continue;
        int32_t& nwg = h->num_wg[kind][ri % 2][var ? 1 : 0];
        if (cfg->num_workgroups > 0) {
          nwg = std::min(cfg->num_workgroups, resident);
        } else {
          nwg = std::min(per_cu, std::max(preferred, 1)) * cus;
        }
      }
    }
    // the static scratch of bsr_attn_run_static: its device address is looked up
    // once per device, here, with the device current
    {
      uint8_t* scratch = nullptr;
      int64_t scratch_bytes = 0;
      if (int rc = bsr::static_scratch(device, &scratch, &scratch_bytes)) {
        delete h;
        return rc;
      }
    }
    e = hipEventCreateWithFlags(&h->upload_done, hipEventDisableTiming);
    if (e != hipSuccess) {
      delete h;
      return hip_fail(e, "hipEventCreateWithFlags");
    }
  } else {
    for (int kind = 1; kind <= 3; ++kind)
      for (int ri = 0; ri < 2; ++ri) h->num_wg[kind][ri][0] = h->num_wg[kind][ri][1] = cfg->num_workgroups;
  }
  int32_t max_wg = 1;
  for (int kind = 1; kind <= 3; ++kind)
    for (int ri = 0; ri < 2; ++ri) max_wg = std::max({max_wg, h->num_wg[kind][ri][0], h->num_wg[kind][ri][1]});

  PlanConfig& pc = h->pc;
  pc.h_qo = cfg->num_qo_heads;
  pc.h_kv = cfg->num_kv_heads;
  pc.group = g;
  pc.head_dim = cfg->head_dim;
  pc.page_size = cfg->page_size;
  pc.causal = cfg->causal != 0;
  pc.bf16 = bf16;
  pc.cap = cap;
  pc.kv8 = kv8;
  pc.static_queues = cfg->static_queues != 0;
  std::memcpy(pc.num_wg, h->num_wg, sizeof(pc.num_wg));
  pc.alpha = cfg->cost_alpha > 0 ? cfg->cost_alpha : 1;
  pc.beta = cfg->cost_beta > 0 ? cfg->cost_beta : 1;
  pc.min_chunk = cfg->min_kv_chunk > 0 ? cfg->min_kv_chunk : 64;
  pc.gamma = cfg->cost_item > 0 ? cfg->cost_item : (cfg->cost_item < 0 ? 0 : 512);
  // Default from a sweep on MI355X (shared-prefix batches, D = 64, 128, 256): the
  // mixed grid runs fastest once MFMA pieces get workgroups of their own, which
  // every weight from 10x up gives; 12x is used.
  pc.mfma_w16 = cfg->cost_mfma > 0 ? cfg->cost_mfma : 192;
  pc.cus = h->cus;
  pc.slot2_speed16 = cfg->slot2_speed > 0 ? cfg->slot2_speed : kSlot2Speed16;
  pc.window = cfg->sliding_window;
  // ALiBi slopes in the units of the unscaled logit q.k: the kernels add
  // (slope / sm_scale) * (j - p) before applying the scale
  const float sm = cfg->sm_scale > 0.0f ? cfg->sm_scale : 1.0f / std::sqrt(float(cfg->head_dim));
  if (cfg->alibi_slopes != nullptr) {
    pc.alibi_raw.resize(cfg->num_qo_heads);
    for (int32_t hq = 0; hq < cfg->num_qo_heads; ++hq) pc.alibi_raw[hq] = cfg->alibi_slopes[hq] / sm;
  }
  h->cfg.alibi_slopes = nullptr;  // read at create only
  pc.max_batch = cfg->max_batch;
  pc.max_total_qo = cfg->max_total_qo;
  pc.max_total_kv = cfg->max_total_kv;
  // partial states: at most 2 * #WG chunks of split units, each at most one tile
  // of folded rows (paper Appendix D.3), plus, for composed formats, one state per
  // format for every query token and query head (two formats: the shared-prefix
  // case; more formats need max_partial_rows)
  const int64_t tile_max = bsr::mfma_tile(cfg->head_dim);
  pc.max_partial_rows = cfg->max_partial_rows > 0
                            ? cfg->max_partial_rows
                            : 2LL * max_wg * tile_max + 2LL * cfg->max_total_qo * cfg->num_qo_heads;
  // plan segment: header, status, epochs, flags, queues, items, merge map
  const int64_t hk = cfg->num_kv_heads;
  const int64_t units = hk * (2LL * cfg->max_batch + (int64_t(cfg->max_total_qo) * g + 31) / 32);
  const int64_t max_items = units + 2LL * max_wg + 64;
  const int64_t max_tasks = int64_t(cfg->max_total_qo) * hk;
  const int64_t max_srcs = 2 * max_tasks + 2LL * max_wg * tile_max;
  // (+ ALiBi slopes and one tree-mask row per query token)
  int64_t cap_bytes = sizeof(bsr::PlanHeader) + 16 + 16 + 4LL * max_wg + 4 * max_items +
                      2 * 4LL * (max_wg + 1) + int64_t(sizeof(bsr::WorkItem)) * max_items +
                      int64_t(sizeof(bsr::MergeTask)) * max_tasks +
                      int64_t(sizeof(bsr::MergeSrc)) * max_srcs + 4LL * cfg->num_qo_heads +
                      8LL * cfg->max_total_qo + 16 * 16;
  h->plan_capacity = align_up(cap_bytes, 256);
  pc.blob_capacity = h->plan_capacity;
  h->partial_o_off = h->plan_capacity;
  h->partial_lse_off = align_up(h->partial_o_off + pc.max_partial_rows * cfg->head_dim * 4, 256);
  h->ws_bytes = align_up(h->partial_lse_off + pc.max_partial_rows * 4, 256);
#ifdef BSR_TRACE
  h->ws_bytes += align_up(int64_t(max_wg) * 64, 256);  // 8 stamps per workgroup
#endif

  bsr::RunParams& p = h->params;
  std::memset(&p, 0, sizeof(p));
  p.h_qo = cfg->num_qo_heads;
  p.h_kv = cfg->num_kv_heads;
  p.group = g;
  p.page_size = cfg->page_size;
  div_magic_for(static_cast<uint32_t>(cfg->page_size), &p.page_magic, &p.page_shift);
  const float scale = cfg->sm_scale > 0.0f ? cfg->sm_scale : 1.0f / std::sqrt(float(cfg->head_dim));
  p.sm_scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.cap = cfg->logits_soft_cap;
  p.cap_inv = cap ? 1.0f / cfg->logits_soft_cap : 0.0f;
  p.cap_log2 = cfg->logits_soft_cap * 1.4426950408889634f;
  p.partial_o_off = h->partial_o_off;
  p.partial_lse_off = h->partial_lse_off;
#ifdef BSR_TRACE
  p.trace_off = align_up(h->partial_lse_off + pc.max_partial_rows * 4, 256);
#endif
  *out = h;
  return BSR_OK;
}

int bsr_attn_workspace_size(bsr_attn_t h, size_t* device_bytes, size_t* host_bytes) {
  if (h == nullptr) return fail(BSR_ERR_INVALID_ARG, "handle is null");
  if (device_bytes) *device_bytes = static_cast<size_t>(h->ws_bytes);
  if (host_bytes) *host_bytes = static_cast<size_t>(h->plan_capacity);
  return BSR_OK;
}

static int finish_plan(bsr_attn_t h, std::vector<BlockRow>& rows, int32_t total_qo, bool composable,
                       void* workspace, void* host_staging, void* stream,
                       const std::vector<uint64_t>* tree_rows = nullptr) {
  if (host_staging == nullptr) return fail(BSR_ERR_INVALID_ARG, "host_staging is null");
  if (workspace != nullptr && h->device < 0)
    return fail(BSR_ERR_INVALID_ARG, "a host-only handle cannot upload to a workspace");
  PlanResult res;
  std::string err;
  int rc = bsr::make_plan(h->pc, rows, total_qo, composable, &res, &err, tree_rows);
  if (rc != BSR_OK) return fail(rc, err);
  const int rows_key = res.kernel == bsr::kKindMfma ? (res.short_tile ? 1 : 0) : res.decode_rows;
  const void* fn = nullptr;
  if (h->device >= 0) {
    fn = bsr::find_kernel(KernelKey{res.kernel, h->pc.bf16, h->pc.head_dim, rows_key,
                                    h->cfg.logits_soft_cap > 0.0f,
                                    res.kernel == bsr::kKindMfma && h->pc.page_size == 1, h->pc.kv8, res.var});
    if (fn == nullptr)
      return fail(BSR_ERR_UNSUPPORTED, "no kernel built for this plan's kind " + std::to_string(res.kernel));
  }
  DeviceGuard guard(h->device);
  if (guard.err != hipSuccess) return hip_fail(guard.err, "hipSetDevice");
  if (h->upload_pending) {
    hipError_t e = hipEventSynchronize(h->upload_done);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    h->upload_pending = false;
  }
  std::memcpy(host_staging, res.blob.data(), res.blob.size());
  h->last_staging = host_staging;
  h->last_kernel = fn;
  if (workspace != nullptr) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(workspace, host_staging, res.blob.size(), hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync");
    e = hipEventRecord(h->upload_done, s);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
    h->upload_pending = true;
  }
  if (workspace != nullptr) {
    // run() launches what the workspace holds: only an uploaded plan changes it
    bsr::PlanHeader hdr;
    std::memcpy(&hdr, res.blob.data(), sizeof(hdr));
    h->off_status = hdr.off_status;
    h->kernel = fn;
    h->run_wg = res.num_wg;
    h->has_upload = true;
  }
  h->last = std::move(res);
  h->has_plan = true;
  return BSR_OK;
}

// Block rows of a single-format plan, validated (see bsr_attn_plan).
static int single_format_rows(bsr_attn_t h, const int32_t* qo_indptr, const int32_t* kv_indptr,
                              const int32_t* last_page_len, int32_t batch, std::vector<BlockRow>* out,
                              int32_t* total_qo_out) {
  if (h == nullptr) return fail(BSR_ERR_INVALID_ARG, "handle is null");
  if (batch < 0) return fail(BSR_ERR_INVALID_ARG, "batch must be >= 0");
  if (batch > h->cfg.max_batch) return fail(BSR_ERR_CAPACITY, "batch exceeds max_batch");
  if (batch > 0 && (qo_indptr == nullptr || kv_indptr == nullptr || last_page_len == nullptr))
    return fail(BSR_ERR_INVALID_ARG, "index array is null");
  const int32_t P = h->cfg.page_size;
  std::vector<BlockRow> rows(batch);
  if (batch > 0 && qo_indptr[0] != 0) return fail(BSR_ERR_INVALID_ARG, "qo_indptr[0] must be 0");
  if (batch > 0 && kv_indptr[0] < 0) return fail(BSR_ERR_INVALID_ARG, "kv_indptr[0] must be >= 0");
  int64_t total_kv = 0;
  for (int32_t r = 0; r < batch; ++r) {
    const int64_t lq = int64_t(qo_indptr[r + 1]) - qo_indptr[r];
    const int64_t np = int64_t(kv_indptr[r + 1]) - kv_indptr[r];
    if (lq < 0 || np < 0) return fail(BSR_ERR_INVALID_ARG, "indptr arrays must be non-decreasing");
    int64_t lkv = 0;
    if (np > 0) {
      if (last_page_len[r] < 1 || last_page_len[r] > P)
        return fail(BSR_ERR_INVALID_ARG, "last_page_len[" + std::to_string(r) + "] outside [1, page_size]");
      lkv = (np - 1) * P + last_page_len[r];
    }
    if (lkv >= (int64_t(1) << 30)) return fail(BSR_ERR_UNSUPPORTED, "a block row holds 2^30 keys or more");
    if (h->cfg.causal && lq > lkv)
      return fail(BSR_ERR_INVALID_ARG, "causal block row " + std::to_string(r) + " has more queries than keys");
    total_kv += lkv;
    rows[r].qo_begin = qo_indptr[r];
    rows[r].qo_len = static_cast<int32_t>(lq);
    rows[r].page_begin = kv_indptr[r];
    rows[r].kv_len = static_cast<int32_t>(lkv);
    rows[r].format = 0;
  }
  const int32_t total_qo = batch > 0 ? qo_indptr[batch] : 0;
  if (total_qo > h->cfg.max_total_qo) return fail(BSR_ERR_CAPACITY, "sum of query lengths exceeds max_total_qo");
  if (total_kv > h->cfg.max_total_kv) return fail(BSR_ERR_CAPACITY, "sum of KV lengths exceeds max_total_kv");
  *out = std::move(rows);
  *total_qo_out = total_qo;
  return BSR_OK;
}

int bsr_attn_plan(bsr_attn_t h, const int32_t* qo_indptr, const int32_t* kv_indptr,
                  const int32_t* last_page_len, int32_t batch, void* workspace, void* host_staging,
                  void* stream) {
  std::vector<BlockRow> rows;
  int32_t total_qo = 0;
  if (int rc = single_format_rows(h, qo_indptr, kv_indptr, last_page_len, batch, &rows, &total_qo)) return rc;
  return finish_plan(h, rows, total_qo, false, workspace, host_staging, stream);
}

int bsr_attn_plan_tree_mask(bsr_attn_t h, const int32_t* qo_indptr, const int32_t* kv_indptr,
                            const int32_t* last_page_len, int32_t batch, const uint8_t* tree_mask,
                            void* workspace, void* host_staging, void* stream) {
  std::vector<BlockRow> rows;
  int32_t total_qo = 0;
  if (int rc = single_format_rows(h, qo_indptr, kv_indptr, last_page_len, batch, &rows, &total_qo)) return rc;
  if (batch > 0 && tree_mask == nullptr) return fail(BSR_ERR_INVALID_ARG, "tree_mask is null");
  // one 64-bit row per query token: bit u = the token sees key l_kv - l_qo + u
  std::vector<uint64_t> tree(total_qo, 0);
  int64_t bit = 0;
  for (int32_t r = 0; r < batch; ++r) {
    BlockRow& br = rows[r];
    const int32_t n = br.qo_len;
    if (n > bsr::kMaxTreeTokens)
      return fail(BSR_ERR_UNSUPPORTED, "block row " + std::to_string(r) + " has more than 64 tree-masked tokens");
    if (n > br.kv_len)
      return fail(BSR_ERR_INVALID_ARG, "block row " + std::to_string(r) + " has more tree tokens than keys");
    br.tree = n > 0;
    for (int32_t t = 0; t < n; ++t) {
      uint64_t row = 0;
      for (int32_t u = 0; u < n; ++u, ++bit)
        if ((tree_mask[bit >> 3] >> (bit & 7)) & 1) row |= uint64_t(1) << u;
      tree[br.qo_begin + t] = row;
    }
  }
  return finish_plan(h, rows, total_qo, false, workspace, host_staging, stream, &tree);
}

int bsr_attn_plan_head_pages(bsr_attn_t h, const int32_t* qo_indptr, const int32_t* kv_indptr,
                             const int32_t* last_page_len, int32_t batch, void* workspace, void* host_staging,
                             void* stream) {
  if (h == nullptr) return fail(BSR_ERR_INVALID_ARG, "handle is null");
  if (batch < 0) return fail(BSR_ERR_INVALID_ARG, "batch must be >= 0");
  if (batch > h->cfg.max_batch) return fail(BSR_ERR_CAPACITY, "batch exceeds max_batch");
  if (batch > 0 && (qo_indptr == nullptr || kv_indptr == nullptr || last_page_len == nullptr))
    return fail(BSR_ERR_INVALID_ARG, "index array is null");
  const int32_t P = h->cfg.page_size;
  const int32_t hk = h->cfg.num_kv_heads;
  if (batch > 0 && qo_indptr[0] != 0) return fail(BSR_ERR_INVALID_ARG, "qo_indptr[0] must be 0");
  if (batch > 0 && kv_indptr[0] < 0) return fail(BSR_ERR_INVALID_ARG, "kv_indptr[0] must be >= 0");
  std::vector<BlockRow> rows;
  rows.reserve(static_cast<size_t>(batch) * hk);
  int64_t total_kv = 0;
  for (int32_t r = 0; r < batch; ++r) {
    const int64_t lq = int64_t(qo_indptr[r + 1]) - qo_indptr[r];
    if (lq < 0) return fail(BSR_ERR_INVALID_ARG, "qo_indptr must be non-decreasing");
    for (int32_t head = 0; head < hk; ++head) {
      const int64_t e = int64_t(r) * hk + head;
      const int64_t np = int64_t(kv_indptr[e + 1]) - kv_indptr[e];
      if (np < 0) return fail(BSR_ERR_INVALID_ARG, "kv_indptr must be non-decreasing");
      int64_t lkv = 0;
      if (np > 0) {
        if (last_page_len[r] < 1 || last_page_len[r] > P)
          return fail(BSR_ERR_INVALID_ARG, "last_page_len[" + std::to_string(r) + "] outside [1, page_size]");
        lkv = (np - 1) * P + last_page_len[r];
      }
      if (lkv >= (int64_t(1) << 30)) return fail(BSR_ERR_UNSUPPORTED, "a block row holds 2^30 keys or more");
      if (h->cfg.causal && lq > lkv)
        return fail(BSR_ERR_INVALID_ARG, "causal block row " + std::to_string(r) + " has more queries than keys");
      total_kv += lkv;
      BlockRow br;
      br.qo_begin = qo_indptr[r];
      br.qo_len = static_cast<int32_t>(lq);
      br.page_begin = kv_indptr[e];
      br.kv_len = static_cast<int32_t>(lkv);
      br.head = head;
      rows.push_back(br);
    }
  }
  const int32_t total_qo = batch > 0 ? qo_indptr[batch] : 0;
  if (total_qo > h->cfg.max_total_qo) return fail(BSR_ERR_CAPACITY, "sum of query lengths exceeds max_total_qo");
  // (per-head rows: a request's keys count once per KV head)
  if (total_kv > h->cfg.max_total_kv * hk)
    return fail(BSR_ERR_CAPACITY, "KV lengths exceed max_total_kv per KV head");
  return finish_plan(h, rows, total_qo, false, workspace, host_staging, stream);
}

int bsr_attn_plan_composable(bsr_attn_t h, int32_t num_formats, const bsr_format* formats,
                             int32_t total_qo, void* workspace, void* host_staging, void* stream) {
  if (h == nullptr) return fail(BSR_ERR_INVALID_ARG, "handle is null");
  if (h->cfg.causal) return fail(BSR_ERR_UNSUPPORTED, "composed formats are not supported with causal masking");
  if (h->cfg.sliding_window > 0)
    return fail(BSR_ERR_UNSUPPORTED, "composed formats are not supported with a sliding window");
  if (!h->pc.alibi_raw.empty())
    return fail(BSR_ERR_UNSUPPORTED, "composed formats are not supported with ALiBi");
  if (num_formats < 1 || formats == nullptr) return fail(BSR_ERR_INVALID_ARG, "need at least one format");
  if (total_qo < 0 || total_qo > h->cfg.max_total_qo)
    return fail(total_qo < 0 ? BSR_ERR_INVALID_ARG : BSR_ERR_CAPACITY, "total_qo outside [0, max_total_qo]");
  const int32_t P = h->cfg.page_size;
  std::vector<BlockRow> rows;
  int64_t total_kv = 0;
  for (int32_t f = 0; f < num_formats; ++f) {
    const bsr_format& fm = formats[f];
    if (fm.num_block_rows < 0) return fail(BSR_ERR_INVALID_ARG, "num_block_rows must be >= 0");
    if (fm.num_block_rows > 0 && (fm.qo_indptr == nullptr || fm.kv_indptr == nullptr || fm.last_page_len == nullptr))
      return fail(BSR_ERR_INVALID_ARG, "format index array is null");
    if (fm.kv_indices_offset < 0) return fail(BSR_ERR_INVALID_ARG, "kv_indices_offset must be >= 0");
    for (int32_t r = 0; r < fm.num_block_rows; ++r) {
      const int64_t q0 = fm.qo_indptr[r], q1 = fm.qo_indptr[r + 1];
      const int64_t np = int64_t(fm.kv_indptr[r + 1]) - fm.kv_indptr[r];
      if (q0 < 0 || q1 < q0 || q1 > total_qo || np < 0 || fm.kv_indptr[r] < 0)
        return fail(BSR_ERR_INVALID_ARG, "format " + std::to_string(f) + " has malformed indptr arrays");
      int64_t lkv = 0;
      if (np > 0) {
        if (fm.last_page_len[r] < 1 || fm.last_page_len[r] > P)
          return fail(BSR_ERR_INVALID_ARG, "format " + std::to_string(f) + " last_page_len outside [1, page_size]");
        lkv = (np - 1) * P + fm.last_page_len[r];
      }
      if (lkv >= (int64_t(1) << 30)) return fail(BSR_ERR_UNSUPPORTED, "a block row holds 2^30 keys or more");
      total_kv += lkv;
      BlockRow br;
      br.qo_begin = static_cast<int32_t>(q0);
      br.qo_len = static_cast<int32_t>(q1 - q0);
      br.page_begin = fm.kv_indices_offset + fm.kv_indptr[r];
      br.kv_len = static_cast<int32_t>(lkv);
      br.format = f;
      rows.push_back(br);
    }
  }
  if (static_cast<int64_t>(rows.size()) > h->cfg.max_batch)
    return fail(BSR_ERR_CAPACITY, "block rows of all formats exceed max_batch");
  if (total_kv > h->cfg.max_total_kv) return fail(BSR_ERR_CAPACITY, "sum of KV lengths exceeds max_total_kv");
  return finish_plan(h, rows, total_qo, true, workspace, host_staging, stream);
}

int bsr_attn_plan_get_info(bsr_attn_t h, bsr_plan_info* info) {
  if (h == nullptr || info == nullptr) return fail(BSR_ERR_INVALID_ARG, "null argument");
  if (!h->has_plan) return fail(BSR_ERR_INVALID_ARG, "no plan has been made on this handle");
  std::memset(info, 0, sizeof(*info));
  const PlanResult& r = h->last;
  info->kernel = r.kernel;
  info->num_workgroups = r.num_wg;
  info->num_items = r.num_items;
  info->num_partial_items = r.num_partial_items;
  info->num_partial_rows = static_cast<int32_t>(r.num_partial_rows);
  info->num_merge_tasks = r.num_merge;
  info->num_merge_sources = r.num_srcs;
  info->q_tile = r.q_tile;
  info->kv_chunk = r.kv_chunk;
  info->max_wg_cost = r.max_wg_cost;
  info->total_cost = r.total_cost;
  info->blob_bytes = static_cast<int32_t>(r.blob.size());
  bsr::PlanHeader hdr;
  std::memcpy(&hdr, r.blob.data(), sizeof(hdr));
  info->instance = hdr.instance;
  return BSR_OK;
}

int bsr_attn_run(bsr_attn_t h, const void* q, const void* k_pool, const void* v_pool,
                 const int32_t* kv_indices, void* o, float* lse, void* workspace, void* stream) {
  if (h == nullptr) return fail(BSR_ERR_INVALID_ARG, "handle is null");
  if (h->device < 0) return fail(BSR_ERR_INVALID_ARG, "a host-only handle cannot run");
  if (!h->has_upload) return fail(BSR_ERR_INVALID_ARG, "run before any plan was uploaded to a workspace");
  if (q == nullptr || k_pool == nullptr || v_pool == nullptr || kv_indices == nullptr || o == nullptr ||
      workspace == nullptr)
    return fail(BSR_ERR_INVALID_ARG, "null device pointer");
  DeviceGuard guard(h->device);
  if (guard.err != hipSuccess) return hip_fail(guard.err, "hipSetDevice");
  bsr::RunParams p = h->params;
  p.q = q;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.kv_indices = kv_indices;
  p.o = o;
  p.lse = lse;
  p.ws = static_cast<uint8_t*>(workspace);
  void* args[] = {&p};
  hipError_t e = hipLaunchKernel(h->kernel, dim3(static_cast<uint32_t>(h->run_wg)),
                                 dim3(bsr::kWgThreads), args, 0, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "hipLaunchKernel");
  return BSR_OK;
}

int bsr_attn_check(bsr_attn_t h, void* workspace, void* stream) {
  if (h == nullptr) return fail(BSR_ERR_INVALID_ARG, "null argument");
  if (h->device < 0) return fail(BSR_ERR_INVALID_ARG, "a host-only handle has no device state");
  // a null workspace checks the runs of bsr_attn_run_static (the static scratch)
  const bool scratch = workspace == nullptr;
  if (scratch ? !h->has_static : !h->has_upload) return BSR_OK;
  DeviceGuard guard(h->device);
  if (guard.err != hipSuccess) return hip_fail(guard.err, "hipSetDevice");
  uint8_t* base = static_cast<uint8_t*>(workspace);
  if (scratch) {
    int64_t bytes = 0;
    if (int rc = bsr::static_scratch(h->device, &base, &bytes)) return rc;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  int32_t status[4] = {0, 0, 0, 0};
  e = hipMemcpy(status, base + (scratch ? h->static_off_status : h->off_status), sizeof(status),
                hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy");
  if (status[bsr::kStatusWrongKernel] != 0)
    return fail(BSR_ERR_DEVICE,
                "the workspace holds a plan made for another kernel instance or grid than the one launched "
                "(a captured run replayed after a plan that needs a different instance); nothing was computed");
  if (status[bsr::kStatusWaitTimeout] != 0)
    return fail(BSR_ERR_DEVICE, "a merge task gave up waiting for a partial state (workgroups not co-resident?)");
  return BSR_OK;
}

extern int bsr_launch_merge_states(const float*, const float*, const float*, const float*, float*,
                                   float*, int64_t, int32_t, hipStream_t);

int bsr_attn_merge_states(const float* o_a, const float* lse_a, const float* o_b, const float* lse_b,
                          float* o, float* lse, int64_t rows, int32_t head_dim, void* stream) {
  if (rows < 0 || head_dim <= 0) return fail(BSR_ERR_INVALID_ARG, "rows must be >= 0 and head_dim > 0");
  if (rows > 0 && (o_a == nullptr || lse_a == nullptr || o_b == nullptr || lse_b == nullptr || o == nullptr ||
                   lse == nullptr))
    return fail(BSR_ERR_INVALID_ARG, "null device pointer");
  if (bsr_launch_merge_states(o_a, lse_a, o_b, lse_b, o, lse, rows, head_dim, static_cast<hipStream_t>(stream)) != 0)
    return fail(BSR_ERR_HIP, "merge_states launch failed");
  return BSR_OK;
}

extern int bsr_launch_append_kv(const void*, const void*, const int32_t*, const int32_t*, const int32_t*,
                                const int32_t*, int32_t, int64_t, int32_t, int32_t, int32_t, int64_t, void*, void*,
                                hipStream_t);

int bsr_attn_append_kv(const void* k_new, const void* v_new, const int32_t* append_indptr, const int32_t* kv_indptr,
                       const int32_t* kv_indices, const int32_t* last_page_len, int32_t batch, int64_t total_new,
                       int32_t num_kv_heads, int32_t head_dim, int32_t page_size, int32_t dtype, void* k_pool,
                       void* v_pool, int64_t num_pages, void* stream) {
  if (batch < 0 || total_new < 0 || num_pages < 0)
    return fail(BSR_ERR_INVALID_ARG, "batch, total_new and num_pages must be >= 0");
  if (num_kv_heads <= 0 || head_dim <= 0 || page_size <= 0)
    return fail(BSR_ERR_INVALID_ARG, "num_kv_heads, head_dim and page_size must be > 0");
  if (dtype != BSR_DTYPE_F32 && dtype != BSR_DTYPE_BF16 && dtype != BSR_DTYPE_BF16_KV_FP8)
    return fail(BSR_ERR_INVALID_ARG, "dtype must be F32, BF16 or BF16_KV_FP8");
  const int64_t row_bytes = int64_t(head_dim) * (dtype == BSR_DTYPE_F32 ? 4 : (dtype == BSR_DTYPE_BF16 ? 2 : 1));
  if (row_bytes % 16 != 0) return fail(BSR_ERR_UNSUPPORTED, "head_dim * element size must be a multiple of 16 bytes");
  if (total_new == 0 || batch == 0) return BSR_OK;
  if (k_new == nullptr || v_new == nullptr || append_indptr == nullptr || kv_indptr == nullptr ||
      kv_indices == nullptr || last_page_len == nullptr || k_pool == nullptr || v_pool == nullptr)
    return fail(BSR_ERR_INVALID_ARG, "null device pointer");
  if (bsr_launch_append_kv(k_new, v_new, append_indptr, kv_indptr, kv_indices, last_page_len, batch, total_new,
                           num_kv_heads, static_cast<int32_t>(row_bytes), page_size, num_pages, k_pool, v_pool,
                           static_cast<hipStream_t>(stream)) != 0)
    return fail(BSR_ERR_HIP, "append_kv launch failed");
  return BSR_OK;
}

extern int bsr_launch_page_summary(const void*, const int32_t*, const int32_t*, const int32_t*, int32_t, int64_t,
                                   int32_t, int32_t, int32_t, int32_t, int64_t, void*, void*, hipStream_t);
extern int bsr_launch_quest_select(const void*, const void*, const void*, const int32_t*, const int32_t*, int32_t,
                                   int64_t, int32_t, int32_t, int32_t, int32_t, int64_t, int32_t, const int32_t*,
                                   int32_t*, float*, hipStream_t);

// Quest page choice: the select kernel keeps one request's candidate keys in LDS.
constexpr int32_t kQuestMaxPages = 16384 + 1;

int bsr_attn_page_summary(const void* k_pool, const int32_t* kv_indptr, const int32_t* kv_indices,
                          const int32_t* last_page_len, int32_t batch, int64_t num_entries, int32_t num_kv_heads,
                          int32_t head_dim, int32_t page_size, int32_t dtype, int64_t num_pages, void* k_min,
                          void* k_max, void* stream) {
  if (batch < 0 || num_entries < 0 || num_pages < 0) return fail(BSR_ERR_INVALID_ARG, "negative size");
  if (num_kv_heads <= 0 || head_dim <= 0 || page_size <= 0)
    return fail(BSR_ERR_INVALID_ARG, "num_kv_heads, head_dim and page_size must be > 0");
  if (dtype != BSR_DTYPE_F32 && dtype != BSR_DTYPE_BF16)
    return fail(BSR_ERR_UNSUPPORTED, "page summaries support F32 and BF16 pools");
  if (batch == 0 || num_entries == 0) return BSR_OK;
  if (k_pool == nullptr || kv_indptr == nullptr || kv_indices == nullptr || last_page_len == nullptr ||
      k_min == nullptr || k_max == nullptr)
    return fail(BSR_ERR_INVALID_ARG, "null device pointer");
  if (bsr_launch_page_summary(k_pool, kv_indptr, kv_indices, last_page_len, batch, num_entries, num_kv_heads,
                              head_dim, page_size, dtype == BSR_DTYPE_F32 ? 4 : 2, num_pages, k_min, k_max,
                              static_cast<hipStream_t>(stream)) != 0)
    return fail(BSR_ERR_HIP, "page_summary launch failed");
  return BSR_OK;
}

int bsr_attn_quest_select(const void* q, const void* k_min, const void* k_max, const int32_t* kv_indptr,
                          const int32_t* kv_indices, int32_t batch, int64_t num_entries, int32_t max_pages,
                          int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                          int64_t num_pages, int32_t page_budget, const int32_t* out_indptr, int32_t* out_indices,
                          float* scores, void* stream) {
  if (batch < 0 || num_entries < 0 || num_pages < 0 || max_pages < 0)
    return fail(BSR_ERR_INVALID_ARG, "negative size");
  if (num_qo_heads <= 0 || num_kv_heads <= 0 || num_qo_heads % num_kv_heads != 0)
    return fail(BSR_ERR_INVALID_ARG, "num_qo_heads must be a positive multiple of num_kv_heads");
  if (head_dim != 64 && head_dim != 128 && head_dim != 256)
    return fail(BSR_ERR_UNSUPPORTED, "head_dim must be 64, 128 or 256");
  if (dtype != BSR_DTYPE_F32 && dtype != BSR_DTYPE_BF16)
    return fail(BSR_ERR_UNSUPPORTED, "the page choice supports F32 and BF16 queries and summaries");
  if (page_budget < 1) return fail(BSR_ERR_INVALID_ARG, "page_budget must be >= 1");
  if (max_pages > kQuestMaxPages)
    return fail(BSR_ERR_UNSUPPORTED, "a request holds more than 16385 pages (the page choice keeps one "
                                     "request's candidates on chip)");
  if (batch == 0) return BSR_OK;
  if (q == nullptr || k_min == nullptr || k_max == nullptr || kv_indptr == nullptr || kv_indices == nullptr ||
      out_indptr == nullptr || out_indices == nullptr || (num_entries > 0 && scores == nullptr))
    return fail(BSR_ERR_INVALID_ARG, "null device pointer");
  if (bsr_launch_quest_select(q, k_min, k_max, kv_indptr, kv_indices, batch, num_entries, num_qo_heads,
                              num_kv_heads, head_dim, dtype == BSR_DTYPE_F32 ? 4 : 2, num_pages, page_budget,
                              out_indptr, out_indices, scores, static_cast<hipStream_t>(stream)) != 0)
    return fail(BSR_ERR_HIP, "quest_select launch failed");
  return BSR_OK;
}

void bsr_attn_destroy(bsr_attn_t h) {
  if (h == nullptr) return;
  if (h->upload_done != nullptr) {
    if (h->upload_pending) (void)hipEventSynchronize(h->upload_done);
    (void)hipEventDestroy(h->upload_done);
  }
  delete h;
}

}  // extern "C"
