// params.h -- launch arguments of the persistent kernel (host and device).
#pragma once

#include <stdint.h>

namespace bsr {

// Pointers and handle constants only, so one captured launch replays any later
// plan of the same kernel.
struct RunParams {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* kv_indices;
  void* o;
  float* lse;        // may be null
  uint8_t* ws;       // workspace base: plan blob at offset 0
  int64_t partial_o_off;
  int64_t partial_lse_off;
  int32_t h_qo, h_kv, group, page_size;
  uint32_t page_magic;  // division by page_size: q = (mulhi(magic, n) + n) >> shift
  int32_t page_shift;
  float scale_log2;     // sm_scale * log2(e), used when there is no soft-cap
  float sm_scale;
  float cap;            // soft-cap (0: off)
  float cap_inv;
  float cap_log2;       // cap * log2(e)
  int32_t pad;
  int64_t trace_off;    // workspace offset of the optional timeline (trace builds only)
};

struct KernelKey {
  int kind;  // KernelKind
  bool bf16;
  int head_dim;
  int rows;  // decode-body folded rows; tile kernel: 0 = 128-row tile, 1 = 64-row tile (D = 128)
  bool cap;
  bool page1 = false;  // instance specialised for one key per page (MFMA kind only)
  bool kv8 = false;    // K/V are FP8 E4M3 codes, Q/O bf16 (decode kind only)
  bool var = false;    // plans with ALiBi slopes or tree masks
};

// Host stub of the matching persistent kernel, or null if not built; the
// instance's preferred workgroups per CU go to *wg_per_cu when non-null.
const void* find_kernel(const KernelKey& key, int* wg_per_cu = nullptr);

}  // namespace bsr
