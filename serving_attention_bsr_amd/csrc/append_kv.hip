// append_kv.hip -- write new K/V rows into the paged (BSR) cache.
//
// Core mechanism 1 of the FlashInfer explainer page (paper section 3.1.1, Figure
// 2): newly generated K/V rows are packed like the queries, addressed by the
// queries' indptr, and then written into the BSR KV cache.  The new tokens of
// request r are the last n_r tokens of its KV as the page table describes it
// after the write: new token j goes to logical position tau = l_kv - n_r + j,
// slot tau % P of page kv_indices[kv_indptr[r] + tau / P], in every head plane.
//
// The write is a scatter of whole rows and is bound by HBM: every byte is read
// once and written once.  One wavefront takes a contiguous range of new tokens,
// finds the first token's request by binary search over append_indptr (scalar
// loads: the index arrays are read-only here) and then steps forward; its lanes
// copy the token's K and V rows of all heads in 16-byte pieces.  Tokens without a
// position (n_r > l_kv) and page ids outside [0, num_pages) are skipped, so no
// write leaves the pool.
#include <hip/hip_runtime.h>

#include "kernels/common.hpp"

namespace bsr {

constexpr int kAppendWaves = 4;  // wavefronts per workgroup

__global__ __launch_bounds__(64 * kAppendWaves) void append_kv_kernel(
    const uint8_t* k_new, const uint8_t* v_new, const int32_t* append_indptr, const int32_t* kv_indptr,
    const int32_t* kv_indices, const int32_t* last_page_len, int32_t batch, int64_t total_new, int32_t h_kv,
    int32_t row_bytes, int32_t page_size, int64_t num_pages, int64_t tokens_per_wave, uint8_t* k_pool,
    uint8_t* v_pool) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * kAppendWaves +
                       __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int64_t t0 = wave * tokens_per_wave;
  const int64_t t1 = t0 + tokens_per_wave < total_new ? t0 + tokens_per_wave : total_new;
  if (t0 >= t1) return;
  // request of the first token: the last r with append_indptr[r] <= t0
  int32_t lo = 0, hi = batch;  // append_indptr[lo] <= t0 < append_indptr[hi] (if t0 is in range)
  while (hi - lo > 1) {
    const int32_t mid = (lo + hi) >> 1;
    if (load_invariant(append_indptr + mid) <= t0)
      lo = mid;
    else
      hi = mid;
  }
  int32_t r = lo;
  const int32_t pieces = row_bytes / 16;    // 16-byte pieces of one head's row
  const int32_t per_token = h_kv * pieces;  // pieces of one token (all heads)
  const int64_t end_all = load_invariant(append_indptr + batch);
  for (int64_t i = t0; i < t1 && i < end_all; ++i) {
    while (r + 1 < batch && load_invariant(append_indptr + r + 1) <= i) ++r;
    const int64_t a0 = load_invariant(append_indptr + r);
    const int64_t n_r = load_invariant(append_indptr + r + 1) - a0;
    const int32_t p0 = load_invariant(kv_indptr + r);
    const int32_t n_pages = load_invariant(kv_indptr + r + 1) - p0;
    if (n_pages <= 0) continue;
    const int64_t l_kv = static_cast<int64_t>(n_pages - 1) * page_size + load_invariant(last_page_len + r);
    const int64_t tau = l_kv - n_r + (i - a0);
    if (tau < 0 || tau / page_size >= n_pages) continue;  // no position, or a last page past P
    const int64_t page = load_invariant(kv_indices + p0 + tau / page_size);
    if (page < 0 || page >= num_pages) continue;
    const int64_t slot = tau % page_size;
    for (int32_t c = lane; c < per_token; c += 64) {
      const int32_t h = c / pieces;
      const int32_t piece = c - h * pieces;
      const int64_t src = (i * h_kv + h) * row_bytes + 16 * piece;
      const int64_t dst = ((page * h_kv + h) * page_size + slot) * row_bytes + 16 * piece;
      const uint4 kv_k = *reinterpret_cast<const uint4*>(k_new + src);
      const uint4 kv_v = *reinterpret_cast<const uint4*>(v_new + src);
      *reinterpret_cast<uint4*>(k_pool + dst) = kv_k;
      *reinterpret_cast<uint4*>(v_pool + dst) = kv_v;
    }
  }
}

}  // namespace bsr

// Grid: up to 16384 workgroups of 4 wavefronts (one token per wavefront up to
// 64k new tokens: the more rows in flight the better), each a contiguous range
// of new tokens.
extern "C" int bsr_launch_append_kv(const void* k_new, const void* v_new, const int32_t* append_indptr,
                                     const int32_t* kv_indptr, const int32_t* kv_indices,
                                     const int32_t* last_page_len, int32_t batch, int64_t total_new,
                                     int32_t h_kv, int32_t row_bytes, int32_t page_size, int64_t num_pages,
                                     void* k_pool, void* v_pool, hipStream_t s) {
  if (total_new == 0 || batch == 0) return 0;
  const int64_t max_waves = 16384LL * bsr::kAppendWaves;
  const int64_t per_wave = (total_new + max_waves - 1) / max_waves;
  const int64_t waves = (total_new + per_wave - 1) / per_wave;
  const int64_t blocks = (waves + bsr::kAppendWaves - 1) / bsr::kAppendWaves;
  hipLaunchKernelGGL(bsr::append_kv_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(64 * bsr::kAppendWaves), 0, s,
                     static_cast<const uint8_t*>(k_new), static_cast<const uint8_t*>(v_new), append_indptr,
                     kv_indptr, kv_indices, last_page_len, batch, total_new, h_kv, row_bytes, page_size, num_pages,
                     per_wave, static_cast<uint8_t*>(k_pool), static_cast<uint8_t*>(v_pool));
  return hipGetLastError() == hipSuccess ? 0 : 1;
}
