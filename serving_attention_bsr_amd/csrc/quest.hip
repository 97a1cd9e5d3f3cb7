// quest.hip -- Quest-style page-budget sparse decode over the BSR cache: page
// summaries and the per-step page choice.
//
// Applicable scenarios item 5 of the FlashInfer explainer page (paper Appendix
// G.5, Tables 9-11): KV-pruning algorithms of the Quest kind keep a budget of KV
// pages per step and run the block-sparse attention (pages of 16 keys) over the
// kept pages only; the kept pages are a BSR matrix like any other, so the
// attention itself is the library's run() over per-KV-head page lists
// (bsr_attn_plan_head_pages).  The choice follows Quest's published criterion:
//   * summary: per page and KV head, the elementwise min and max of its valid
//     keys (the last page of a request holds last_page_len of them);
//   * score: per query head, sum_d max(q_d min_d, q_d max_d), an upper bound of
//     q.k over the page's keys; a KV head takes its query heads' maximum;
//   * per request and KV head, the last page is always kept and the budget - 1
//     best other pages join it, ties to the earlier page; the kept pages are
//     written in logical order, the last page last.
//
// Kernels:
//   page_summary_kernel  one wavefront per (page-table entry, KV head); the head's
//                        [P, D] block of a page is contiguous.  Runs when pages
//                        fill (off the per-step path).
//   quest_score_kernel   D / E lanes per (entry, KV head), E elements (16 bytes)
//                        per lane; HBM-bound: 2 D elements of summaries per pair.
//   quest_select_kernel  one workgroup per (request, KV head): the candidate
//                        scores as order-preserving 32-bit keys in LDS, a 4-pass
//                        8-bit radix select of the (budget - 1)-th largest key
//                        (histogram in LDS, bin search by a workgroup scan), then
//                        ordered scans that keep every larger key and the
//                        earliest equal ones.  Deterministic (LDS histogram counts
//                        are exact integers; the output order is the index order).
#include <hip/hip_runtime.h>

#include "kernels/common.hpp"

namespace bsr {

constexpr int kQuestThreads = 256;
constexpr int kQuestMaxCandidates = 16384;  // pages of one request, the last one excluded

// Request r of page-table entry e: the last r with kv_indptr[r] <= e.
__device__ __forceinline__ int32_t request_of(const int32_t* kv_indptr, int32_t batch, int64_t e) {
  int32_t lo = 0, hi = batch;
  while (hi - lo > 1) {
    const int32_t mid = (lo + hi) >> 1;
    if (kv_indptr[mid] <= e)
      lo = mid;
    else
      hi = mid;
  }
  return lo;
}

template <typename T>
__device__ __forceinline__ float elem_f32(T x);
template <>
__device__ __forceinline__ float elem_f32<uint16_t>(uint16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}
template <>
__device__ __forceinline__ float elem_f32<float>(float x) {
  return x;
}
template <typename T>
__device__ __forceinline__ T f32_elem(float x);
template <>
__device__ __forceinline__ uint16_t f32_elem<uint16_t>(float x) {
  return static_cast<uint16_t>(__float_as_uint(x) >> 16);  // exact: x is a bf16 value
}
template <>
__device__ __forceinline__ float f32_elem<float>(float x) {
  return x;
}

template <typename T>
__global__ __launch_bounds__(kQuestThreads) void page_summary_kernel(const T* k_pool, const int32_t* kv_indptr,
                                                                    const int32_t* kv_indices,
                                                                    const int32_t* last_page_len, int32_t batch,
                                                                    int64_t entries, int32_t h_kv, int32_t d,
                                                                    int32_t page_size, int64_t num_pages, T* kmin,
                                                                    T* kmax) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * (kQuestThreads / 64) + (threadIdx.x >> 6);
  if (wave >= entries * h_kv) return;
  const int64_t e = wave / h_kv;
  const int32_t head = static_cast<int32_t>(wave % h_kv);
  const int32_t r = request_of(kv_indptr, batch, e);
  const int32_t valid = e == kv_indptr[r + 1] - 1 ? last_page_len[r] : page_size;
  const int64_t page = kv_indices[e];
  if (page < 0 || page >= num_pages || valid < 1 || valid > page_size) return;
  const T* blk = k_pool + (page * h_kv + head) * static_cast<int64_t>(page_size) * d;
  T* omin = kmin + (page * h_kv + head) * static_cast<int64_t>(d);
  T* omax = kmax + (page * h_kv + head) * static_cast<int64_t>(d);
  for (int c = lane; c < d; c += 64) {
    float mn = __builtin_inff(), mx = -__builtin_inff();
    for (int s = 0; s < valid; ++s) {
      const float x = elem_f32<T>(blk[static_cast<int64_t>(s) * d + c]);
      mn = __builtin_fminf(mn, x);
      mx = __builtin_fmaxf(mx, x);
    }
    omin[c] = f32_elem<T>(mn);
    omax[c] = f32_elem<T>(mx);
  }
}

// Sum over aligned groups of N lanes (N = 8 .. 64).
template <int N>
__device__ __forceinline__ float lanes_sum(float x) {
  x = group_sum<(N < 16 ? N : 16)>(x);
  if constexpr (N >= 32) x = pair_sum<16>(x);
  if constexpr (N >= 64) x = pair_sum<32>(x);
  return x;
}

template <typename T, int D>
__global__ __launch_bounds__(kQuestThreads) void quest_score_kernel(const T* q, const T* kmin, const T* kmax,
                                                                   const int32_t* kv_indptr,
                                                                   const int32_t* kv_indices, int32_t batch,
                                                                   int64_t entries, int32_t h_qo, int32_t h_kv,
                                                                   int64_t num_pages, float* scores) {
  constexpr int E = 16 / sizeof(T);  // elements per lane (one 16-byte load)
  constexpr int LPP = D / E;         // lanes per (entry, KV head)
  constexpr int PPW = 64 / LPP;      // pairs per wavefront
  static_assert(LPP >= 8 && LPP <= 64 && 64 % LPP == 0, "lanes per pair");
  const int lane = threadIdx.x & 63;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * (kQuestThreads / 64) + (threadIdx.x >> 6);
  const int64_t pair = wave * PPW + lane / LPP;
  const int sub = lane % LPP;
  // every lane takes part in the group sums below; lanes past the end compute on
  // the first pair and do not store
  const bool live = pair < entries * h_kv;
  const int64_t pr = live ? pair : 0;
  const int64_t e = pr / h_kv;
  const int32_t hk = static_cast<int32_t>(pr % h_kv);
  const int32_t r = request_of(kv_indptr, batch, e);
  const int64_t page = kv_indices[e];
  const bool in_pool = page >= 0 && page < num_pages;
  const int64_t pg = in_pool ? page : 0;
  const int g = h_qo / h_kv;
  const uint4 mn_raw = *reinterpret_cast<const uint4*>(kmin + (pg * h_kv + hk) * D + sub * E);
  const uint4 mx_raw = *reinterpret_cast<const uint4*>(kmax + (pg * h_kv + hk) * D + sub * E);
  const T* mn = reinterpret_cast<const T*>(&mn_raw);
  const T* mx = reinterpret_cast<const T*>(&mx_raw);
  float best = -__builtin_inff();
  for (int j = 0; j < g; ++j) {
    const uint4 q_raw = *reinterpret_cast<const uint4*>(q + (static_cast<int64_t>(r) * h_qo + hk * g + j) * D + sub * E);
    const T* qv = reinterpret_cast<const T*>(&q_raw);
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const float qi = elem_f32<T>(qv[i]);
      part += __builtin_fmaxf(qi * elem_f32<T>(mn[i]), qi * elem_f32<T>(mx[i]));
    }
    best = __builtin_fmaxf(best, lanes_sum<LPP>(part));
  }
  if (live && sub == 0) scores[static_cast<int64_t>(hk) * entries + e] = in_pool ? best : -__builtin_inff();
}

// Exclusive prefix sum over the 256 threads of the workgroup, in thread order
// (lane prefix by shuffles, then the wavefront totals through LDS); every thread
// of the workgroup must call it.  tmp: 4 ints of LDS.
__device__ __forceinline__ int32_t block_exclusive_scan(int32_t x, int32_t* tmp) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int32_t inc = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t y = __shfl_up(inc, o, 64);
    if (lane >= o) inc += y;
  }
  if (lane == 63) tmp[wave] = inc;
  __syncthreads();
  int32_t before = 0;
  for (int w = 0; w < wave; ++w) before += tmp[w];
  __syncthreads();  // tmp is free for the next call
  return before + inc - x;
}

// Order-preserving 32-bit key of a float (larger float, larger key).
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ __launch_bounds__(kQuestThreads) void quest_select_kernel(const float* scores, const int32_t* kv_indptr,
                                                                    const int32_t* kv_indices, int32_t h_kv,
                                                                    int64_t entries, int32_t budget,
                                                                    const int32_t* out_indptr,
                                                                    int32_t* out_indices) {
  static_assert(kQuestThreads == 256, "one histogram bin per thread");
  __shared__ uint32_t keys[kQuestMaxCandidates];
  __shared__ uint32_t hist[256];
  __shared__ int32_t scan_tmp[4];
  __shared__ uint32_t shared_digit;
  __shared__ int32_t shared_krem;
  const int tid = threadIdx.x;
  const int32_t r = blockIdx.x / h_kv;
  const int32_t hk = blockIdx.x % h_kv;
  const int32_t base = kv_indptr[r];
  const int32_t n = kv_indptr[r + 1] - base;
  const int32_t out0 = out_indptr[blockIdx.x];
  const int32_t room = out_indptr[blockIdx.x + 1] - out0;  // the caller sized it min(n, budget)
  if (n <= budget) {
    for (int32_t i = tid; i < n && i < room; i += kQuestThreads) out_indices[out0 + i] = kv_indices[base + i];
    return;
  }
  const int32_t m = n - 1;  // candidates: every page but the last
  if (m > kQuestMaxCandidates) return;  // rejected on the host
  const int32_t k = budget - 1;
  const float* sc = scores + static_cast<int64_t>(hk) * entries + base;
  for (int32_t i = tid; i < m; i += kQuestThreads) keys[i] = order_key(sc[i]);
  // radix select, most significant digit first: the k-th largest key T
  uint32_t prefix = 0, mask = 0;
  int32_t krem = k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    hist[tid] = 0;
    __syncthreads();
    if (pass == 0) {
      // Scores of similar size share their top key byte, so on the first digit
      // most candidates fall into one or two bins and one LDS atomic per key would
      // serialize on a single address.  Each wavefront instead adds each distinct
      // bin of its 64 keys once (lanes with the leader's bin found by a ballot).
      const int lane = tid & 63;
      for (int32_t i0 = tid - lane; i0 < m; i0 += kQuestThreads) {  // the same for the whole wavefront
        const int32_t i = i0 + lane;
        const bool valid = i < m;
        const uint32_t bin = valid ? keys[i] >> 24 : 0u;
        uint64_t pending = __ballot(valid);
        while (pending != 0) {
          const int leader = __builtin_ctzll(pending);
          const uint32_t lb = __shfl(bin, leader, 64);
          const uint64_t same = __ballot(valid && bin == lb);
          if (lane == leader) atomicAdd(&hist[lb], static_cast<uint32_t>(__builtin_popcountll(same)));
          pending &= ~same;
        }
      }
    } else {
      for (int32_t i = tid; i < m; i += kQuestThreads) {
        const uint32_t key = keys[i];
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
    }
    __syncthreads();
    // thread t holds bin 255 - t: its exclusive prefix counts the keys in higher
    // bins; exactly one bin holds the k-th largest key
    const int32_t c = static_cast<int32_t>(hist[255 - tid]);
    const int32_t above = block_exclusive_scan(c, scan_tmp);
    if (above < krem && krem <= above + c) {
      shared_digit = static_cast<uint32_t>(255 - tid);
      shared_krem = krem - above;
    }
    __syncthreads();
    prefix |= shared_digit << shift;
    mask |= 0xffu << shift;
    krem = shared_krem;
    __syncthreads();
  }
  const uint32_t thr = prefix;  // keys > thr are kept; krem of the keys == thr, earliest first
  // each thread owns a contiguous run of candidates, so that scans keep index order
  const int32_t per = (m + kQuestThreads - 1) / kQuestThreads;
  const int32_t i0 = min(tid * per, m), i1 = min(i0 + per, m);
  int32_t gt = 0, eq = 0;
  for (int32_t i = i0; i < i1; ++i) {
    gt += keys[i] > thr;
    eq += keys[i] == thr;
  }
  // equal keys before this thread's run, then this thread's kept count and its
  // first output position
  const int32_t eq_before = block_exclusive_scan(eq, scan_tmp);
  const int32_t take = max(0, min(eq, krem - eq_before));  // equal keys this thread keeps
  int32_t pos = block_exclusive_scan(gt + take, scan_tmp);
  int32_t eq_left = take;
  for (int32_t i = i0; i < i1; ++i) {
    const uint32_t key = keys[i];
    bool keep = key > thr;
    if (key == thr && eq_left > 0) {
      keep = true;
      --eq_left;
    }
    if (keep) {
      if (pos < room) out_indices[out0 + pos] = kv_indices[base + i];
      ++pos;
    }
  }
  if (tid == 0 && k < room) out_indices[out0 + k] = kv_indices[base + m];  // the last page, last
}

}  // namespace bsr

extern "C" int bsr_launch_page_summary(const void* k_pool, const int32_t* kv_indptr, const int32_t* kv_indices,
                                        const int32_t* last_page_len, int32_t batch, int64_t entries, int32_t h_kv,
                                        int32_t d, int32_t page_size, int32_t elt_bytes, int64_t num_pages,
                                        void* kmin, void* kmax, hipStream_t s) {
  const int64_t waves = entries * h_kv;
  if (waves == 0) return 0;
  const int64_t blocks = (waves + 3) / 4;
  if (elt_bytes == 2)
    hipLaunchKernelGGL(bsr::page_summary_kernel<uint16_t>, dim3(static_cast<uint32_t>(blocks)),
                       dim3(bsr::kQuestThreads), 0, s, static_cast<const uint16_t*>(k_pool), kv_indptr, kv_indices,
                       last_page_len, batch, entries, h_kv, d, page_size, num_pages, static_cast<uint16_t*>(kmin),
                       static_cast<uint16_t*>(kmax));
  else
    hipLaunchKernelGGL(bsr::page_summary_kernel<float>, dim3(static_cast<uint32_t>(blocks)),
                       dim3(bsr::kQuestThreads), 0, s, static_cast<const float*>(k_pool), kv_indptr, kv_indices,
                       last_page_len, batch, entries, h_kv, d, page_size, num_pages, static_cast<float*>(kmin),
                       static_cast<float*>(kmax));
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

template <typename T, int D>
static void launch_score(const void* q, const void* kmin, const void* kmax, const int32_t* kv_indptr,
                         const int32_t* kv_indices, int32_t batch, int64_t entries, int32_t h_qo, int32_t h_kv,
                         int64_t num_pages, float* scores, hipStream_t s) {
  constexpr int PPW = 64 / (D / (16 / sizeof(T)));
  const int64_t waves = (entries * h_kv + PPW - 1) / PPW;
  const int64_t blocks = (waves + 3) / 4;
  hipLaunchKernelGGL((bsr::quest_score_kernel<T, D>), dim3(static_cast<uint32_t>(blocks)), dim3(bsr::kQuestThreads),
                     0, s, static_cast<const T*>(q), static_cast<const T*>(kmin), static_cast<const T*>(kmax),
                     kv_indptr, kv_indices, batch, entries, h_qo, h_kv, num_pages, scores);
}

extern "C" int bsr_launch_quest_select(const void* q, const void* kmin, const void* kmax, const int32_t* kv_indptr,
                                        const int32_t* kv_indices, int32_t batch, int64_t entries, int32_t h_qo,
                                        int32_t h_kv, int32_t d, int32_t elt_bytes, int64_t num_pages, int32_t budget,
                                        const int32_t* out_indptr, int32_t* out_indices, float* scores,
                                        hipStream_t s) {
  if (batch == 0) return 0;
  if (entries > 0) {
    if (elt_bytes == 2) {
      if (d == 64) launch_score<uint16_t, 64>(q, kmin, kmax, kv_indptr, kv_indices, batch, entries, h_qo, h_kv,
                                              num_pages, scores, s);
      else if (d == 128) launch_score<uint16_t, 128>(q, kmin, kmax, kv_indptr, kv_indices, batch, entries, h_qo,
                                                     h_kv, num_pages, scores, s);
      else launch_score<uint16_t, 256>(q, kmin, kmax, kv_indptr, kv_indices, batch, entries, h_qo, h_kv, num_pages,
                                       scores, s);
    } else {
      if (d == 64) launch_score<float, 64>(q, kmin, kmax, kv_indptr, kv_indices, batch, entries, h_qo, h_kv,
                                           num_pages, scores, s);
      else if (d == 128) launch_score<float, 128>(q, kmin, kmax, kv_indptr, kv_indices, batch, entries, h_qo, h_kv,
                                                  num_pages, scores, s);
      else launch_score<float, 256>(q, kmin, kmax, kv_indptr, kv_indices, batch, entries, h_qo, h_kv, num_pages,
                                    scores, s);
    }
  }
  hipLaunchKernelGGL(bsr::quest_select_kernel, dim3(static_cast<uint32_t>(batch) * h_kv), dim3(bsr::kQuestThreads), 0,
                     s, scores, kv_indptr, kv_indices, h_kv, entries, budget, out_indptr, out_indices);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}
