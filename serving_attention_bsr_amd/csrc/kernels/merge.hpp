// merge.hpp -- the ⊕ contraction of partial attention states.
//
// Terms "Attention State and ⊕" of the FlashInfer explainer page (paper section
// 2.2): a state is (O, LSE); combining states of disjoint key sets weights each O
// by exp(LSE) of its set.  Core mechanism 6 (paper Algorithm 1, section 3.3.1):
// the contraction follows the merge map the planner wrote, in a fixed order, with
// no atomic accumulation, inside the same persistent kernel as the attention.
//
// Partial states are stored in base 2 (LSE2 = log2 of the key set's weight);
// results leave in natural log.
//
// A whole workgroup merges one task (g folded rows of one query token) at a time.
// The contraction sits at the tail of the kernel, so it is organised for latency:
// each source's ready stamp is polled by its own thread; the sources' LSEs are
// read in parallel into LDS (max pass, then weight pass); the partial outputs are
// read as 16-byte loads, four sources per step, by threads split into source
// groups.  A task thus costs a few memory round trips however many sources it
// has.  Within a source group the sum runs in map order and the groups are added
// in a fixed order, so the result is deterministic.
#pragma once

#include "common.hpp"

namespace bsr {

constexpr int kMergeMaxGroup = 16;   // query heads per KV head the merge supports
constexpr int kMergeSrcPass = 256;   // sources staged in LDS per pass

template <int D, bool BF16>
struct MergeBody {
  // LDS floats: staged LSE/weights, group partial sums, row max and row sums.
  static constexpr int LDS_FLOATS = kMergeSrcPass * kMergeMaxGroup + kWgThreads * 4 + 2 * kMergeMaxGroup;

  // Wait (bounded) for the ready stamps of a task's sources, one thread per
  // source; false if one never came.  All threads of the workgroup take part.
  static __device__ bool wait(const MergeTask& t, const MergeSrc* srcs, const int32_t* flags,
                              int32_t epoch) {
    bool ok = true;
    for (int s = threadIdx.x; s < t.src_count; s += kWgThreads)
      if (ok) ok = wait_flag(flags + srcs[t.src_begin + s].flag_id, epoch);
    return ok;
  }

  // Merge one task (all threads).  The caller has waited and acquired.
  static __device__ void run(const RunParams& p, const MergeTask& t, const MergeSrc* srcs,
                             float* lds) {
    const int g = p.group;
    const int n = t.src_count;
    const MergeSrc* src = srcs + t.src_begin;
    const float* po = reinterpret_cast<const float*>(p.ws + p.partial_o_off);
    const float* pl = reinterpret_cast<const float*>(p.ws + p.partial_lse_off);
    float* stage = lds;                                      // [kMergeSrcPass][g]
    float* part = lds + kMergeSrcPass * kMergeMaxGroup;      // [kWgThreads] float4
    float* rmax = part + kWgThreads * 4;                     // [g]
    float* rsum = rmax + kMergeMaxGroup;                     // [g]
    const int tid = threadIdx.x;
    // float4 slots of the g rows of one token; threads split into source groups
    const int slots = g * D / 4;
    const int groups = slots >= kWgThreads ? 1 : kWgThreads / slots;
    const int slot0 = tid % slots;
    const int grp = tid / slots;

    // pass 1: row maxima of LSE2
    float my_max = kNegInf;
    for (int base = 0; base < n; base += kMergeSrcPass) {
      const int cnt = min(kMergeSrcPass, n - base);
      for (int i = tid; i < cnt * g; i += kWgThreads) stage[i] = pl[src[base + i / g].partial_row + i % g];
      __syncthreads();
      if (tid < g)
        for (int s = 0; s < cnt; ++s) my_max = __builtin_fmaxf(my_max, stage[s * g + tid]);
      __syncthreads();
    }
    if (tid < g) rmax[tid] = my_max;
    __syncthreads();

    // pass 2: weights 2^(lse - max), their row sums, and the weighted outputs
    float4 acc[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    float my_sum = 0.0f;
    for (int base = 0; base < n; base += kMergeSrcPass) {
      const int cnt = min(kMergeSrcPass, n - base);
      for (int i = tid; i < cnt * g; i += kWgThreads) {
        const float m = rmax[i % g];
        const float l = pl[src[base + i / g].partial_row + i % g];
        stage[i] = m == kNegInf ? 0.0f : fast_exp2(l - m);
      }
      __syncthreads();
      if (tid < g)
        for (int s = 0; s < cnt; ++s) my_sum += stage[s * g + tid];
      if (grp < groups) {
        // four sources per step, loads issued together; past-the-end sources are
        // clamped to the last one with weight zero
        for (int s = grp; s < cnt; s += 4 * groups) {
          int sj[4];
          float wsel[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int sv = s + j * groups;
            sj[j] = min(sv, cnt - 1);
            wsel[j] = sv < cnt ? 1.0f : 0.0f;
          }
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int slot = slot0 + k * kWgThreads;
            if (k * kWgThreads < slots && slot < slots) {
              const int r = (slot * 4) / D;
              const int d = (slot * 4) % D;
              float4 v[4];
#pragma unroll
              for (int j = 0; j < 4; ++j)
                v[j] = *reinterpret_cast<const float4*>(
                    po + static_cast<int64_t>(src[base + sj[j]].partial_row + r) * D + d);
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const float w = wsel[j] * stage[sj[j] * g + r];
                acc[k].x = __builtin_fmaf(w, v[j].x, acc[k].x);
                acc[k].y = __builtin_fmaf(w, v[j].y, acc[k].y);
                acc[k].z = __builtin_fmaf(w, v[j].z, acc[k].z);
                acc[k].w = __builtin_fmaf(w, v[j].w, acc[k].w);
              }
            }
          }
        }
      }
      __syncthreads();
    }
    if (tid < g) rsum[tid] = my_sum;
    // source groups are added in a fixed order (groups > 1 only when one slot
    // per thread covers the rows)
    if (groups > 1) {
      reinterpret_cast<float4*>(part)[tid] = acc[0];
      __syncthreads();
      if (grp == 0) {
        for (int q = 1; q < groups; ++q) {
          const float4 v = reinterpret_cast<const float4*>(part)[q * slots + slot0];
          acc[0].x += v.x;
          acc[0].y += v.y;
          acc[0].z += v.z;
          acc[0].w += v.w;
        }
      }
    }
    __syncthreads();
    if (grp == 0) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int slot = slot0 + k * kWgThreads;
        if (k * kWgThreads < slots && slot < slots) {
          const int r = (slot * 4) / D;
          const int d = (slot * 4) % D;
          const float z = rsum[r];
          const float inv = z > 0.0f ? 1.0f / z : 0.0f;
          const int64_t orow = static_cast<int64_t>(t.qo_row) * p.h_qo + t.kv_head * g + r;
          const float o0 = acc[k].x * inv, o1 = acc[k].y * inv, o2 = acc[k].z * inv, o3 = acc[k].w * inv;
          if constexpr (BF16) {
            uint2 pk;
            pk.x = pack_bf16x2(o0, o1);
            pk.y = pack_bf16x2(o2, o3);
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.o) + orow * D + d) = pk;
          } else {
            *reinterpret_cast<float4*>(static_cast<float*>(p.o) + orow * D + d) = make_float4(o0, o1, o2, o3);
          }
          if (d == 0 && p.lse != nullptr) p.lse[orow] = z > 0.0f ? (rmax[r] + fast_log2(z)) * kLn2 : kNegInf;
        }
      }
    }
    __syncthreads();
  }
};

}  // namespace bsr
