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
#pragma once

#include "common.hpp"

namespace bsr {

template <int D, bool BF16>
struct MergeBody {
  static constexpr int EPL = D / 64;  // elements per lane per row

  // One wavefront merges one task: g folded rows x D, sources in map order.
  // Returns false if a source's ready flag never arrived (bounded wait).
  static __device__ bool run(const RunParams& p, const MergeTask& t, const MergeSrc* srcs,
                             const int32_t* flags, int32_t epoch) {
    const int lane = threadIdx.x & 63;
    bool ok = true;
    for (int s = 0; s < t.src_count; ++s) ok = wait_flag(flags + srcs[t.src_begin + s].flag_id, epoch) && ok;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    const float* po = reinterpret_cast<const float*>(p.ws + p.partial_o_off);
    const float* pl = reinterpret_cast<const float*>(p.ws + p.partial_lse_off);
    const int g = p.group;
    for (int r = 0; r < g; ++r) {
      float big = kNegInf;
      for (int s = 0; s < t.src_count; ++s) big = __builtin_fmaxf(big, pl[srcs[t.src_begin + s].partial_row + r]);
      const float m_use = big == kNegInf ? 0.0f : big;
      float acc[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
      float wsum = 0.0f;
      for (int s = 0; s < t.src_count; ++s) {
        const int32_t row = srcs[t.src_begin + s].partial_row + r;
        const float w = fast_exp2(pl[row] - m_use);
        wsum += w;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = __builtin_fmaf(w, po[static_cast<int64_t>(row) * D + e * 64 + lane], acc[e]);
      }
      const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
      const int64_t orow = static_cast<int64_t>(t.qo_row) * p.h_qo + t.kv_head * g + r;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float val = acc[e] * inv;
        if constexpr (BF16) {
          static_cast<uint16_t*>(p.o)[orow * D + e * 64 + lane] = f32_to_bf16(val);
        } else {
          static_cast<float*>(p.o)[orow * D + e * 64 + lane] = val;
        }
      }
      if (p.lse != nullptr && lane == 0) p.lse[orow] = wsum > 0.0f ? (big + fast_log2(wsum)) * kLn2 : kNegInf;
    }
    return ok;
  }
};

}  // namespace bsr
