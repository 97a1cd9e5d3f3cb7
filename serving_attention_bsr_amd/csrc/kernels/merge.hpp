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
// each source's ready stamp is polled by its own thread, then a single pass
// folds the sources in with a running maximum (online ⊕): each thread owns
// float4 slots of the g rows and loads the LSE and partial outputs of a batch of
// sources together, so a task costs about one memory round trip per batch.  When
// the rows have fewer slots than the workgroup has threads, the threads split
// into source groups (source s goes to group s mod groups) whose states are
// combined in group order through LDS.  Sources are folded in map order within a
// group, so the result is deterministic.
#pragma once

#include "common.hpp"

namespace bsr {

constexpr int kMergeMaxGroup = 16;   // query heads per KV head the merge supports

template <int D, bool BF16>
struct MergeBody {
  static constexpr int MAX_SLOTS = kMergeMaxGroup * D / 4;                       // float4 slots of a task
  static constexpr int KSLOTS = (MAX_SLOTS + kWgThreads - 1) / kWgThreads;       // slots per thread, at most
  static constexpr int SB = KSLOTS >= 4 ? 2 : (KSLOTS >= 2 ? 4 : 8);            // sources per batch
  // tasks whose rows need at most one float4 slot per thread (g * D <= 1024) load
  // this many sources per batch, so one round trip covers a task of up to
  // FAST_SB * (threads / slots) sources
  static constexpr int FAST_SB = 16;
  // LDS floats: per-thread group states (m, l, acc) for the cross-group combine
  static constexpr int LDS_FLOATS = kWgThreads * 6;

  // Wait (bounded) for the ready stamps of a task's sources, one thread per
  // source; false if one never came.  All threads of the workgroup take part.
  static __device__ bool wait(const MergeTask& t, const MergeSrc* srcs, const int32_t* flags,
                              int32_t epoch, int32_t spin_limit) {
    bool ok = true;
    for (int s = threadIdx.x; s < t.src_count; s += kWgThreads)
      if (ok) ok = wait_flag(flags + srcs[t.src_begin + s].flag_id, epoch, spin_limit);
    return ok;
  }

  // Merge one task (all threads).  The caller has waited for the sources' stamps;
  // states are read with device-scope loads.
  static __device__ void run(const RunParams& p, const MergeTask& t, const MergeSrc* srcs, float* lds) {
    if (p.group * D <= 4 * kWgThreads)
      run_slots<1, FAST_SB>(p, t, srcs, lds);
    else
      run_slots<KSLOTS, SB>(p, t, srcs, lds);
  }

  // KS float4 slots per thread, NB sources per batch.
  template <int KS, int NB>
  static __device__ __forceinline__ void run_slots(const RunParams& p, const MergeTask& t, const MergeSrc* srcs,
                                                   float* lds) {
    const int g = p.group;
    const int n = t.src_count;
    const MergeSrc* src = srcs + t.src_begin;
    const float* po = reinterpret_cast<const float*>(p.ws + p.partial_o_off);
    const float* pl = reinterpret_cast<const float*>(p.ws + p.partial_lse_off);
    const int tid = threadIdx.x;
    const int slots = g * D / 4;
    const int groups = slots >= kWgThreads ? 1 : kWgThreads / slots;
    const int slot0 = tid % slots;
    const int grp = tid / slots;
    const bool active = grp < groups;

    // per slot k: running max (base 2), sum of weights, weighted sum of outputs
    float m[KS], l[KS];
    float4 acc[KS];
    int row[KS], dcol[KS];
    bool has[KS];
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const int slot = slot0 + k * kWgThreads;
      has[k] = active && (k == 0 || slots > kWgThreads) && slot < slots;
      row[k] = has[k] ? (slot * 4) / D : 0;
      dcol[k] = has[k] ? (slot * 4) % D : 0;
      m[k] = kNegInf;
      l[k] = 0.0f;
      acc[k] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
    if (active) {
      // sources grp, grp + groups, ... in batches of NB loaded together; past the
      // end a batch repeats the group's last source with weight zero
      const int mine = n > grp ? (n - grp + groups - 1) / groups : 0;
      for (int b = 0; b < mine; b += NB) {
        // the batch's partial-state rows first, then all its loads: the load
        // counter completes in order, so reading a row index between the state
        // loads would wait for every load before it
        int prow[NB];
        bool live[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          live[j] = b + j < mine;
          prow[j] = load_invariant(&src[grp + groups * min(b + j, mine - 1)].partial_row);
        }
        float ls[NB][KS];
        float4 os[NB][KS];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
#pragma unroll
          for (int k = 0; k < KS; ++k) {
            if (!has[k]) continue;
            ls[j][k] = load_dev_f32(pl + prow[j] + row[k]);
            os[j][k] = load_dev_f32x4(po + static_cast<int64_t>(prow[j] + row[k]) * D + dcol[k]);
          }
        }
#pragma unroll
        for (int k = 0; k < KS; ++k) {
          if (!has[k]) continue;
          float mb = m[k];
#pragma unroll
          for (int j = 0; j < NB; ++j)
            if (live[j]) mb = __builtin_fmaxf(mb, ls[j][k]);
          const float m_use = mb == kNegInf ? 0.0f : mb;
          const float sc = fast_exp2(m[k] - m_use);
          l[k] *= sc;
          acc[k].x *= sc;
          acc[k].y *= sc;
          acc[k].z *= sc;
          acc[k].w *= sc;
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            const float w = live[j] ? fast_exp2(ls[j][k] - m_use) : 0.0f;
            l[k] += w;
            acc[k].x = __builtin_fmaf(w, os[j][k].x, acc[k].x);
            acc[k].y = __builtin_fmaf(w, os[j][k].y, acc[k].y);
            acc[k].z = __builtin_fmaf(w, os[j][k].z, acc[k].z);
            acc[k].w = __builtin_fmaf(w, os[j][k].w, acc[k].w);
          }
          m[k] = mb;
        }
      }
    }
    // source groups are combined in group order (groups > 1 only with one slot
    // per thread)
    if (groups > 1) {
      if (active) {
        float* st = lds + tid * 6;
        st[0] = m[0];
        st[1] = l[0];
        st[2] = acc[0].x;
        st[3] = acc[0].y;
        st[4] = acc[0].z;
        st[5] = acc[0].w;
      }
      __syncthreads();
      if (grp == 0) {
        for (int q = 1; q < groups; ++q) {
          const float* st = lds + (q * slots + slot0) * 6;
          const float mq = st[0];
          const float mn = __builtin_fmaxf(m[0], mq);
          const float m_use = mn == kNegInf ? 0.0f : mn;
          const float a = fast_exp2(m[0] - m_use), bq = fast_exp2(mq - m_use);
          l[0] = l[0] * a + st[1] * bq;
          acc[0].x = acc[0].x * a + st[2] * bq;
          acc[0].y = acc[0].y * a + st[3] * bq;
          acc[0].z = acc[0].z * a + st[4] * bq;
          acc[0].w = acc[0].w * a + st[5] * bq;
          m[0] = mn;
        }
      }
    }
    if (grp == 0) {
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        if (!has[k]) continue;
        const float z = l[k];
        const float inv = z > 0.0f ? 1.0f / z : 0.0f;
        const int64_t orow = static_cast<int64_t>(t.qo_row) * p.h_qo + t.kv_head * g + row[k];
        const float o0 = acc[k].x * inv, o1 = acc[k].y * inv, o2 = acc[k].z * inv, o3 = acc[k].w * inv;
        if constexpr (BF16) {
          uint2 pk;
          pk.x = pack_bf16x2(o0, o1);
          pk.y = pack_bf16x2(o2, o3);
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.o) + orow * D + dcol[k]) = pk;
        } else {
          *reinterpret_cast<float4*>(static_cast<float*>(p.o) + orow * D + dcol[k]) = make_float4(o0, o1, o2, o3);
        }
        if (dcol[k] == 0 && p.lse != nullptr) p.lse[orow] = z > 0.0f ? (m[k] + fast_log2(z)) * kLn2 : kNegInf;
      }
    }
    __syncthreads();  // LDS and the next task
  }
};

}  // namespace bsr
