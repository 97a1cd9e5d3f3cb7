// persistent.hpp -- the run() kernel: a fixed grid of workgroups that executes
// the plan's work queues, then the merge map, in one launch.
//
// Core mechanism 6 and 7 of the FlashInfer explainer page (paper Algorithm 1,
// section 3.3.1, Appendix D): the grid is fixed; every workgroup walks its own
// queue of work items; split items write partial states into the workspace and
// unsplit ones write O/LSE directly; the contraction of partial states runs in
// the same kernel, in the order the plan fixed, without atomic accumulation.
//
// Ordering between a partial's writer and its merger uses release/acquire ready
// stamps, not read-modify-write: the writer stores the run's epoch into the
// partial's flag after its stores; the merger waits until the flag equals the
// epoch.  Each workgroup keeps its own run counter in the plan blob; the plan
// upload zeroes all counters and every run advances each by one, so all
// workgroups of a run agree on its epoch and stamps of older runs never match.
// Every workgroup finishes its attention items before it merges, and the grid
// never exceeds what the device keeps resident, so every awaited stamp is
// eventually written; the wait is bounded anyway and reports expiry through a
// status word instead of hanging.
#pragma once

#include "common.hpp"
#include "decode.hpp"
#include "merge.hpp"

namespace bsr {

template <int D, bool BF16, int ROWS, int TB, bool CAP, int KIND>
struct PersistentKernel {
  using Decode = DecodeBody<D, BF16, ROWS, TB, CAP>;
  using Merge = MergeBody<D, BF16>;
  static constexpr int LDS_FLOATS = Decode::LDS_FLOATS;
};

template <int D, bool BF16, int ROWS, int TB, bool CAP, int KIND>
__global__ __launch_bounds__(kWgThreads) void bsr_persistent_kernel(RunParams p) {
  using K = PersistentKernel<D, BF16, ROWS, TB, CAP, KIND>;
  __shared__ float lds[K::LDS_FLOATS];
  __shared__ int32_t s_epoch;
  uint8_t* ws = p.ws;
  const PlanHeader* hdr = plan_header(ws);
  const int wg = blockIdx.x;
  if (wg >= hdr->num_wg) return;  // grid larger than this plan's (never by construction)

  int32_t* epochs = plan_i32(ws, hdr->off_epochs);
  int32_t* flags = plan_i32(ws, hdr->off_flags);
  int32_t* status = plan_i32(ws, hdr->off_status);
  if (threadIdx.x == 0) s_epoch = epochs[wg] + 1;
  __syncthreads();
  const int32_t epoch = s_epoch;
  const int g = p.group;

  // ---- attention items -------------------------------------------------------
  const int32_t* item_ptr = plan_i32(ws, hdr->off_item_ptr);
  const WorkItem* items = reinterpret_cast<const WorkItem*>(ws + hdr->off_items);
  const int32_t ib = item_ptr[wg], ie = item_ptr[wg + 1];
  for (int32_t i = ib; i < ie; ++i) {
    const WorkItem it = items[i];
    if (it.flags & kItemPartial) {
      float* po = reinterpret_cast<float*>(ws + p.partial_o_off);
      float* pl = reinterpret_cast<float*>(ws + p.partial_lse_off);
      auto emit = [&](int r, int d, float o0, float o1, float lse2) {
        const int64_t row = static_cast<int64_t>(it.partial_row) + r;
        *reinterpret_cast<float2*>(po + row * D + d) = make_float2(o0, o1);
        if (d == 0) pl[row] = lse2;
      };
      K::Decode::run(p, it, lds, emit);
      publish_flag(flags + it.flag_id, epoch);
    } else {
      auto emit = [&](int r, int d, float o0, float o1, float lse2) {
        const int64_t orow =
            static_cast<int64_t>(it.qo_begin + r / g) * p.h_qo + it.kv_head * g + r % g;
        if constexpr (BF16) {
          *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(p.o) + orow * D + d) = pack_bf16x2(o0, o1);
        } else {
          *reinterpret_cast<float2*>(static_cast<float*>(p.o) + orow * D + d) = make_float2(o0, o1);
        }
        if (d == 0 && p.lse != nullptr) p.lse[orow] = lse2 == kNegInf ? kNegInf : lse2 * kLn2;
      };
      K::Decode::run(p, it, lds, emit);
    }
  }

  // ---- contraction of partial states -----------------------------------------
  const int32_t* merge_ptr = plan_i32(ws, hdr->off_merge_ptr);
  const MergeTask* tasks = reinterpret_cast<const MergeTask*>(ws + hdr->off_merge);
  const MergeSrc* srcs = reinterpret_cast<const MergeSrc*>(ws + hdr->off_srcs);
  const int32_t mb = merge_ptr[wg], me = merge_ptr[wg + 1];
  const int wave = threadIdx.x >> 6;
  bool ok = true;
  for (int32_t t = mb + wave; t < me; t += kWaves) ok = K::Merge::run(p, tasks[t], srcs, flags, epoch) && ok;
  if (!ok && (threadIdx.x & 63) == 0) status[kStatusWaitTimeout] = 1;

  __syncthreads();
  if (threadIdx.x == 0) epochs[wg] = epoch;
}

}  // namespace bsr
