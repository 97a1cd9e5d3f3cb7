// persistent.hpp -- the run() kernel: a fixed grid of workgroups that executes
// the plan's work queues, then the merge map, in one launch.
//
// Core mechanism 6 and 7 of the FlashInfer explainer page (paper Algorithm 1,
// section 3.3.1, Appendix D): the grid is fixed; every workgroup walks its own
// queue of work items; split items write partial states into the workspace and
// unsplit ones write O/LSE directly; the contraction of partial states runs in
// the same kernel, in the order the plan fixed, without atomic accumulation.
//
// Ordering between a partial's writer and its merger uses ready stamps, not
// read-modify-write.  Partial states, stamps and the merger's reads of both are
// device-scope accesses (written through to, and read from, the device's
// coherence point, past the per-XCD L2 caches): after its attention items a
// workgroup waits until its partial-state stores have completed, meets, and
// stores the run's epoch into the flag of each partial state it wrote; a merging
// workgroup waits until the flags of its sources equal the epoch, then reads the
// states.  A device-scope release/acquire fence would instead write back and
// invalidate whole L2 caches, which costs about 10 us per workgroup at the end of
// a busy kernel.  Each workgroup keeps its own run counter in the plan blob; the plan
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
#include "prefill.hpp"
#include "prefill16.hpp"

namespace bsr {

constexpr int cmax(int a, int b) { return a > b ? a : b; }

// KIND selects the attention bodies: decode only, MFMA only (bf16), or both
// (chosen per work item).
template <int D, bool BF16, int ROWS, int TB, bool CAP, int KIND, bool PAGE1, bool KV8, bool VAR>
struct PersistentKernel {
  static_assert(KIND == kKindDecode || BF16, "the MFMA body is bf16 only");
  static_assert(KIND == kKindDecode || !KV8 || D <= 128, "an FP8 K/V cache runs on the 32-row MFMA body only");
  using Decode = DecodeBody<D, BF16, ROWS, TB, CAP, KV8, VAR>;
  // 32 rows per wavefront up to D = 128; 16 rows (two workgroups per CU) at D = 256
  // (the tile kernel's ROWS = 1 selects the 64-row tile: the 16-row body at D = 128)
  static constexpr bool kShortTile = KIND == kKindMfma && ROWS == 1;
  using Mfma = typename std::conditional<D == 256 || kShortTile, MfmaBody16<D, CAP, PAGE1, VAR>,
                                         MfmaBody<D, CAP, PAGE1, VAR, KV8>>::type;
  using Merge = MergeBody<D, BF16>;
  static constexpr int LDS_FLOATS =
      cmax(Merge::LDS_FLOATS, cmax(KIND == kKindMfma ? 0 : Decode::LDS_FLOATS,
                                   KIND == kKindDecode ? 0 : Mfma::LDS_FLOATS));

  template <typename Emit>
  static __device__ __forceinline__ void attend(const RunParams& p, const WorkItem& it, const Variant& var,
                                                float* lds, Emit&& emit) {
    if constexpr (KIND == kKindDecode) {
      Decode::run(p, it, var, lds, emit);
    } else if constexpr (KIND == kKindMfma) {
      Mfma::run(p, it, var, lds, emit);
    } else {
      if (it.flags & kItemMfma)
        Mfma::run(p, it, var, lds, emit);
      else
        Decode::run(p, it, var, lds, emit);
    }
  }
};

// Optional per-workgroup timeline (compile with BSR_TRACE): wall-clock stamps at
// phase boundaries, stored after the partial-state segments of the workspace.
#ifdef BSR_TRACE
#define BSR_STAMP(k)                                                                         \
  do {                                                                                       \
    if (threadIdx.x == 0)                                                                    \
      reinterpret_cast<uint64_t*>(ws + p.trace_off)[wg * 8 + (k)] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#else
#define BSR_STAMP(k) \
  do {               \
  } while (0)
#endif

// OCC: workgroups per CU the register allocation must allow.  PAGE1: the pool has
// one key per page (MFMA bodies skip the page division).  KV8: K and V are FP8
// E4M3 codes (decode body; Q and O bf16).  VAR: plans with ALiBi slopes or tree
// masks.
template <int D, bool BF16, int ROWS, int TB, bool CAP, int KIND, int OCC, bool PAGE1 = false, bool KV8 = false,
          bool VAR = false>
__global__ __launch_bounds__(kWgThreads, OCC) void bsr_persistent_kernel(RunParams p) {
  using K = PersistentKernel<D, BF16, ROWS, TB, CAP, KIND, PAGE1, KV8, VAR>;
  __shared__ float lds[K::LDS_FLOATS];
  uint8_t* ws = p.ws;
  // the whole header in one read (its fields are uniform; the empty asm keeps the
  // offsets from being loaded separately after the check below)
  const PlanHeader h = *plan_header(ws);
  asm volatile("" ::"s"(h.off_epochs), "s"(h.off_item_ptr), "s"(h.off_items), "s"(h.off_flags), "s"(h.pool_begin),
               "s"(h.off_claim));
  const Variant var{h.off_alibi != 0, reinterpret_cast<const float*>(ws + h.off_alibi),
                    reinterpret_cast<const uint64_t*>(ws + h.off_tree)};
  const PlanHeader* hdr = &h;
  const int wg = blockIdx.x;
  int32_t* status = plan_i32(ws, hdr->off_status);
  // A plan made for another instance (kind, decode rows, head dim, switches) or
  // another grid is refused as a whole: nothing is written but the status word,
  // which the host's check reports.  This is what a captured launch meets when a
  // later plan needs a different instance.
  constexpr int32_t kKey =
      instance_key(KIND, KIND == kKindMfma ? (K::kShortTile ? 1 : 0) : ROWS, D, BF16, CAP, PAGE1, KV8, VAR);
  if (hdr->instance != kKey || hdr->num_wg != static_cast<int32_t>(gridDim.x)) {
    if (wg == 0 && threadIdx.x == 0) status[kStatusWrongKernel] = 1;
    return;
  }

  int32_t* epochs = plan_i32(ws, hdr->off_epochs);
  int32_t* flags = plan_i32(ws, hdr->off_flags);
  BSR_STAMP(0);
  // the run counter is first needed after the attention items: its (uniform) load
  // is issued here and waited for there, off the items' latency chain
  const int32_t epoch = epochs[wg] + 1;
  const int g = p.group;
  // claim counters: this run uses the one of its epoch's parity (cleared by the
  // previous run, or zero as uploaded) and clears the other for the next run; the
  // previous run, the last user of that one, has ended before this one started
  const bool pooled = hdr->pool_begin < hdr->num_items;
  int32_t* claims = plan_i32(ws, hdr->off_claim);
  if (pooled && wg == 0 && threadIdx.x == 0)
    __hip_atomic_store(claims + ((epoch + 1) & 1), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // ---- attention items -------------------------------------------------------
  // The queue is read-only during the run: scalar loads, and the next item is
  // read while this one runs.
  const int32_t* item_ptr = plan_i32(ws, hdr->off_item_ptr);
  const WorkItem* items = reinterpret_cast<const WorkItem*>(ws + hdr->off_items);
  const int32_t ib = load_invariant(item_ptr + wg), ie = load_invariant(item_ptr + wg + 1);
  bool any_partial = false;
  WorkItem nxt;
  if (ib < ie) nxt = load_invariant(items + ib);
  auto process = [&](const WorkItem& it) {
    if (it.flags & kItemPartial) {
      float* po = reinterpret_cast<float*>(ws + p.partial_o_off);
      float* pl = reinterpret_cast<float*>(ws + p.partial_lse_off);
      auto emit = [&](int r, int d, float o0, float o1, float lse2) {
        const int64_t row = static_cast<int64_t>(it.partial_row) + r;
        const uint64_t pair = (static_cast<uint64_t>(__float_as_uint(o1)) << 32) | __float_as_uint(o0);
        __hip_atomic_store(reinterpret_cast<uint64_t*>(po + row * D + d), pair, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        if (d == 0)
          __hip_atomic_store(reinterpret_cast<uint32_t*>(pl + row), __float_as_uint(lse2), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      };
      K::attend(p, it, var, lds, emit);
      any_partial = true;
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
      K::attend(p, it, var, lds, emit);
    }
  };
  // The workgroup's queue first, then the claimed pool (see below): one loop, so
  // that the bodies are inlined once.
  __shared__ int32_t next_claim;
  int32_t* claim = claims + (epoch & 1);
  int32_t qi = ib;        // next queued item
  bool in_pool = false;   // the queue is done
  bool part_prev = false; // the previous pool item wrote a partial state
  int32_t flag_prev = 0;
  int32_t after = 0;      // thread 0: the claim issued for the next pool item
  while (true) {
    int32_t i;
    if (qi < ie) {
      i = qi++;
    } else {
      if (!in_pool) {
        BSR_STAMP(6);  // (timeline builds: the queue is done)
        // Stamps for the partial states of the queue: every wavefront waits until
        // its device-scope stores have completed (vector memory counter at 0), the
        // workgroup meets, and wavefront 0 stores the stamps.  This is the
        // agent-scope release sequence of the AMDGPU memory model (wait for the
        // vector memory counter, then store the flag) without its write-back of the
        // L2 cache, which only data written into the L2 by non-atomic stores needs:
        // every store of a partial state must stay an agent-scope atomic store, and
        // the merge's reads agent-scope atomic loads (the acquire side without the
        // L2 invalidate).
        if (any_partial) {
          __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
          __syncthreads();
          if (threadIdx.x < 64) {
            for (int32_t k = ib + static_cast<int32_t>(threadIdx.x); k < ie; k += 64) {
              const WorkItem& it = items[k];
              if ((it.flags & (kItemPartial | kItemRelease)) == kItemPartial)
                __hip_atomic_store(flags + it.flag_id, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
          }
        }
        if (!pooled) break;
        // Claimed items: the pool runs in array order (the plan's longest-first
        // order), one item per claim; the next claim is issued before an item runs
        // and read after it.  A partial state is stamped right after its item, with
        // the same release sequence.  Every pool item is claimed by a workgroup that
        // runs it to the end without waiting on anything, and a workgroup reaches
        // its merge tasks only after the pool is exhausted, so every stamp a merge
        // waits for is stored.
        in_pool = true;
        if (threadIdx.x == 0)
          next_claim = __hip_atomic_fetch_add(claim, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
      } else {
        if (part_prev) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();  // every partial store done; every wavefront past next_claim
        if (threadIdx.x == 0) {
          if (part_prev) __hip_atomic_store(flags + flag_prev, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          next_claim = after;
        }
        __syncthreads();
      }
      i = __builtin_amdgcn_readfirstlane(hdr->pool_begin + next_claim);
      if (i >= hdr->num_items) break;
      nxt = load_invariant(items + i);
      if (threadIdx.x == 0) after = __hip_atomic_fetch_add(claim, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const WorkItem it = nxt;
    // the next queued item is read while this one runs
    if (qi < ie) nxt = load_invariant(items + qi);
    part_prev = (it.flags & kItemPartial) != 0;
    flag_prev = it.flag_id;
    process(it);
    // a queued partial state the plan marks for early release is stamped now
    // (the same release sequence), so that its merge need not wait for the rest
    // of this queue (decode and mixed grids; tile grids claim their queue tails)
    if (KIND != kKindMfma && !in_pool && (it.flags & kItemRelease)) {
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();
      if (threadIdx.x == 0) __hip_atomic_store(flags + it.flag_id, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
#ifdef BSR_TRACE
    if (in_pool && threadIdx.x == 0) reinterpret_cast<uint64_t*>(ws + p.trace_off)[wg * 8 + 7] += 1;  // claimed items
    if (!pooled && qi == ib + 1) BSR_STAMP(7);  // end of the first item (plans without a pool)
#endif
  }
  BSR_STAMP(1);

  BSR_STAMP(2);
  // ---- contraction of partial states -----------------------------------------
  const int32_t* merge_ptr = plan_i32(ws, hdr->off_merge_ptr);
  const MergeTask* tasks = reinterpret_cast<const MergeTask*>(ws + hdr->off_merge);
  const MergeSrc* srcs = reinterpret_cast<const MergeSrc*>(ws + hdr->off_srcs);
  const int32_t mb = merge_ptr[wg], me = merge_ptr[wg + 1];
  // the workgroup waits for every source of its tasks (one thread per source),
  // then merges its tasks one after another (the merge reads the states with
  // device-scope loads, so no cache of this XCD can hold them stale)
  bool ok = true;
  if (mb < me) {
    for (int32_t t = mb; t < me && ok; ++t) ok = K::Merge::wait(tasks[t], srcs, flags, epoch, hdr->spin_limit);
    BSR_STAMP(3);
    __syncthreads();
    BSR_STAMP(5);
    for (int32_t t = mb; t < me; ++t) K::Merge::run(p, tasks[t], srcs, lds);
  }
  BSR_STAMP(4);
  if (!ok) status[kStatusWaitTimeout] = 1;

  __syncthreads();
  if (threadIdx.x == 0) epochs[wg] = epoch;
}

}  // namespace bsr
