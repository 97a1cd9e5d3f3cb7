// common.hpp -- gfx950 device helpers shared by the attention bodies.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../layout.h"
#include "../params.h"

namespace bsr {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// tanh from its exponential definition: tanh|x| = (1 - e) / (1 + e), e = exp(-2|x|).
__device__ __forceinline__ float tanh_exp(float x) {
  const float ax = __builtin_fabsf(x);
  const float e = fast_exp2(-2.0f * kLog2e * ax);
  const float t = (1.0f - e) * fast_rcp(1.0f + e);
  return __builtin_copysignf(t, x);
}

// Lazy reference maximum of the online softmax (base 2) of the MFMA bodies: a
// row's reference moves only when a tile's maximum exceeds it by more than
// kLazyMax, so most tiles leave the output accumulator unscaled.  The result is the
// same: O and the sum are both relative to the reference, and exp2(s - m_ref) is
// then at most 2^kLazyMax, which the fp32 sums and the bf16 probabilities hold as
// accurately as values up to 1.  A first finite maximum is always taken
// (-inf + kLazyMax = -inf).
constexpr float kLazyMax = 8.0f;
__device__ __forceinline__ float lazy_max(float m_ref, float tile_max) {
  return tile_max > m_ref + kLazyMax ? tile_max : m_ref;
}

// Unsigned division of n < 2^31 by a divisor fixed at set-up (Granlund and
// Montgomery, "Division by invariant integers using multiplication", 1994).
__device__ __forceinline__ uint32_t div_magic(uint32_t n, uint32_t magic, int32_t shift) {
  return (__umulhi(magic, n) + n) >> shift;
}

// bf16 <-> fp32.  A bf16 is the high half of an fp32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));  // round to nearest even
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Row gather through a structured buffer resource: the address unit computes
// base + row * stride + offset itself, so a KV row index (32 bits, pools up to
// 2^31 rows) needs no 64-bit address arithmetic on the vector ALU.  Offsets stay
// below the row stride (the range check of structured buffers).
__device__ u32x4_t bsr_struct_load_b128(__amdgpu_buffer_rsrc_t rsrc, int vindex, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.struct.ptr.buffer.load.v4i32");

// The same 16-byte row gather written straight into LDS, without passing through
// registers: lane i of the wavefront lands at lds + 16 i (lds is wave-uniform;
// the low 32 bits of a generic pointer into LDS are its LDS address).  Completion
// is counted by the vector memory counter like any load; the writes are visible
// to the rest of the workgroup after that counter drains and a barrier, which the
// callers issue explicitly before a gathered buffer is read.  The load is issued
// from an asm statement (it writes no register; M0 is set in the same statement):
// the compiler cannot tell two LDS buffers apart, so for the intrinsic it would
// wait for every gather in flight (the next tile's, into the other buffer) before
// any later LDS read it cannot prove independent, such as the transpose reads.
typedef int i32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void lds_gather_b128(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds_addr, int vindex,
                                                int voffset) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
  const i32x2_t va = {vindex, voffset};
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 idxen offen lds" ::"s"(m0), "v"(va), "s"(rsrc)
               : "memory");
}
__device__ __forceinline__ uint32_t lds_addr_of(const void* lds) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
}
__device__ __forceinline__ void lds_gather_b128(__amdgpu_buffer_rsrc_t rsrc, void* lds, int vindex, int voffset) {
  lds_gather_b128(rsrc, lds_addr_of(lds), vindex, voffset);
}

// Element i of a 32-bit array through a raw buffer resource (32-bit offset).
__device__ __forceinline__ uint32_t load_u32(__amdgpu_buffer_rsrc_t rsrc, int i) {
  return __builtin_amdgcn_raw_buffer_load_b32(rsrc, i * 4, 0, 0);
}

// Resource over rows of `stride` bytes starting at base (dword 3: 32-bit data,
// the raw-buffer format of gfx9 parts).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, int stride) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(stride), 0x7fffffff,
                                           0x00020000);
}
// Two OCP FP8 E4M3 codes (the low or high 16 bits of w) as a bf16 pair, exactly
// (E4M3 values are bf16 values): the gfx950 scaled conversion with scale 1, whose
// decoding of all 256 codes was checked against the format on the GPU.
template <bool HIGH>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HIGH));
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// DPP lane moves (row = 16 lanes).  Control words of the gfx9 DPP encoding.
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141; // lane i <-> 7-i within each 8
constexpr int kDppRowMirror = 0x140;     // lane i <-> 15-i within each 16

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of N lanes (N in 1, 2, 4, 8, 16); every lane of a group
// ends with the group's sum.  Quad steps pair lanes by xor; the mirror steps pair
// each lane with one of the other half, whose value is already the half's sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "group size");
  if constexpr (N >= 2) x += dpp_mov<kDppQuadXor1>(x);
  if constexpr (N >= 4) x += dpp_mov<kDppQuadXor2>(x);
  if constexpr (N >= 8) x += dpp_mov<kDppRowHalfMirror>(x);
  if constexpr (N >= 16) x += dpp_mov<kDppRowMirror>(x);
  return x;
}

// The values of this lane and of the lane MASK (16 or 32) lanes away, as a pair in
// lane order (the same pair on both lanes), by the gfx950 lane-half swaps: no LDS
// round trip, and both lanes combine the pair in the same order.
template <int MASK>
__device__ __forceinline__ void lane_pair(float x, float& lo, float& hi) {
  static_assert(MASK == 16 || MASK == 32, "lane-half swaps exchange 16 or 32 lanes apart");
  const uint32_t u = __float_as_uint(x);
  if constexpr (MASK == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
  }
}
template <int MASK>
__device__ __forceinline__ float pair_max(float x) {
  float lo, hi;
  lane_pair<MASK>(x, lo, hi);
  return __builtin_fmaxf(lo, hi);
}
template <int MASK>
__device__ __forceinline__ float pair_sum(float x) {
  float lo, hi;
  lane_pair<MASK>(x, lo, hi);
  return lo + hi;
}

// Variant data of one plan, read from its blob: ALiBi slopes per query head in
// units of the unscaled logit (slope / sm_scale), and one 64-bit tree-mask row
// per query token (bit u: the token sees key tree_lo + u of its block row).  An
// absent array points at the start of the workspace instead of null, so that no
// load, even one the compiler issues early, leaves valid memory (the workspace
// holds at least 4 H_qo + 8 max_total_qo bytes).
struct Variant {
  bool has_alibi;
  const float* alibi;
  const uint64_t* tree;
};

// Workspace views.
__device__ __forceinline__ const PlanHeader* plan_header(const uint8_t* ws) {
  return reinterpret_cast<const PlanHeader*>(ws);
}
__device__ __forceinline__ int32_t* plan_i32(uint8_t* ws, int32_t off) {
  return reinterpret_cast<int32_t*>(ws + off);
}


// Load of memory that no thread writes during the kernel (the plan's queues),
// through the constant address space: uniform reads become scalar loads, which
// can be issued ahead of use without holding vector registers.  (The host pass
// of the single-source compile sees a plain read; it never runs this code.)
template <typename T>
__device__ __forceinline__ T load_invariant(const T* p) {
  static_assert(sizeof(T) % 4 == 0, "whole dwords");
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(4))) const uint32_t c_u32;
  c_u32* q = (c_u32*)(p);
  uint32_t w[sizeof(T) / 4];
#pragma unroll
  for (int i = 0; i < static_cast<int>(sizeof(T) / 4); ++i) w[i] = q[i];
  return __builtin_bit_cast(T, w);
#else
  return *p;
#endif
}

// s_waitcnt operand (gfx9 encoding) that waits for every outstanding vector
// memory access: vmcnt 0, expcnt and lgkmcnt left at their maxima.
constexpr int kWaitVmcnt0 = 0x0F70;

// Device-scope loads of partial states (read past the per-XCD L2 caches).
__device__ __forceinline__ float load_dev_f32(const float* p) {
  return __uint_as_float(
      __hip_atomic_load(reinterpret_cast<const uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ float4 load_dev_f32x4(const float* p) {
  const uint64_t a = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t b =
      __hip_atomic_load(reinterpret_cast<const uint64_t*>(p) + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float4(__uint_as_float(static_cast<uint32_t>(a)), __uint_as_float(static_cast<uint32_t>(a >> 32)),
                     __uint_as_float(static_cast<uint32_t>(b)), __uint_as_float(static_cast<uint32_t>(b >> 32)));
}

// Wait (bounded) until *flag == epoch: at most spin_limit polls.  Returns false if
// the bound expired.
__device__ __forceinline__ bool wait_flag(const int32_t* flag, int32_t epoch, int32_t spin_limit) {
  int spins = 0;
  while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != epoch) {
    __builtin_amdgcn_s_sleep(2);
    if (++spins > spin_limit) return false;
  }
  return true;
}

}  // namespace bsr
