// instances.hpp -- explicit instances of the persistent kernel for one head_dim.
#pragma once

#include "persistent.hpp"
#include "registry.h"

namespace bsr {

// KV rows per lane group per wavefront step: two for bf16; one for fp32, whose
// rows take twice the registers.
#ifndef BSR_DECODE_TB
#define BSR_DECODE_TB 2
#endif
#ifndef BSR_DECODE_OCC
#define BSR_DECODE_OCC 1
#endif
template <bool BF16>
constexpr int kDecodeTb = BF16 ? BSR_DECODE_TB : 1;

// Workgroups per CU the register allocation must allow.
template <int D, bool BF16, int ROWS>
constexpr int kDecodeOcc = (BF16 && ROWS == 4) ? BSR_DECODE_OCC : 1;
// Default grid of the decode body: one workgroup per CU.  The KV stream is
// bound by the chip's bandwidth, not by per-CU latency hiding, and a second
// workgroup per CU only shortens chunks (more partial states) and shares the CU.
constexpr int kDecodeWgPerCu = 1;

template <int D, bool BF16, int ROWS, bool CAP, bool VAR>
inline void add_decode(std::vector<KernelEntry>* out) {
  out->push_back({KernelKey{kKindDecode, BF16, D, ROWS, CAP, false, false, VAR},
                  reinterpret_cast<const void*>(
                      &bsr_persistent_kernel<D, BF16, ROWS, kDecodeTb<BF16>, CAP, kKindDecode,
                                             kDecodeOcc<D, BF16, ROWS>, false, false, VAR>),
                  kDecodeWgPerCu});
}

// FP8 (E4M3) K/V with bf16 Q/O: four KV rows per lane group and step, the bytes in
// flight of the bf16 body's two.
template <int D, int ROWS, bool CAP, bool VAR>
inline void add_decode_kv8(std::vector<KernelEntry>* out) {
  out->push_back({KernelKey{kKindDecode, true, D, ROWS, CAP, false, true, VAR},
                  reinterpret_cast<const void*>(
                      &bsr_persistent_kernel<D, true, ROWS, 2 * kDecodeTb<true>, CAP, kKindDecode, 1, false, true,
                                             VAR>),
                  kDecodeWgPerCu});
}

// MFMA kernels: two workgroups per CU, so that one workgroup's softmax and
// gather run while the other's matrix products do (both MFMA bodies fit 256
// registers per lane).
template <int D>
constexpr int kMfmaOcc = 2;

template <int D, bool CAP, bool PAGE1, bool VAR, bool KV8 = false>
inline void add_mfma(std::vector<KernelEntry>* out) {
  out->push_back({KernelKey{kKindMfma, true, D, 0, CAP, PAGE1, KV8, VAR},
                  reinterpret_cast<const void*>(
                      &bsr_persistent_kernel<D, true, 4, kDecodeTb<true>, CAP, kKindMfma, kMfmaOcc<D>, PAGE1, KV8,
                                             VAR>),
                  kMfmaOcc<D>});
}

// The 64-row tile at head dim 128 (short query rows: speculative drafts, small
// prefill chunks): the 16-row body, whose 153 registers per lane allow three
// workgroups per CU (kernel key rows = 1).
template <bool CAP, bool PAGE1, bool VAR>
inline void add_mfma_short(std::vector<KernelEntry>* out) {
  out->push_back({KernelKey{kKindMfma, true, 128, 1, CAP, PAGE1, false, VAR},
                  reinterpret_cast<const void*>(
                      &bsr_persistent_kernel<128, true, 1, kDecodeTb<true>, CAP, kKindMfma, 3, PAGE1, false, VAR>),
                  3});
}

// (an FP8 cache's decode body takes four KV rows per lane group and step)
template <int D, int ROWS, bool CAP, bool VAR, bool KV8 = false>
inline void add_mixed(std::vector<KernelEntry>* out) {
  out->push_back({KernelKey{kKindMixed, true, D, ROWS, CAP, false, KV8, VAR},
                  reinterpret_cast<const void*>(
                      &bsr_persistent_kernel<D, true, ROWS, (KV8 ? 2 : 1) * kDecodeTb<true>, CAP, kKindMixed, 1,
                                             false, KV8, VAR>),
                  1});
}

// VAR: instances for plans with ALiBi slopes or tree masks (compiled in their own
// translation units).
template <int D, bool VAR>
inline void register_head_dim(std::vector<KernelEntry>* out) {
  add_mfma<D, false, false, VAR>(out);
  add_mfma<D, true, false, VAR>(out);
  // one key per page (radix-tree layout): prefill without the page division
  add_mfma<D, false, true, VAR>(out);
  add_mfma<D, true, true, VAR>(out);
  add_mixed<D, 4, false, VAR>(out);
  add_mixed<D, 4, true, VAR>(out);
  add_mixed<D, 8, false, VAR>(out);
  add_mixed<D, 8, true, VAR>(out);
  add_decode<D, true, 4, false, VAR>(out);
  add_decode<D, true, 4, true, VAR>(out);
  add_decode<D, true, 8, false, VAR>(out);
  add_decode<D, true, 8, true, VAR>(out);
  add_decode<D, false, 4, false, VAR>(out);
  add_decode<D, false, 4, true, VAR>(out);
  add_decode<D, false, 8, false, VAR>(out);
  add_decode<D, false, 8, true, VAR>(out);
  add_decode_kv8<D, 4, false, VAR>(out);
  add_decode_kv8<D, 4, true, VAR>(out);
  add_decode_kv8<D, 8, false, VAR>(out);
  add_decode_kv8<D, 8, true, VAR>(out);
  if constexpr (D == 128) {
    add_mfma_short<false, false, VAR>(out);
    add_mfma_short<true, false, VAR>(out);
    add_mfma_short<false, true, VAR>(out);
    add_mfma_short<true, true, VAR>(out);
  }
  if constexpr (D <= 128) {
    // FP8 K/V on the 32-row MFMA body (prefill and wide rows)
    add_mfma<D, false, false, VAR, true>(out);
    add_mfma<D, true, false, VAR, true>(out);
    add_mfma<D, false, true, VAR, true>(out);
    add_mfma<D, true, true, VAR, true>(out);
    add_mixed<D, 4, false, VAR, true>(out);
    add_mixed<D, 4, true, VAR, true>(out);
    add_mixed<D, 8, false, VAR, true>(out);
    add_mixed<D, 8, true, VAR, true>(out);
  }
}

}  // namespace bsr
