// registry.h -- the persistent-kernel instances built into the library.
#pragma once

#include <vector>

#include "../params.h"

namespace bsr {

struct KernelEntry {
  KernelKey key;
  const void* fn;     // host stub of __global__ void(RunParams)
  int wg_per_cu;      // default grid: this many workgroups per CU (if resident)
};

// Each instance file appends its kernels.
void register_d64(std::vector<KernelEntry>* out);
void register_d128(std::vector<KernelEntry>* out);
void register_d256(std::vector<KernelEntry>* out);
// instances for plans with ALiBi slopes or tree masks
void register_d64_var(std::vector<KernelEntry>* out);
void register_d128_var(std::vector<KernelEntry>* out);
void register_d256_var(std::vector<KernelEntry>* out);

}  // namespace bsr
