// Persistent-kernel instances for head_dim 256, for plans with ALiBi slopes or
// tree masks.
#include "kernels/instances.hpp"

namespace bsr {
void register_d256_var(std::vector<KernelEntry>* out) { register_head_dim<256, true>(out); }
}  // namespace bsr
