// Persistent-kernel instances for head_dim 64, for plans with ALiBi slopes or
// tree masks.
#include "kernels/instances.hpp"

namespace bsr {
void register_d64_var(std::vector<KernelEntry>* out) { register_head_dim<64, true>(out); }
}  // namespace bsr
