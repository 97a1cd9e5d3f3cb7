// Persistent-kernel instances for head_dim 128, for plans with ALiBi slopes or
// tree masks.
#include "kernels/instances.hpp"

namespace bsr {
void register_d128_var(std::vector<KernelEntry>* out) { register_head_dim<128, true>(out); }
}  // namespace bsr
