// Persistent-kernel instances for head_dim 256.
#include "kernels/instances.hpp"

namespace bsr {
void register_d256(std::vector<KernelEntry>* out) { register_head_dim<256, false>(out); }
}  // namespace bsr
