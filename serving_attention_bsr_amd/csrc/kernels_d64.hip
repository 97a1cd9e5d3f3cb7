// Persistent-kernel instances for head_dim 64.
#include "kernels/instances.hpp"

namespace bsr {
void register_d64(std::vector<KernelEntry>* out) { register_head_dim<64, false>(out); }
}  // namespace bsr
