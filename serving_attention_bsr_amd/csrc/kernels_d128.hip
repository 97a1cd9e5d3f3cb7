// Persistent-kernel instances for head_dim 128.
#include "kernels/instances.hpp"

namespace bsr {
void register_d128(std::vector<KernelEntry>* out) { register_head_dim<128, false>(out); }
}  // namespace bsr
