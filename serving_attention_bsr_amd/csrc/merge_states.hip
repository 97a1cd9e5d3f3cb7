// merge_states.hip -- stand-alone ⊕ of two arrays of attention states.
//
// Terms "Attention State and ⊕" of the FlashInfer explainer page (paper section
// 2.2): (O_a, a) ⊕ (O_b, b) = ((e^a O_a + e^b O_b) / (e^a + e^b), log(e^a + e^b)),
// evaluated with the larger LSE factored out; (0, -inf) is the identity.  Natural
// log in and out.  One wavefront per row: every lane reads the row's two LSEs
// and its own elements before writing, so the output may alias an input.
#include <hip/hip_runtime.h>

#include "kernels/common.hpp"

namespace bsr {

__global__ __launch_bounds__(256) void merge_states_kernel(const float* o_a, const float* lse_a,
                                                           const float* o_b, const float* lse_b,
                                                           float* o, float* lse, int64_t rows,
                                                           int32_t d) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;
  const float a = lse_a[r], b = lse_b[r];
  const float m = __builtin_fmaxf(a, b);
  const bool empty = m == kNegInf;
  const float wa = empty ? 0.0f : __expf(a - m);
  const float wb = empty ? 0.0f : __expf(b - m);
  const float z = wa + wb;
  const float inv = empty ? 0.0f : 1.0f / z;
  for (int32_t e = lane; e < d; e += 64) {
    const int64_t i = r * d + e;
    o[i] = (wa * o_a[i] + wb * o_b[i]) * inv;
  }
  if (lane == 0) lse[r] = empty ? kNegInf : m + __logf(z);
}

}  // namespace bsr

extern "C" int bsr_launch_merge_states(const float* o_a, const float* lse_a, const float* o_b,
                                        const float* lse_b, float* o, float* lse, int64_t rows,
                                        int32_t d, hipStream_t s) {
  if (rows == 0) return 0;
  const int64_t blocks = (rows + 3) / 4;
  hipLaunchKernelGGL(bsr::merge_states_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, s,
                     o_a, lse_a, o_b, lse_b, o, lse, rows, d);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}
