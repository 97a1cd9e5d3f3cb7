// run_static.hip -- bsr_attn_run_static: run() without a caller-provided
// workspace, for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The workspace (plan blob, partial states, ready stamps, status words) lives in
// one file-scope device array of fixed size.  Its device address is looked up
// once per device, with that device current, at handle creation; host code uses
// only that address (the array's name on the host is a stand-in, not a device
// address).  Each call copies the plan staged by the handle's last plan call into
// the array, which also clears every word that must start at zero (run counters,
// ready stamps, status words), then launches the persistent kernel on it.  Every
// call on one device shares that device's array: calls that overlap on one device
// (several streams or handles) race and must be ordered by the caller.
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>
#include <string>

#include "bsr_attn.h"
#include "handle.h"
#include "layout.h"

namespace bsr {

namespace {

// Workspace bytes of the static variant: a handle whose workspace is larger is
// rejected (lower max_partial_rows or the other maxima at create).
constexpr int64_t kScratchBytes = int64_t(64) << 20;
constexpr int kMaxDevices = 64;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

int static_scratch(int device, uint8_t** ptr, int64_t* bytes) {
  if (device < 0 || device >= kMaxDevices) return fail(BSR_ERR_UNSUPPORTED, "device index beyond the scratch table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[device] == nullptr) {
    DeviceGuard guard(device);
    if (guard.err != hipSuccess) return hip_fail(guard.err, "hipSetDevice");
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[device] = static_cast<uint8_t*>(p);
  }
  *ptr = g_scratch_ptr[device];
  *bytes = kScratchBytes;
  return BSR_OK;
}

}  // namespace bsr

extern "C" int bsr_attn_run_static(bsr_attn_t h, const void* q, const void* k_pool, const void* v_pool,
                                   const int32_t* kv_indices, void* o, float* lse, const void* host_staging,
                                   void* stream) {
  using bsr::fail;
  using bsr::hip_fail;
  if (h == nullptr) return fail(BSR_ERR_INVALID_ARG, "handle is null");
  if (h->device < 0) return fail(BSR_ERR_INVALID_ARG, "a host-only handle cannot run");
  if (!h->has_plan || h->last_kernel == nullptr) return fail(BSR_ERR_INVALID_ARG, "run_static before any plan");
  if (host_staging == nullptr || host_staging != h->last_staging)
    return fail(BSR_ERR_INVALID_ARG, "host_staging must be the buffer the handle's last plan was written to");
  if (q == nullptr || k_pool == nullptr || v_pool == nullptr || kv_indices == nullptr || o == nullptr)
    return fail(BSR_ERR_INVALID_ARG, "null device pointer");
  uint8_t* ws = nullptr;
  int64_t bytes = 0;
  if (int rc = bsr::static_scratch(h->device, &ws, &bytes)) return rc;
  if (h->ws_bytes > bytes)
    return fail(BSR_ERR_CAPACITY, "this handle's workspace (" + std::to_string(h->ws_bytes) +
                                      " bytes) exceeds the static scratch (" + std::to_string(bytes) +
                                      " bytes); create it with a smaller max_partial_rows or smaller maxima");
  bsr::DeviceGuard guard(h->device);
  if (guard.err != hipSuccess) return hip_fail(guard.err, "hipSetDevice");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t blob = h->last.blob.size();
  hipError_t e = hipMemcpyAsync(ws, host_staging, blob, hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync");
  // the next plan call waits for this copy before it rewrites the staging buffer
  // (under capture the copy happens at each replay, and ordering re-plans against
  // replays is the caller's)
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  e = hipStreamIsCapturing(s, &cap);
  if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
  if (cap == hipStreamCaptureStatusNone) {
    e = hipEventRecord(h->upload_done, s);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
    h->upload_pending = true;
  }
  bsr::RunParams p = h->params;
  p.q = q;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.kv_indices = kv_indices;
  p.o = o;
  p.lse = lse;
  p.ws = ws;
  void* args[] = {&p};
  e = hipLaunchKernel(h->last_kernel, dim3(static_cast<uint32_t>(h->last.num_wg)), dim3(bsr::kWgThreads), args, 0, s);
  if (e != hipSuccess) return hip_fail(e, "hipLaunchKernel");
  bsr::PlanHeader hdr;
  std::memcpy(&hdr, h->last.blob.data(), sizeof(hdr));
  h->static_off_status = hdr.off_status;
  h->has_static = true;
  return BSR_OK;
}
