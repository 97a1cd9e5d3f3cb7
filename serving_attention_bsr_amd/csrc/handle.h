// handle.h -- the library's handle and the host helpers its C entry points share
// (private: not part of the C ABI).
#pragma once

#include <hip/hip_runtime_api.h>

#include <stdint.h>

#include <string>

#include "params.h"
#include "plan.h"

namespace bsr {

// Thread-local message of the last failed call (bsr_attn_last_error).
extern thread_local std::string g_error;
int fail(int code, const std::string& msg);
int hip_fail(hipError_t e, const char* what);

inline int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Makes a device current for the duration of a call, then restores the caller's.
struct DeviceGuard {
  int prev = -1;
  bool active = false;
  hipError_t err = hipSuccess;
  explicit DeviceGuard(int dev) {
    if (dev < 0) return;
    err = hipGetDevice(&prev);
    if (err != hipSuccess) return;
    if (prev != dev) {
      err = hipSetDevice(dev);
      active = err == hipSuccess;
    }
  }
  ~DeviceGuard() {
    if (active) (void)hipSetDevice(prev);
  }
};

// Device address of the library's static scratch array on the current device
// (looked up once per device; defined next to the array).  Returns BSR_OK or a
// status with the message set.
int static_scratch(int device, uint8_t** ptr, int64_t* bytes);

}  // namespace bsr

struct bsr_attn {
  bsr_attn_config cfg;
  int device = -1;
  int cus = 0;  // compute units of the device (0 for host-only handles)
  bsr::PlanConfig pc;
  int32_t num_wg[4][2][2] = {};  // [kind][decode rows 4/8][variant data]
  int64_t plan_capacity = 0;
  int64_t partial_o_off = 0, partial_lse_off = 0, ws_bytes = 0;
  hipEvent_t upload_done = nullptr;
  bool upload_pending = false;
  bool has_plan = false;
  bsr::PlanResult last;            // the last plan made (reported by plan_get_info)
  const void* last_kernel = nullptr;  // its kernel (device handles)
  const void* last_staging = nullptr; // the staging buffer it was written to
  // the last plan uploaded into a workspace: what run() launches
  bool has_upload = false;
  int32_t off_status = 0;
  int32_t run_wg = 0;
  const void* kernel = nullptr;
  // the last plan uploaded into the static scratch (bsr_attn_run_static)
  bool has_static = false;
  int32_t static_off_status = 0;
  bsr::RunParams params;
};
