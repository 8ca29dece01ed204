// Host bookkeeping for the device entry points: the per-thread last HIP
// error and the status a launch reports.
#include <hip/hip_runtime.h>

#include "binade.h"
#include "device_common.h"

namespace binade {

namespace {
thread_local int32_t g_last_hip_error = 0;
}

void set_last_hip_error(int32_t e) { g_last_hip_error = e; }

int32_t launch_status() {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int32_t>(e);
    return BINADE_EHIP;
  }
  return BINADE_OK;
}

}  // namespace binade

extern "C" int32_t binade_last_hip_error(void) {
  return binade::g_last_hip_error;
}
