// Host-side plumbing shared by every entry point: thread-local error text and
// a per-device attribute cache.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <mutex>

#include "hs_common.hpp"

namespace hs {

static thread_local char g_last_error[512] = "";

int set_error(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int device_info(DeviceInfo* out) {
  static std::mutex mu;
  static DeviceInfo cache[64];
  static bool have[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return set_error(HS_ELAUNCH, "hipGetDevice failed");
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!have[dev]) {
    int lds = 0, cus = 0;
    if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
      (void)hipGetLastError();
      return set_error(HS_ELAUNCH, "hipDeviceGetAttribute failed on device %d", dev);
    }
    cache[dev] = DeviceInfo{dev, lds, cus};
    have[dev] = true;
  }
  *out = cache[dev];
  return HS_OK;
}

}  // namespace hs

extern "C" const char* hisparse_last_error(void) { return hs::g_last_error; }
