// Error reporting and device queries shared by the three entry points.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "common.hpp"

namespace {
thread_local char g_msg[512] = "";
}

namespace spec {

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_msg[0] = '\0'; }

int launched(const char *what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SPEC_EHIP, "%s: %s", what, hipGetErrorString(e));
  return SPEC_OK;
}

int device_cus() {
  static std::mutex mu;
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

int ensure_dynamic_lds(const void *kernel, size_t bytes, std::atomic<uint64_t> &done,
                       const char *who) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(SPEC_EHIP, "%s: hipGetDevice failed", who);
  const uint64_t bit = (dev >= 0 && dev < 64) ? (1ull << dev) : 0ull;
  if (bit != 0 && (done.load(std::memory_order_acquire) & bit) != 0) return SPEC_OK;
  if (hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) !=
      hipSuccess)
    return fail(SPEC_EHIP, "%s: cannot reserve %zu bytes of LDS on device %d", who, bytes, dev);
  done.fetch_or(bit, std::memory_order_release);
  return SPEC_OK;
}

}  // namespace spec

extern "C" int spec_version(void) { return (1 << 16) | 0; }

extern "C" const char *spec_last_error(void) { return g_msg; }
