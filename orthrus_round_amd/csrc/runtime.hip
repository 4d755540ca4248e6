// Host-side plumbing shared by all entry points: thread-local error string, status helpers,
// ABI version.
#include <cstdarg>
#include <mutex>
#include <vector>

#include "common.hpp"

namespace orthrus {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

int32_t fail(int32_t status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

void allow_lds_once(const void* kernel, size_t bytes) {
  static std::mutex mu;
  static std::vector<const void*> done;
  std::lock_guard<std::mutex> lock(mu);
  for (const void* k : done)
    if (k == kernel) return;
  (void)hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  done.push_back(kernel);
}

int32_t check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ORTHRUS_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ORTHRUS_OK;
}

}  // namespace orthrus

extern "C" int32_t orthrus_abi_version(void) { return ORTHRUS_ABI_VERSION; }
extern "C" const char* orthrus_last_error(void) { return orthrus::g_last_error.c_str(); }
