// Status strings and per-device host state of libpagedkv.
#include <mutex>

#include "common.hpp"

extern "C" const char* pkv_status_string(pkv_status status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID_ARG: return "invalid argument";
    case PKV_ERR_UNSUPPORTED: return "unsupported dtype, head_dim, head ratio or block size";
    case PKV_ERR_WORKSPACE_TOO_SMALL: return "decode workspace too small";
    case PKV_ERR_HIP: return "HIP kernel launch failed";
  }
  return "unknown status";
}

namespace pkv_host {

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
int g_cu[kMaxDevices];
}  // namespace

int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  std::call_once(g_once[dev], [dev] {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    g_cu[dev] = n;
  });
  return g_cu[dev];
}

pkv_status launch_status() { return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP; }

}  // namespace pkv_host
