// Status strings, HIP error bookkeeping and the gfx950 device check.
#include <cstring>

#include "common.h"

namespace {
thread_local int g_last_hip_error = 0;
constexpr int kMaxDevices = 64;
int g_device_ok[kMaxDevices] = {0};  // 0 unknown, 1 gfx950, 2 other
int g_cu_count[kMaxDevices] = {0};   // 0 unknown
}  // namespace

namespace moe {

moe_status_t check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_DEVICE;
  int state = __atomic_load_n(&g_device_ok[dev], __ATOMIC_RELAXED);
  if (state == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e);
    state = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    __atomic_store_n(&g_device_ok[dev], state, __ATOMIC_RELAXED);
  }
  return state == 1 ? MOE_OK : MOE_ERR_DEVICE;
}

int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int n = __atomic_load_n(&g_cu_count[dev], __ATOMIC_RELAXED);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    __atomic_store_n(&g_cu_count[dev], n, __ATOMIC_RELAXED);
  }
  return n;
}

moe_status_t allow_dynamic_lds(const void* func, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t{1} << dev) : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return MOE_OK;
  e = hipFuncSetAttribute(func, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return hip_fail(e);
  if (bit) done.fetch_or(bit, std::memory_order_release);
  return MOE_OK;
}

moe_status_t hip_fail(hipError_t e) {
  g_last_hip_error = static_cast<int>(e);
  return MOE_ERR_HIP;
}

moe_status_t launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? MOE_OK : hip_fail(e);
}

}  // namespace moe

extern "C" const char* moe_status_str(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_NULL: return "MOE_ERR_NULL: a required pointer is NULL";
    case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE: a size is out of range or not a required multiple";
    case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN: a pointer is not 16-byte aligned";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or too small";
    case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE: the current device is not gfx950";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: unsupported argument combination";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP call failed";
  }
  return "unknown moe_status_t";
}

extern "C" int moe_last_hip_error(void) { return g_last_hip_error; }
