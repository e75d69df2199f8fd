// Per-device facts the launchers need, set up once per device and process.
//
// The launchers size persistent grids by the device's CU count and raise some kernels' dynamic
// LDS limit above the default.  Both are properties of a device, so they are kept per device
// (the calling thread's current device, which the caller's stream belongs to) and initialised
// under std::call_once / a mutex, so that host threads may call the library concurrently and a
// process may drive several GPUs.  Nothing else persists between calls.
#include <mutex>
#include <set>
#include <utility>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kMaxDevices = 64;

std::once_flag g_cu_once[kMaxDevices];
int g_cu_count[kMaxDevices];
hipError_t g_cu_err[kMaxDevices];

std::mutex g_attr_mutex;
std::set<std::pair<int, std::pair<const void*, int>>> g_attr_done;   // (device, (kernel, bytes))

}  // namespace

hipError_t current_device(int* dev) {
  hipError_t e = hipGetDevice(dev);
  if (e != hipSuccess) return e;
  return (*dev >= 0 && *dev < kMaxDevices) ? hipSuccess : hipErrorInvalidDevice;
}

hipError_t device_cu_count(int* n_cu) {
  int dev = 0;
  hipError_t e = current_device(&dev);
  if (e != hipSuccess) return e;
  std::call_once(g_cu_once[dev], [dev] {
    g_cu_err[dev] = hipDeviceGetAttribute(&g_cu_count[dev], hipDeviceAttributeMultiprocessorCount, dev);
  });
  if (g_cu_err[dev] != hipSuccess) return g_cu_err[dev];
  *n_cu = g_cu_count[dev];
  return hipSuccess;
}

hipError_t ensure_dynamic_lds(const void* kernel, int bytes) {
  int dev = 0;
  hipError_t e = current_device(&dev);
  if (e != hipSuccess) return e;
  const auto key = std::make_pair(dev, std::make_pair(kernel, bytes));
  std::lock_guard<std::mutex> lock(g_attr_mutex);
  if (g_attr_done.count(key)) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) g_attr_done.insert(key);
  return e;
}

}  // namespace moe
