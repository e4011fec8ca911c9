// Device scratch of contexts created with gpuos_create_static (the entry
// point for callers that cannot allocate device memory): the scheduler state
// the resident kernel uses (control block, device descriptor ring, ticket
// ends, completion words, tile counters) lives in this file-scope array
// instead of hipMalloc'd memory.  Each device the library runs on holds its
// own copy of the array until the process ends.  In host code the array's
// name is not a device address: its address on a device is taken once per
// device, with that device current, and only that address is used.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gpuos_internal.h"
#include "kernels.h"

namespace gpuos {

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {

struct DeviceScratch {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
DeviceScratch g_scratch[kMaxStaticDevices];

}  // namespace

hipError_t static_scratch(int device, void** ptr) {
  *ptr = nullptr;
  if (device < 0 || device >= kMaxStaticDevices) return hipErrorInvalidDevice;
  DeviceScratch& d = g_scratch[device];
  std::call_once(d.once, [&d, device] {
    int prev = -1;
    const hipError_t g = hipGetDevice(&prev);
    d.err = hipSetDevice(device);
    if (d.err == hipSuccess) d.err = hipGetSymbolAddress(&d.ptr, HIP_SYMBOL(scratch));
    if (g == hipSuccess && prev != device) (void)hipSetDevice(prev);
    if (d.err != hipSuccess) d.ptr = nullptr;
  });
  *ptr = d.ptr;
  return d.err;
}

}  // namespace gpuos
