// Per-op comparator kernel (gfx950): one launch per descriptor, every wave
// runs tiles wave, wave + waves, ... of that descriptor with the same tile
// bodies as the resident kernel and the default cache policy (the kernel
// boundary orders each launch's memory accesses after the previous one's).
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "gpuos_internal.h"
#include "kernels.h"
#include "tile_ops.h"

namespace gpuos {

__global__ __launch_bounds__(256) void gpuos_single(DevDesc d, uint32_t* err) {
  const uint32_t wave = (blockIdx.x * blockDim.x + threadIdx.x) / 64;
  const uint32_t waves = gridDim.x * blockDim.x / 64;
  // the descriptor goes to this wave's LDS slot, as in the resident kernel
  __shared__ uint32_t sdesc[4][64];
  __shared__ float sscr[4][kWaveScratch];
  lds_u32* slot = (lds_u32*)&sdesc[threadIdx.x / 64][0];
  lds_f32* scr = (lds_f32*)&sscr[threadIdx.x / 64][0];
  slot[lane_id()] = reinterpret_cast<const uint32_t*>(&d)[lane_id()];
  const SDesc v{slot};
  const uint32_t ntiles = v(6);
  for (uint32_t t = wave; t < ntiles; t += waves) {
    const uint32_t e = exec_tile<CP_DEFAULT, CP_DEFAULT>(v, t, scr);
    if (e && lane_id() == 0 && err) *err = e;
  }
}

hipError_t launch_single(const DevDesc& d, uint32_t* err, hipStream_t s) {
  uint32_t waves = d.ntiles;
  uint32_t blocks = (waves + 3) / 4;
  if (blocks > 16384) blocks = 16384;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(gpuos_single, dim3(blocks), dim3(256), 0, s, d, err);
  return hipGetLastError();
}

// An empty kernel: one workgroup of one wave that does nothing, so that a
// launch measures the launch path alone.
__global__ __launch_bounds__(64) void gpuos_empty() {}

hipError_t launch_empty(hipStream_t s) {
  hipLaunchKernelGGL(gpuos_empty, dim3(1), dim3(64), 0, s);
  return hipGetLastError();
}

}  // namespace gpuos
