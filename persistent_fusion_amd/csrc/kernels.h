// Host-side launchers of the device kernels (kernels.hip).
#pragma once

#include <hip/hip_runtime_api.h>

#include "gpuos_internal.h"

namespace gpuos {

// Launches the resident scheduler kernel: `blocks` workgroups of 256 threads
// (4 waves each); wave 0 of block 0 is the doorbell wave, the rest workers.
hipError_t launch_resident(const KArgs& a, uint32_t blocks, hipStream_t s);

// Launches one descriptor as its own kernel (per-op comparator).  `err`
// (device memory, nullable) receives a device error code if a tile fails.
hipError_t launch_single(const DevDesc& d, uint32_t* err, hipStream_t s);

// Launches an empty kernel (one wave) on stream s.
hipError_t launch_empty(hipStream_t s);

// The resident kernel's function handle (for occupancy queries).
const void* resident_kernel();

// Address on `device` of the file-scope device scratch array of
// static_scratch.hip (kStaticScratchBytes), taken once per device with that
// device current (hipGetSymbolAddress); the error of that first call is
// returned on every later one.
hipError_t static_scratch(int device, void** ptr);

}  // namespace gpuos
