// Wave-level helpers for gfx950 (CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gpuos {

__device__ __forceinline__ uint32_t lane_id() {
  return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// Broadcast lane 0's value (the first active lane) to the whole wave.
__device__ __forceinline__ uint32_t bcast(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}
__device__ __forceinline__ uint64_t bcast64(uint64_t v) {
  uint32_t lo = bcast((uint32_t)v);
  uint32_t hi = bcast((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Scoped atomics.  Agent scope orders device memory between waves on any XCD;
// system scope additionally orders against the host (pinned host memory).
template <typename T>
__device__ __forceinline__ T ld_acq_agent(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_rlx_agent(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ void st_rel_agent(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ void st_rlx_agent(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_rlx_sys(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
template <typename T>
__device__ __forceinline__ void st_rel_sys(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}
template <typename T>
__device__ __forceinline__ void st_rlx_sys(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ void fence_rel_agent() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
__device__ __forceinline__ void fence_acq_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }
__device__ __forceinline__ void fence_acq_sys() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, ""); }

__device__ __forceinline__ uint64_t now_ticks() { return __builtin_amdgcn_s_memrealtime(); }

// ---------------------------------------------------------------------------
// bf16 <-> fp32.  bf16 is the upper half of an IEEE binary32 word; narrowing
// rounds to nearest with ties to even and keeps NaN a quiet NaN.

__device__ __forceinline__ float bf2f(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------------------
// Wave reductions (butterfly over all 64 lanes; every lane gets the result).

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ __forceinline__ float nan_max(float a, float b) {
  if (a != a) return a;
  if (b != b) return b;
  return a > b ? a : b;
}

__device__ __forceinline__ float wave_max_nan(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = nan_max(v, __shfl_xor(v, m, 64));
  return v;
}

// Sum over aligned groups of G consecutive lanes (G a power of two <= 64).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int m = G / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ __forceinline__ bool aligned16(uint64_t p) { return (p & 15u) == 0; }

// Global-memory accessors.  Pointers carried in descriptors are plain 64-bit
// addresses; casting them to the global address space gives global_load /
// global_store instructions instead of flat ones.  16-byte accesses use a
// native 4 x u32 vector so values stay in registers.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#define GPUOS_GLOBAL __attribute__((address_space(1)))

template <typename T>
__device__ __forceinline__ T ldg(uint64_t addr) {
  return *reinterpret_cast<const GPUOS_GLOBAL T*>(addr);
}
template <typename T>
__device__ __forceinline__ void stg(uint64_t addr, T v) {
  *reinterpret_cast<GPUOS_GLOBAL T*>(addr) = v;
}

}  // namespace gpuos
