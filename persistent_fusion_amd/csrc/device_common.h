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
// Wave reductions with DPP.  Within a row of 16 lanes, four DPP steps
// combine each lane with a partner (quad_perm [1,0,3,2], then [2,3,0,1], then
// row_half_mirror, then row_mirror); every combine pairs lanes symmetrically,
// so all 16 lanes of a row end with the same value.  The four row values are
// then read into scalar registers (v_readlane) and combined as
// (r0 + r1) + (r2 + r3), so the wave-wide result is uniform.  DPP moves data
// between lanes inside the VALU instruction, without the LDS crossbar a
// ds_bpermute shuffle takes.  Every lane of the wave must be active.

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
enum : int {
  DPP_QUAD_1032 = 0xB1,     // quad_perm [1,0,3,2]: lane i <-> i ^ 1
  DPP_QUAD_2301 = 0x4E,     // quad_perm [2,3,0,1]: lane i <-> i ^ 2
  DPP_ROW_HALF_MIRROR = 0x141,  // lane i <-> 7 - i within each 8 lanes
  DPP_ROW_MIRROR = 0x140,   // lane i <-> 15 - i within each 16 lanes
};

__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Sum over aligned groups of G lanes (G a power of two, 2..16): every lane
// receives its group's sum.
template <int G>
__device__ __forceinline__ float row_group_sum(float v) {
  static_assert(G >= 2 && G <= 16 && (G & (G - 1)) == 0, "groups of 2..16 lanes");
  v += dpp_f<DPP_QUAD_1032>(v);
  if constexpr (G >= 4) v += dpp_f<DPP_QUAD_2301>(v);
  if constexpr (G >= 8) v += dpp_f<DPP_ROW_HALF_MIRROR>(v);
  if constexpr (G >= 16) v += dpp_f<DPP_ROW_MIRROR>(v);
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
  v = row_group_sum<16>(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}

__device__ __forceinline__ float nan_max(float a, float b) {
  if (a != a) return a;
  if (b != b) return b;
  return a > b ? a : b;
}

// NaN-propagating maximum over the wave, uniform in every lane.
__device__ __forceinline__ float wave_max_nan(float v) {
  v = nan_max(v, dpp_f<DPP_QUAD_1032>(v));
  v = nan_max(v, dpp_f<DPP_QUAD_2301>(v));
  v = nan_max(v, dpp_f<DPP_ROW_HALF_MIRROR>(v));
  v = nan_max(v, dpp_f<DPP_ROW_MIRROR>(v));
  return nan_max(nan_max(lane_f(v, 0), lane_f(v, 16)), nan_max(lane_f(v, 32), lane_f(v, 48)));
}

// Sum over aligned groups of G consecutive lanes (G a power of two <= 64);
// every lane receives its group's sum.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (G == 1) {
    return v;
  } else if constexpr (G <= 16) {
    return row_group_sum<G>(v);
  } else if constexpr (G == 32) {
    v = row_group_sum<16>(v);
    const float lo = lane_f(v, 0) + lane_f(v, 16), hi = lane_f(v, 32) + lane_f(v, 48);
    return lane_id() < 32 ? lo : hi;
  } else {
    return wave_sum(v);
  }
}

__device__ __forceinline__ bool aligned16(uint64_t p) { return (p & 15u) == 0; }

// Buffer-resource memory access.  Every tile body reads and writes through a
// raw buffer resource (base address in SGPRs, 32-bit byte offset per lane) so
// that the cache policy of each access is explicit:
//   CP_DEFAULT  ordinary loads / stores (kernel boundaries order them);
//   CP_DEVICE   device-scope coherent (`sc1`): loads read the device
//               coherence point, stores write through to it.  The resident
//               kernel uses it for all tensor data, so results become visible
//               to waves on other XCDs once the stores are acknowledged, with
//               no L2 writeback or invalidate in the op path.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

enum : int { CP_DEFAULT = 0, CP_DEVICE = 16, CP_SYSTEM = 17 };

// 0x00020000: raw (untyped) 32-bit data format word of the gfx9 resource.
__device__ __forceinline__ rsrc_t make_rsrc(uint64_t base) {
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(base), 0, -1, 0x00020000);
}
// A resource covering exactly `bytes` bytes (0 for a null pointer): accesses
// at offsets past the end are dropped by the hardware range check (loads
// return zero), so vector loops need no per-lane bounds tests.
__device__ __forceinline__ rsrc_t make_rsrc_n(uint64_t base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(base), 0,
                                           base ? (int)bytes : 0, 0x00020000);
}
// Byte offset of 16-byte vector q, saturated (operand extents are at most
// 0xFFF00000 bytes, checked on the host) so an index past the end stays out of
// range instead of wrapping.
__device__ __forceinline__ uint32_t vec_off(uint32_t q) {
  return q < 0x0FFF0000u ? q * 16u : 0xFFF00000u;
}

template <int CP>
__device__ __forceinline__ u32x4 ld128(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CP);
}
template <int CP>
__device__ __forceinline__ uint32_t ld32(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, CP);
}
template <int CP>
__device__ __forceinline__ uint16_t ld16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, CP);
}
template <int CP>
__device__ __forceinline__ void st128(rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, CP);
}
template <int CP>
__device__ __forceinline__ void st32(rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, CP);
}
template <int CP>
__device__ __forceinline__ void st16(rsrc_t r, uint32_t off, uint16_t v) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, CP);
}

// Waits until every memory access this wave issued has completed (stores
// acknowledged by their scope's coherence point).  The compiler fences keep
// the surrounding memory operations on their side of the wait.
__device__ __forceinline__ void wait_mem() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
__device__ __forceinline__ void compiler_fence() { __atomic_signal_fence(__ATOMIC_SEQ_CST); }

}  // namespace gpuos
