// Opcode switch of the run-time compiled resident kernel variant.
//
// "GPUOS: A GPU Operating System Primitive for Transparent Operation Fusion"
// (section "The Paper") compiles operators at run time and installs them into
// the running persistent kernel.  Here the unit that is compiled and swapped
// is the resident kernel itself: the runtime writes each defined program's
// body as straight-line code (gpuos_rtc_bodies.h, generated per compile),
// builds this variant with hipRTC, and hands the queue from one kernel to the
// other only where the queue has drained.  A descriptor names its compiled
// body in dword 51 (body index + 1; 0 = none).
//
// The variant runs a subset of the op table, chosen so that it compiles in
// seconds: PROGRAM ops with a compiled body, NOP, 4-byte COPY, the fp32
// elementwise ops and fused fp32 chains (plain layouts).  The host sends any
// other descriptor to the built-in kernel.
#pragma once

#include "gpuos_rtc_bodies.h"

namespace gpuos {

// GPUOS_RTC_DTYPES: mask of the dtypes (1 << gpuos_dtype) the bodies are
// compiled for.
template <class Body, int CPL, int CPS>
__device__ __forceinline__ uint32_t rtc_body_tile(uint32_t dt, SDesc d, uint32_t t) {
  Body body;
  if ((GPUOS_RTC_DTYPES >> GPUOS_F32) & 1u) {
    if (dt == GPUOS_F32) {
      prog_each<GPUOS_F32, CPL, CPS>(d, t, body);
      return 0;
    }
  }
  if ((GPUOS_RTC_DTYPES >> GPUOS_BF16) & 1u) {
    if (dt == GPUOS_BF16) {
      prog_each<GPUOS_BF16, CPL, CPS>(d, t, body);
      return 0;
    }
  }
  if ((GPUOS_RTC_DTYPES >> GPUOS_F16) & 1u) {
    if (dt == GPUOS_F16) {
      prog_each<GPUOS_F16, CPL, CPS>(d, t, body);
      return 0;
    }
  }
  return (uint32_t)DERR_BAD_OPCODE;
}

template <int CPL, int CPS>
__device__ __forceinline__ uint32_t exec_rtc_cp(uint32_t op, uint32_t dt, SDesc d, uint32_t t) {
  if (op == GPUOS_OP_PROGRAM) {
    switch (d(51)) {
#define GPUOS_RTC_CASE(K) \
      case K + 1: return rtc_body_tile<RtcBody##K, CPL, CPS>(dt, d, t);
      GPUOS_RTC_BODIES(GPUOS_RTC_CASE)
#undef GPUOS_RTC_CASE
      default: return (uint32_t)DERR_BAD_OPCODE;
    }
  }
  if (op == GPUOS_OP_COPY && (dt == GPUOS_F32 || dt == GPUOS_I32)) {
    copy_tile<4, CPL, CPS>(d, t);
    return 0;
  }
  if (dt != GPUOS_F32) return (uint32_t)DERR_BAD_OPCODE;
  switch (op) {
    case GPUOS_OP_ADD: ew_tile<GPUOS_OP_ADD, GPUOS_F32, CPL, CPS>(d, t); return 0;
    case GPUOS_OP_MUL: ew_tile<GPUOS_OP_MUL, GPUOS_F32, CPL, CPS>(d, t); return 0;
    case GPUOS_OP_RELU: ew_tile<GPUOS_OP_RELU, GPUOS_F32, CPL, CPS>(d, t); return 0;
    case GPUOS_OP_SCALE: ew_tile<GPUOS_OP_SCALE, GPUOS_F32, CPL, CPS>(d, t); return 0;
    case GPUOS_OP_EXP: ew_tile<GPUOS_OP_EXP, GPUOS_F32, CPL, CPS>(d, t); return 0;
    case GPUOS_OP_SILU_MUL: ew_tile<GPUOS_OP_SILU_MUL, GPUOS_F32, CPL, CPS>(d, t); return 0;
    case OP_FUSED_EW: fused_tile<GPUOS_F32, CPL, CPS>(d, t); return 0;
    default: return (uint32_t)DERR_BAD_OPCODE;
  }
}

// Streamed descriptors (GPUOS_FLAG_NONTEMPORAL, set by the runtime on large
// operands) take the non-temporal policies, as in the built-in kernel.
template <int CPL, int CPS>
__device__ __forceinline__ uint32_t exec_rtc(SDesc d, uint32_t t) {
  const uint32_t w0 = d(0);
  const uint32_t op = w0 & 0xffu, dt = (w0 >> 8) & 0xffu, fl = (w0 >> 16) & 0xffu;
  if (fl & DF_VIEW) return (uint32_t)DERR_BAD_OPCODE;
  if (op == GPUOS_OP_NOP) return 0;
  if (fl & GPUOS_FLAG_NONTEMPORAL) return exec_rtc_cp<CPL | CP_NT, CPS | CP_NT>(op, dt, d, t);
  return exec_rtc_cp<CPL, CPS>(op, dt, d, t);
}

}  // namespace gpuos
