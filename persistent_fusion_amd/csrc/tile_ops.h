// Tile bodies of the op table, shared by the resident kernel and the per-op
// launch comparator.  A body runs on one wave64 and processes one tile of one
// descriptor; `d(i)` returns dword i of the descriptor (uniform), `d.q(i)` the
// 64-bit value at dwords i, i+1.  The descriptor sits in the wave's LDS slot
// and every field read is an LDS load made uniform with readfirstlane, which
// is correct under any set of active lanes (a lane-indexed register copy read
// with readlane is not: inside a divergent region the inactive lanes of a
// reloaded register hold stale values).  CPL / CPS are the cache policies of tensor
// access: CPL for loads, CPS for stores (device-coherent in the resident
// kernel, default in the comparator).
//
// Memory-bound ops stream with 128-bit accesses (4 fp32 or 8 bf16 per lane)
// and keep several loads in flight per lane; reductions sweep a row with the
// whole wave and reduce across lanes.  No op here is a dense contraction
// (batch-1 GEMV moves ~2 bytes per flop), so nothing uses MFMA.  Exact-class
// ops (COPY, GATHER, ADD, MUL, SCALE, RELU, ROPE) are single IEEE operations
// per element; the library is compiled with contraction off so a*b+c is never
// fused into an FMA.  Tensor byte offsets fit in 32 bits (checked on the
// host).
#pragma once

#include "device_common.h"
#include "gpuos_internal.h"
#include "../../include/gpuos.h"

namespace gpuos {

typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) float lds_f32;

// The 64 dwords of a descriptor in LDS.
struct SDesc {
  const lds_u32* p;
  __device__ __forceinline__ uint32_t operator()(int i) const {
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)p[i]);
  }
  __device__ __forceinline__ uint64_t q(int i) const {
    return (uint64_t)(*this)(i) | ((uint64_t)(*this)(i + 1) << 32);
  }
};

// ---------------------------------------------------------------------------
// element types

template <int DT, int CPL, int CPS>
struct DTr;

template <int CPL, int CPS>
struct DTr<GPUOS_F32, CPL, CPS> {
  static constexpr int V = 4;   // elements per 16-byte access
  static constexpr int ES = 4;  // bytes per element
  __device__ static __forceinline__ float ld(rsrc_t r, uint32_t i) {
    return __uint_as_float(ld32<CPL>(r, 4u * i));
  }
  __device__ static __forceinline__ void st(rsrc_t r, uint32_t i, float v) {
    st32<CPS>(r, 4u * i, __float_as_uint(v));
  }
  __device__ static __forceinline__ void ldv(rsrc_t r, uint32_t i, float (&x)[4]) {
    const u32x4 t = ld128<CPL>(r, 4u * i);
    x[0] = __uint_as_float(t.x); x[1] = __uint_as_float(t.y);
    x[2] = __uint_as_float(t.z); x[3] = __uint_as_float(t.w);
  }
  __device__ static __forceinline__ void stv(rsrc_t r, uint32_t i, const float (&x)[4]) {
    u32x4 t;
    t.x = __float_as_uint(x[0]); t.y = __float_as_uint(x[1]);
    t.z = __float_as_uint(x[2]); t.w = __float_as_uint(x[3]);
    st128<CPS>(r, 4u * i, t);
  }
  // 16-byte vector q (elements 4q .. 4q + 3)
  __device__ static __forceinline__ void ldq(rsrc_t r, uint32_t q, float (&x)[4]) {
    const u32x4 t = ld128<CPL>(r, vec_off(q));
    x[0] = __uint_as_float(t.x); x[1] = __uint_as_float(t.y);
    x[2] = __uint_as_float(t.z); x[3] = __uint_as_float(t.w);
  }
  __device__ static __forceinline__ void stq(rsrc_t r, uint32_t q, const float (&x)[4]) {
    u32x4 t;
    t.x = __float_as_uint(x[0]); t.y = __float_as_uint(x[1]);
    t.z = __float_as_uint(x[2]); t.w = __float_as_uint(x[3]);
    st128<CPS>(r, vec_off(q), t);
  }
  __device__ static __forceinline__ float round(float v) { return v; }
};

__device__ __forceinline__ void unpack_bf16x8(const u32x4& t, float (&w)[8]) {
  w[0] = bf2f(t.x & 0xffffu); w[1] = bf2f(t.x >> 16);
  w[2] = bf2f(t.y & 0xffffu); w[3] = bf2f(t.y >> 16);
  w[4] = bf2f(t.z & 0xffffu); w[5] = bf2f(t.z >> 16);
  w[6] = bf2f(t.w & 0xffffu); w[7] = bf2f(t.w >> 16);
}

template <int CPL, int CPS>
struct DTr<GPUOS_BF16, CPL, CPS> {
  static constexpr int V = 8;
  static constexpr int ES = 2;
  __device__ static __forceinline__ float ld(rsrc_t r, uint32_t i) {
    return bf2f(ld16<CPL>(r, 2u * i));
  }
  __device__ static __forceinline__ void st(rsrc_t r, uint32_t i, float v) {
    st16<CPS>(r, 2u * i, (uint16_t)f2bf(v));
  }
  __device__ static __forceinline__ void ldv(rsrc_t r, uint32_t i, float (&x)[8]) {
    unpack_bf16x8(ld128<CPL>(r, 2u * i), x);
  }
  __device__ static __forceinline__ void stv(rsrc_t r, uint32_t i, const float (&x)[8]) {
    u32x4 t;
    t.x = f2bf(x[0]) | (f2bf(x[1]) << 16);
    t.y = f2bf(x[2]) | (f2bf(x[3]) << 16);
    t.z = f2bf(x[4]) | (f2bf(x[5]) << 16);
    t.w = f2bf(x[6]) | (f2bf(x[7]) << 16);
    st128<CPS>(r, 2u * i, t);
  }
  // 16-byte vector q (elements 8q .. 8q + 7)
  __device__ static __forceinline__ void ldq(rsrc_t r, uint32_t q, float (&x)[8]) {
    unpack_bf16x8(ld128<CPL>(r, vec_off(q)), x);
  }
  __device__ static __forceinline__ void stq(rsrc_t r, uint32_t q, const float (&x)[8]) {
    u32x4 t;
    t.x = f2bf(x[0]) | (f2bf(x[1]) << 16);
    t.y = f2bf(x[2]) | (f2bf(x[3]) << 16);
    t.z = f2bf(x[4]) | (f2bf(x[5]) << 16);
    t.w = f2bf(x[6]) | (f2bf(x[7]) << 16);
    st128<CPS>(r, vec_off(q), t);
  }
  // value after a round trip through bf16 storage
  __device__ static __forceinline__ float round(float v) { return bf2f(f2bf(v)); }
};

// fp16: widened exactly to fp32, narrowed with the hardware conversion
// (round to nearest even, NaN stays NaN, subnormals kept).  Both directions
// are kept opaque to the compiler's floating-point combines: it folds
// "multiply in fp32, narrow to fp16" into a mixed-precision FMA with a +0
// addend, which turns a -0 product into +0.  The widening is written out on
// the bits; the narrowing is the conversion instruction itself.
__device__ __forceinline__ float h2f(uint32_t b) {
  const uint32_t sign = (b & 0x8000u) << 16, e = (b >> 10) & 0x1fu, m = b & 0x3ffu;
  const uint32_t p = 31u - (uint32_t)__builtin_clz(m | 1u);  // leading bit of a subnormal
  const uint32_t sub = ((p + 103u) << 23) | ((m << (23u - p)) & 0x7fffffu);
  uint32_t bits = ((e + 112u) << 23) | (m << 13);  // normal
  bits = e == 0x1fu ? 0x7f800000u | (m << 13) : bits;  // inf, NaN
  bits = e == 0u ? (m ? sub : 0u) : bits;             // zero, subnormal
  return __uint_as_float(sign | bits);
}
__device__ __forceinline__ uint32_t f2h(float v) {
  uint32_t r;
  asm("v_cvt_f16_f32 %0, %1" : "=v"(r) : "v"(v));
  return r & 0xffffu;
}
__device__ __forceinline__ void unpack_f16x8(const u32x4& t, float (&w)[8]) {
  w[0] = h2f(t.x & 0xffffu); w[1] = h2f(t.x >> 16);
  w[2] = h2f(t.y & 0xffffu); w[3] = h2f(t.y >> 16);
  w[4] = h2f(t.z & 0xffffu); w[5] = h2f(t.z >> 16);
  w[6] = h2f(t.w & 0xffffu); w[7] = h2f(t.w >> 16);
}
__device__ __forceinline__ u32x4 pack_f16x8(const float (&x)[8]) {
  u32x4 t;
  t.x = f2h(x[0]) | (f2h(x[1]) << 16);
  t.y = f2h(x[2]) | (f2h(x[3]) << 16);
  t.z = f2h(x[4]) | (f2h(x[5]) << 16);
  t.w = f2h(x[6]) | (f2h(x[7]) << 16);
  return t;
}

template <int CPL, int CPS>
struct DTr<GPUOS_F16, CPL, CPS> {
  static constexpr int V = 8;
  static constexpr int ES = 2;
  __device__ static __forceinline__ float ld(rsrc_t r, uint32_t i) { return h2f(ld16<CPL>(r, 2u * i)); }
  __device__ static __forceinline__ void st(rsrc_t r, uint32_t i, float v) {
    st16<CPS>(r, 2u * i, (uint16_t)f2h(v));
  }
  __device__ static __forceinline__ void ldv(rsrc_t r, uint32_t i, float (&x)[8]) {
    unpack_f16x8(ld128<CPL>(r, 2u * i), x);
  }
  __device__ static __forceinline__ void stv(rsrc_t r, uint32_t i, const float (&x)[8]) {
    st128<CPS>(r, 2u * i, pack_f16x8(x));
  }
  __device__ static __forceinline__ void ldq(rsrc_t r, uint32_t q, float (&x)[8]) {
    unpack_f16x8(ld128<CPL>(r, vec_off(q)), x);
  }
  __device__ static __forceinline__ void stq(rsrc_t r, uint32_t q, const float (&x)[8]) {
    st128<CPS>(r, vec_off(q), pack_f16x8(x));
  }
  __device__ static __forceinline__ float round(float v) { return h2f(f2h(v)); }
};

// int32: the same 4-byte moves as fp32; values travel as bit patterns in
// float registers and only ew_apply<OP, GPUOS_I32> interprets them.
template <int CPL, int CPS>
struct DTr<GPUOS_I32, CPL, CPS> : DTr<GPUOS_F32, CPL, CPS> {};

// ---------------------------------------------------------------------------
// elementwise semantics (one IEEE operation each; see gpuos.h)

template <int OP, int DT = GPUOS_F32>
__device__ __forceinline__ float ew_apply(float x, float y, float alpha) {
  if constexpr (DT == GPUOS_I32) {  // two's-complement, wrapping
    const uint32_t a = __float_as_uint(x), b = __float_as_uint(y);
    if constexpr (OP == GPUOS_OP_ADD) return __uint_as_float(a + b);
    else if constexpr (OP == GPUOS_OP_MUL) return __uint_as_float(a * b);
    else return __uint_as_float((int32_t)a > 0 ? a : 0u);  // RELU
  }
  else if constexpr (OP == GPUOS_OP_COPY) return x;
  else if constexpr (OP == GPUOS_OP_ADD) return x + y;
  else if constexpr (OP == GPUOS_OP_MUL) return x * y;
  else if constexpr (OP == GPUOS_OP_SCALE) return alpha * x;
  else if constexpr (OP == GPUOS_OP_RELU) return x > 0.0f ? x : 0.0f;
  else if constexpr (OP == GPUOS_OP_EXP) return expf(x);
  else {  // SILU_MUL
    const float den = 1.0f + expf(-x);
    return x / den * y;
  }
}

template <int OP>
constexpr bool ew_binary() {
  return OP == GPUOS_OP_ADD || OP == GPUOS_OP_MUL || OP == GPUOS_OP_SILU_MUL;
}

// Elementwise tiles are interleaved: the op's whole 16-byte vectors form
// rows of 64 (one per lane), U adjacent rows form a group, and tile t of T
// takes groups t, t + T, t + 2T, ...  At any moment the waves of a large op
// sweep adjacent memory together (like a grid-stride loop), and each wave's
// U rows in flight are one contiguous U KiB (fp32) block per operand, which
// keeps fewer DRAM pages open than U rows spread T rows apart.  The n % V
// leftover elements belong to the last tile.  A source read cyclically, or
// a misaligned operand, uses the per-element path interleaved by lanes.
template <int OP, int DT, int CPL, int CPS, class D>
__device__ __forceinline__ void ew_tile(D d, uint32_t t) {
  using T = DTr<DT, CPL, CPS>;
  constexpr int V = T::V;
  constexpr bool BIN = ew_binary<OP>();
  constexpr int U = DT == GPUOS_F32 ? 4 : 2;
  const uint32_t n = d(1), ntiles = d(6);
  const rsrc_t out = make_rsrc(d.q(18)), a = make_rsrc(d.q(20)), b = make_rsrc(d.q(22));
  const uint32_t ca = d(26), cb = d(27);
  const float alpha = __uint_as_float(d(28));
  const uint32_t lane = lane_id();
  const bool fast = ca == 0 && (!BIN || cb == 0) && aligned16(d.q(18)) && aligned16(d.q(20)) &&
                    (!BIN || aligned16(d.q(22)));
  if (fast) {
    // whole vectors only; rows past the end fall outside the resources
    const uint32_t nv = n / V, nrows = (nv + 63) / 64;
    const rsrc_t vo = make_rsrc_n(d.q(18), nv * 16u), va = make_rsrc_n(d.q(20), nv * 16u);
    const rsrc_t vb = make_rsrc_n(BIN ? d.q(22) : 0, nv * 16u);
    const uint32_t ngroups = (nrows + U - 1) / U;
    float x[U][V], y[U][V];
    auto load = [&](uint32_t g) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t q = (g * U + u) * 64 + lane;
        T::ldq(va, q, x[u]);
        if constexpr (BIN) T::ldq(vb, q, y[u]);
      }
    };
    // software pipeline: group g + T is requested before group g is computed
    if (t < ngroups) load(t);
    for (uint32_t g = t; g < ngroups; g += ntiles) {
      float cx[U][V], cy[U][V];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < V; ++e) {
          cx[u][e] = x[u][e];
          cy[u][e] = BIN ? y[u][e] : 0.0f;
        }
      if (g + ntiles < ngroups) load(g + ntiles);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t q = (g * U + u) * 64 + lane;
        float r[V];
#pragma unroll
        for (int e = 0; e < V; ++e) r[e] = ew_apply<OP, DT>(cx[u][e], cy[u][e], alpha);
        T::stq(vo, q, r);
      }
    }
    if (t + 1 == ntiles) {
      for (uint32_t i = nv * V + lane; i < n; i += 64) {
        const float y = BIN ? T::ld(b, i) : 0.0f;
        T::st(out, i, ew_apply<OP, DT>(T::ld(a, i), y, alpha));
      }
    }
    return;
  }
  for (uint32_t i = t * 64 + lane; i < n; i += 64 * ntiles) {
    const float x = T::ld(a, ca ? i % ca : i);
    const float y = BIN ? T::ld(b, cb ? i % cb : i) : 0.0f;
    T::st(out, i, ew_apply<OP, DT>(x, y, alpha));
  }
}

// ---------------------------------------------------------------------------
// PROGRAM ops: a register program defined at run time (gpuos_program in
// gpuos.h), carried by value in the descriptor (dword 26: n_insns | result
// << 8 | n_inputs << 16 | zero-init mask << 24; dwords 27-42: instructions
// op | dst << 5 | a << 8 | b << 12 | c << 16; dwords 43-50: constants).  The
// program is uniform across the wave, so each instruction is a few scalar
// branches and one 4-wide vector operation per lane.  Registers r0..r7 are
// eight separate vector values (never an indexed array, which the compiler
// would have to place in scratch memory); r8..r15 are uniform constants.

typedef float pvec __attribute__((ext_vector_type(4)));

struct PRegs {
  pvec r0, r1, r2, r3, r4, r5, r6, r7;
};

// IEEE 754-2019 minimum / maximum: NaN if either operand is NaN, -0 < +0.
__device__ __forceinline__ float prog_min(float a, float b) {
  if (a != a || b != b) return a + b;
  if (a < b) return a;
  if (b < a) return b;
  return __uint_as_float(__float_as_uint(a) | __float_as_uint(b));  // equal: -0 wins
}
__device__ __forceinline__ float prog_max(float a, float b) {
  if (a != a || b != b) return a + b;
  if (a > b) return a;
  if (b > a) return b;
  return __uint_as_float(__float_as_uint(a) & __float_as_uint(b));  // equal: +0 wins
}

// Source register i: r0..r7, or constant i - 8 (lane 16 + (i - 8) of pw).
__device__ __forceinline__ pvec prog_src(uint32_t pw, const PRegs& R, uint32_t i) {
  switch (i) {
    case 0: return R.r0;
    case 1: return R.r1;
    case 2: return R.r2;
    case 3: return R.r3;
    case 4: return R.r4;
    case 5: return R.r5;
    case 6: return R.r6;
    case 7: return R.r7;
    default: return pvec(__uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)pw, 16 + (int)(i & 7u))));
  }
}

__device__ __forceinline__ void prog_dst(PRegs& R, uint32_t i, pvec y) {
  switch (i) {
    case 0: R.r0 = y; break;
    case 1: R.r1 = y; break;
    case 2: R.r2 = y; break;
    case 3: R.r3 = y; break;
    case 4: R.r4 = y; break;
    case 5: R.r5 = y; break;
    case 6: R.r6 = y; break;
    default: R.r7 = y; break;
  }
}

// The instructions' per-element operations on 4-element vectors; the
// interpreter and compiled program bodies both use them.
__device__ __forceinline__ pvec pv_min(pvec a, pvec b) {
  pvec y;
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = prog_min(a[e], b[e]);
  return y;
}
__device__ __forceinline__ pvec pv_max(pvec a, pvec b) {
  pvec y;
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = prog_max(a[e], b[e]);
  return y;
}
__device__ __forceinline__ pvec pv_neg(pvec a) {
  pvec y;
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = __uint_as_float(__float_as_uint(a[e]) ^ 0x80000000u);
  return y;
}
__device__ __forceinline__ pvec pv_abs(pvec a) {
  pvec y;
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = __uint_as_float(__float_as_uint(a[e]) & 0x7fffffffu);
  return y;
}
__device__ __forceinline__ pvec pv_relu(pvec a) {
  pvec y;
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = a[e] > 0.0f ? a[e] : 0.0f;
  return y;
}
__device__ __forceinline__ pvec pv_exp(pvec a) {
  pvec y;
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = expf(a[e]);
  return y;
}
__device__ __forceinline__ pvec pv_lt(pvec a, pvec b) {
  pvec y;
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = a[e] < b[e] ? 1.0f : 0.0f;
  return y;
}
__device__ __forceinline__ pvec pv_sel(pvec a, pvec b, pvec c) {
  pvec y;
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = a[e] != 0.0f ? b[e] : c[e];
  return y;
}

// Instructions that read b (binary ops and LT) and c (SEL).
constexpr uint32_t kPReadsB = (1u << GPUOS_P_ADD) | (1u << GPUOS_P_SUB) | (1u << GPUOS_P_MUL) |
                              (1u << GPUOS_P_DIV) | (1u << GPUOS_P_MIN) | (1u << GPUOS_P_MAX) |
                              (1u << GPUOS_P_LT) | (1u << GPUOS_P_SEL);

// Runs the program on R and returns the result register.  pw holds the
// program in lanes: lane s < 16 instruction s, lane 16 + j constant j (read
// with readlane: it was loaded while every lane was active).
__device__ __forceinline__ pvec prog_run(uint32_t pw, uint32_t meta, PRegs& R) {
  const uint32_t ni = meta & 31u;
  for (uint32_t s = 0; s < ni; ++s) {
    const uint32_t w = (uint32_t)__builtin_amdgcn_readlane((int)pw, (int)s);
    const uint32_t op = w & 31u;
    const pvec a = prog_src(pw, R, (w >> 8) & 15u);
    pvec b = a, c = a, y;
    if ((kPReadsB >> op) & 1u) b = prog_src(pw, R, (w >> 12) & 15u);
    if (op == GPUOS_P_SEL) c = prog_src(pw, R, (w >> 16) & 15u);
    switch (op) {
      case GPUOS_P_ADD: y = a + b; break;
      case GPUOS_P_SUB: y = a - b; break;
      case GPUOS_P_MUL: y = a * b; break;
      case GPUOS_P_DIV: y = a / b; break;
      case GPUOS_P_MIN: y = pv_min(a, b); break;
      case GPUOS_P_MAX: y = pv_max(a, b); break;
      case GPUOS_P_NEG: y = pv_neg(a); break;
      case GPUOS_P_ABS: y = pv_abs(a); break;
      case GPUOS_P_RELU: y = pv_relu(a); break;
      case GPUOS_P_EXP: y = pv_exp(a); break;
      case GPUOS_P_LT: y = pv_lt(a, b); break;
      case GPUOS_P_SEL: y = pv_sel(a, b, c); break;
      default: y = a; break;  // MOV
    }
    prog_dst(R, (w >> 5) & 7u, y);
  }
  return prog_src(pw, R, (meta >> 8) & 15u);
}

// A pass's registers: the inputs in r0..r(nin-1), then +0 in every register
// the program reads before writing (mask in meta bits 24-31; never an input
// register).  The others keep the previous pass's values, which the program
// overwrites before reading.
__device__ __forceinline__ void prog_init(PRegs& R, uint32_t nin, uint32_t zmask, pvec x0, pvec x1,
                                          pvec x2) {
  const pvec z = pvec(0.0f);
  R.r0 = x0;
  if (nin >= 2) R.r1 = x1; else if (zmask & 2u) R.r1 = z;
  if (nin >= 3) R.r2 = x2; else if (zmask & 4u) R.r2 = z;
  if (zmask & 8u) R.r3 = z;
  if (zmask & 16u) R.r4 = z;
  if (zmask & 32u) R.r5 = z;
  if (zmask & 64u) R.r6 = z;
  if (zmask & 128u) R.r7 = z;
}

// Tiles as ew_tile: whole 16-byte vectors form rows of 64 (one per lane), U
// adjacent rows a group of 8 elements per lane (2 rows of fp32, 1 of 16-bit
// types), tile t takes groups t, t + T, ...  The program runs on 4 elements
// at a time; as soon as a pass has copied the last of a row's inputs into
// its registers, the same row of the tile's next group is requested, so
// about a group's 3U vectors per lane stay in flight.  The copies complete
// before that request (a copy the compiler sank into the program's register
// switch would wait for the newer loads too: the vector-memory counter is in
// order), and the loads are unconditional, past the end they fall outside
// the bounded resources and return 0, which keeps the counter's waits exact.
// The n % V leftover elements belong to the last tile; misaligned operands
// use per-element accesses.
// `body(x0, x1, x2)` computes 4 elements' results from their inputs (inputs
// past n_inputs are +0): the interpreter below, or a compiled program body.
template <int DT, int CPL, int CPS, class Body>
__device__ __forceinline__ void prog_each(SDesc d, uint32_t t, Body& body) {
  using T = DTr<DT, CPL, CPS>;
  constexpr int V = T::V;
  constexpr int G = 8;      // elements per lane per group
  constexpr int U = G / V;  // rows per group
  constexpr int P = G / 4;  // program passes per group (4 elements each)
  const uint32_t n = d(1), ntiles = d(6), meta = d(26);
  const uint32_t nin = (meta >> 16) & 3u;
  const uint64_t po = d.q(18), p0 = d.q(20), p1 = nin >= 2 ? d.q(22) : 0, p2 = nin >= 3 ? d.q(24) : 0;
  const uint32_t lane = lane_id();
  const bool fast = aligned16(po) && aligned16(p0) && aligned16(p1) && aligned16(p2);
  if (fast) {
    const uint32_t nv = n / V, nrows = (nv + 63) / 64, ngroups = (nrows + U - 1) / U;
    const rsrc_t vo = make_rsrc_n(po, nv * 16u), v0 = make_rsrc_n(p0, nv * 16u),
                 v1 = make_rsrc_n(p1, nv * 16u), v2 = make_rsrc_n(p2, nv * 16u);
    float x0[U][V], x1[U][V], x2[U][V];
    auto load_row = [&](uint32_t g, int u) {
      // past the end: clamped to a vector out of every range (loads give 0)
      const uint64_t q64 = ((uint64_t)g * U + u) * 64 + lane;
      const uint32_t q = q64 < 0x0FFF0000u ? (uint32_t)q64 : 0x0FFF0000u;
      T::ldq(v0, q, x0[u]);
      T::ldq(v1, q, x1[u]);
      T::ldq(v2, q, x2[u]);
    };
    if (t < ngroups) {
#pragma unroll
      for (int u = 0; u < U; ++u) load_row(t, u);
    }
    for (uint32_t g = t; g < ngroups; g += ntiles) {
      float w[G];
#pragma unroll
      for (int k = 0; k < P; ++k) {
        const int u = 4 * k / V, e0 = 4 * k % V;  // row and first element of pass k
        pvec a0, a1, a2;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a0[e] = x0[u][e0 + e];
          a1[e] = x1[u][e0 + e];
          a2[e] = x2[u][e0 + e];
        }
        asm volatile("" : "+v"(a0), "+v"(a1), "+v"(a2));
        if (e0 + 4 == V) load_row(g + ntiles, u);  // row u fully taken
        const pvec o = body(a0, a1, a2);
#pragma unroll
        for (int e = 0; e < 4; ++e) w[4 * k + e] = o[e];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float wr[V];
#pragma unroll
        for (int e = 0; e < V; ++e) wr[e] = w[u * V + e];
        T::stq(vo, (g * U + u) * 64 + lane, wr);
      }
    }
    if (t + 1 == ntiles && nv * V < n) {  // fewer than V leftover elements
      const uint32_t nb = n * (uint32_t)T::ES;  // bounded: lanes past n read 0
      const rsrc_t so = make_rsrc_n(po, nb), s0 = make_rsrc_n(p0, nb), s1 = make_rsrc_n(p1, nb),
                   s2 = make_rsrc_n(p2, nb);
      const uint32_t i = nv * V + lane;
      pvec y0 = pvec(0.0f), y1 = pvec(0.0f), y2 = pvec(0.0f);
      y0[0] = T::ld(s0, i);
      if (nin >= 2) y1[0] = T::ld(s1, i);
      if (nin >= 3) y2[0] = T::ld(s2, i);
      const pvec o = body(y0, y1, y2);
      if (i < n) T::st(so, i, o[0]);
    }
    return;
  }
  const uint32_t nb = n * (uint32_t)T::ES;  // bounded: lanes past n read 0
  const rsrc_t so = make_rsrc_n(po, nb), s0 = make_rsrc_n(p0, nb), s1 = make_rsrc_n(p1, nb),
               s2 = make_rsrc_n(p2, nb);
  for (uint64_t base = (uint64_t)t * 256u; base < n; base += (uint64_t)256u * ntiles) {
    pvec y0, y1 = pvec(0.0f), y2 = pvec(0.0f);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t i = (uint32_t)base + (uint32_t)e * 64 + lane;
      y0[e] = T::ld(s0, i);
      if (nin >= 2) y1[e] = T::ld(s1, i);
      if (nin >= 3) y2[e] = T::ld(s2, i);
    }
    const pvec o = body(y0, y1, y2);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t i = (uint32_t)base + (uint32_t)e * 64 + lane;
      if (i < n) T::st(so, i, o[e]);
    }
  }
}

// A PROGRAM op interpreted: the program rides in the descriptor.
template <int DT, int CPL, int CPS>
__device__ __forceinline__ void prog_tile(SDesc d, uint32_t t) {
  const uint32_t meta = d(26);
  const uint32_t nin = (meta >> 16) & 3u, zmask = meta >> 24;
  // instructions (dwords 27-42) in lanes 0-15, constants (43-50) in lanes 16-23
  const uint32_t pw = d.p[27 + (lane_id() & 31u)];
  PRegs R;
  R.r0 = R.r1 = R.r2 = R.r3 = R.r4 = R.r5 = R.r6 = R.r7 = pvec(0.0f);
  auto run = [&](pvec x0, pvec x1, pvec x2) {
    prog_init(R, nin, zmask, x0, x1, x2);
    return prog_run(pw, meta, R);
  };
  prog_each<DT, CPL, CPS>(d, t, run);
}

// COPY over a transposed view (DF_VIEW_T): out[b][r][c] = in[b][c * si + r]
// for batches b < shape[1] (strides d(39), d(43)), rows r < R and columns
// c < L, the output's rows contiguous with row stride so.  Tile t is a block of K = 128 / ES rows (one 128-byte line of each input
// column) by 128 columns.  A lane holds P = 4 / ES adjacent columns per step
// (one for fp32, two for 16-bit types), two steps for fp32: it reads each of
// its columns' K elements with eight 16-byte loads (all issued before the
// first store, line by line so the first rows arrive first) and then writes
// row by row 4-byte words, so each store instruction writes 256 consecutive
// output bytes.  Bottom-edge blocks, misaligned input columns and 16-bit
// outputs whose pairs are not 4-byte aligned move element by element.
template <int ES, int CPL, int CPS>
__device__ __forceinline__ void copy_transposed_tile(SDesc d, uint32_t t) {
  constexpr uint32_t K = kTBlockBytes / ES, P = 4 / ES, CS = 2 / P;
  constexpr uint32_t W = kTBlockBytes / 16;  // 16-byte loads per column
  const uint32_t R = d(36), L = d(37);
  const uint32_t so = d(38 + 2), si = d(42 + 3);
  const uint32_t ncb = (L + kTCols - 1) / kTCols, nb = ((R + K - 1) / K) * ncb;
  // batch and block within it; the tile index is the same in every lane, and
  // saying so keeps the batch's base addresses (buffer resources) scalar
  uint32_t tb = t;
  uint64_t pout = d.q(18), pin = d.q(20);
  if (d(35) > 1) {
    const uint32_t tu = __builtin_amdgcn_readfirstlane(t), bi = tu / nb;
    tb = tu - bi * nb;
    pout += (uint64_t)ES * bi * d(38 + 1);
    pin += (uint64_t)ES * bi * d(42 + 1);
  }
  const uint32_t r0 = (tb / ncb) * K, c0 = (tb % ncb) * kTCols;
  const rsrc_t out = make_rsrc(pout), in = make_rsrc(pin);
  const uint32_t lane = lane_id();
  const bool vec = r0 + K <= R && aligned16(pin) && (si * ES) % 16u == 0 &&
                   (ES == 4 || ((pout & 3u) == 0 && so % 2u == 0));
  if (vec) {
    u32x4 w[CS][P][W];
#pragma unroll
    for (uint32_t v = 0; v < W; ++v)
#pragma unroll
      for (uint32_t k = 0; k < CS; ++k)
#pragma unroll
        for (uint32_t j = 0; j < P; ++j) {
          // columns past the edge read the last column (stores skip them)
          const uint32_t c = min(c0 + 64 * P * k + P * lane + j, L - 1);
          w[k][j][v] = ld128<CPL>(in, ES * (c * si + r0) + 16u * v);
        }
    auto word = [&](uint32_t k, uint32_t j, uint32_t m) {  // the dword holding element m
      const uint32_t q = (m * ES) / 4, v = q / 4, e = q % 4;
      const u32x4 x = w[k][j][v];
      return e == 0 ? x.x : e == 1 ? x.y : e == 2 ? x.z : x.w;
    };
#pragma unroll
    for (uint32_t m = 0; m < K; ++m)
#pragma unroll
      for (uint32_t k = 0; k < CS; ++k) {
        const uint32_t c = c0 + 64 * P * k + P * lane;
        const uint32_t o = ES * ((r0 + m) * so + c);
        if constexpr (ES == 4) {
          if (c < L) st32<CPS>(out, o, word(k, 0, m));
        } else {
          const uint32_t sh = 16 * (m % 2);
          const uint32_t lo = (word(k, 0, m) >> sh) & 0xffffu, hi = (word(k, 1, m) >> sh) & 0xffffu;
          if (c + 1 < L) st32<CPS>(out, o, lo | (hi << 16));
          else if (c < L) st16<CPS>(out, o, (uint16_t)lo);
        }
      }
    return;
  }
  for (uint32_t k = 0; k < CS; ++k)
    for (uint32_t j = 0; j < P; ++j) {
      const uint32_t c = c0 + 64 * P * k + P * lane + j;
      if (c >= L) continue;
      for (uint32_t m = 0; m < K && r0 + m < R; ++m) {
        const uint32_t e = c * si + r0 + m, o = ES * ((r0 + m) * so + c);
        if constexpr (ES == 2) st16<CPS>(out, o, ld16<CPL>(in, 2u * e));
        else st32<CPS>(out, o, ld32<CPL>(in, 4u * e));
      }
    }
}

// Elementwise op over a strided or broadcast view (DF_VIEW).  The index space
// is `rows` = shape[0] x shape[1] x shape[2] rows of shape[3] elements; tile t
// takes `tile` rows from row t * tile, and the lanes split each row, four
// elements per lane in flight.  Each operand's element offset is the dot
// product of the index with its strides (an exact in-place op reads and
// writes each element in the same lane).  COPY moves bits.
template <int OP, int DT, int CPL, int CPS, class D>
__device__ __forceinline__ void ew_view_tile(D d, uint32_t t) {
  using T = DTr<DT, CPL, CPS>;
  constexpr bool BIN = ew_binary<OP>();
  constexpr int U = 4;
  const uint32_t s1 = d(35), s2 = d(36), L = d(37);
  const uint32_t rows = d(34) * s1 * s2, tile = d(7);
  uint32_t st[3][4];
#pragma unroll
  for (int k = 0; k < 3; ++k)
#pragma unroll
    for (int j = 0; j < 4; ++j) st[k][j] = d(38 + 4 * k + j);
  const rsrc_t out = make_rsrc(d.q(18)), a = make_rsrc(d.q(20)), b = make_rsrc(d.q(22));
  const float alpha = __uint_as_float(d(28));
  const uint32_t r0 = t * tile;
  const uint32_t r1 = r0 + tile < rows ? r0 + tile : rows;
  const uint32_t lane = lane_id();
  // Rows that are contiguous in the output and contiguous or broadcast (one
  // value per row) in every input, with 16-byte aligned row starts, move
  // 16-byte vectors: V elements per lane per access, UV vectors per chunk,
  // the next chunk in flight while one is computed.
  constexpr int V = T::V;
  constexpr int UV = DT == GPUOS_F32 || DT == GPUOS_I32 ? 4 : 2;
  // An operand read as vectors (inner stride 1) needs 16-byte aligned row
  // starts; a broadcast one (inner stride 0) is read one element per row.
  // COPY moves raw 16-byte words, so its input must be contiguous too.
  bool vec = st[0][3] == 1 && st[1][3] <= 1 && (OP != GPUOS_OP_COPY || st[1][3] == 1) &&
             (!BIN || st[2][3] <= 1) && L % V == 0;
  const uint64_t ptr[3] = {d.q(18), d.q(20), d.q(22)};
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    if (k == 2 && !BIN) continue;
    if (st[k][3] != 1) continue;
    vec = vec && aligned16(ptr[k]);
#pragma unroll
    for (int j = 0; j < 3; ++j) vec = vec && (st[k][j] * (uint32_t)T::ES) % 16u == 0;
  }
  if (vec) {
    // the tile's rows cut into chunks of 64 x UV vectors, one flat sequence;
    // after chunk c's stores, chunk c + 1's inputs are copied out (behind an
    // asm barrier) and chunk c + 2 is requested, so the copies wait for loads
    // only and a chunk is in flight while one is computed
    const uint32_t nv = L / V, cpr = (nv + 64 * UV - 1) / (64 * UV), nchunks = (r1 - r0) * cpr;
    auto row_base = [&](uint32_t c, int k) {
      const uint32_t r = r0 + c / cpr;
      const uint32_t i2 = r % s2, q = r / s2;
      const uint32_t i1 = q % s1, i0 = q / s1;
      return i0 * st[k][0] + i1 * st[k][1] + i2 * st[k][2];
    };
    if constexpr (OP == GPUOS_OP_COPY) {  // bits, 16 bytes at a time
      u32x4 w[UV];
      auto load = [&](uint32_t c) {
        const uint32_t ba = row_base(c, 1), q0 = (c % cpr) * 64 * UV;
#pragma unroll
        for (int u = 0; u < UV; ++u) {
          const uint32_t qv = q0 + 64 * u + lane;
          if (qv < nv) w[u] = ld128<CPL>(a, T::ES * (ba + qv * V));
        }
      };
      u32x4 cw[UV];
      auto take_then_load = [&](uint32_t next) {
#pragma unroll
        for (int u = 0; u < UV; ++u) {
          cw[u] = w[u];
          asm volatile("" : "+v"(cw[u]));
        }
        if (next < nchunks) load(next);
      };
      if (nchunks) {
        load(0);
        take_then_load(1);
      }
      for (uint32_t c = 0; c < nchunks; ++c) {
        const uint32_t bo = row_base(c, 0), q0 = (c % cpr) * 64 * UV;
#pragma unroll
        for (int u = 0; u < UV; ++u) {
          const uint32_t qv = q0 + 64 * u + lane;
          if (qv < nv) st128<CPS>(out, T::ES * (bo + qv * V), cw[u]);
        }
        if (c + 1 < nchunks) take_then_load(c + 2);
      }
    } else {
      float x[UV][V], y[UV][V];
      auto load = [&](uint32_t c) {
        const uint32_t ba = row_base(c, 1), bb = row_base(c, 2), q0 = (c % cpr) * 64 * UV;
        // a broadcast input (inner stride 0) has one value per row
        const float xa = st[1][3] == 0 ? T::ld(a, ba) : 0.0f;
        const float yb = BIN && st[2][3] == 0 ? T::ld(b, bb) : 0.0f;
#pragma unroll
        for (int u = 0; u < UV; ++u) {
          const uint32_t qv = q0 + 64 * u + lane;
#pragma unroll
          for (int e = 0; e < V; ++e) x[u][e] = xa, y[u][e] = yb;
          if (qv >= nv) continue;
          if (st[1][3]) T::ldv(a, ba + qv * V, x[u]);
          if (BIN && st[2][3]) T::ldv(b, bb + qv * V, y[u]);
        }
      };
      float cx[UV][V], cy[UV][V];
      auto take_then_load = [&](uint32_t next) {
#pragma unroll
        for (int u = 0; u < UV; ++u) {
#pragma unroll
          for (int e = 0; e < V; ++e) {
            cx[u][e] = x[u][e];
            cy[u][e] = y[u][e];
            asm volatile("" : "+v"(cx[u][e]), "+v"(cy[u][e]));
          }
        }
        if (next < nchunks) load(next);
      };
      if (nchunks) {
        load(0);
        take_then_load(1);
      }
      for (uint32_t c = 0; c < nchunks; ++c) {
        const uint32_t bo = row_base(c, 0), q0 = (c % cpr) * 64 * UV;
#pragma unroll
        for (int u = 0; u < UV; ++u) {
          const uint32_t qv = q0 + 64 * u + lane;
          if (qv >= nv) continue;
          float rr[V];
#pragma unroll
          for (int e = 0; e < V; ++e) rr[e] = ew_apply<OP, DT>(cx[u][e], cy[u][e], alpha);
          T::stv(out, bo + qv * V, rr);
        }
        if (c + 1 < nchunks) take_then_load(c + 2);
      }
    }
    return;
  }
  for (uint32_t r = r0; r < r1; ++r) {
    const uint32_t i2 = r % s2, q = r / s2;
    const uint32_t i1 = q % s1, i0 = q / s1;
    uint32_t base[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) base[k] = i0 * st[k][0] + i1 * st[k][1] + i2 * st[k][2];
    for (uint32_t j0 = 0; j0 < L; j0 += 64 * U) {
      float x[U], y[U];
      uint32_t raw[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t j = j0 + 64 * u + lane;
        const bool ok = j < L;
        const uint32_t oa = base[1] + j * st[1][3];
        raw[u] = 0;
        x[u] = 0.0f;
        y[u] = 0.0f;
        if (!ok) continue;  // no access past the row
        if constexpr (OP == GPUOS_OP_COPY) {
          raw[u] = T::ES == 2 ? (uint32_t)ld16<CPL>(a, 2u * oa) : ld32<CPL>(a, 4u * oa);
        } else {
          x[u] = T::ld(a, oa);
          if constexpr (BIN) y[u] = T::ld(b, base[2] + j * st[2][3]);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t j = j0 + 64 * u + lane;
        if (j >= L) continue;
        const uint32_t oo = base[0] + j * st[0][3];
        if constexpr (OP == GPUOS_OP_COPY) {
          if constexpr (T::ES == 2) st16<CPS>(out, 2u * oo, (uint16_t)raw[u]);
          else st32<CPS>(out, 4u * oo, raw[u]);
        } else {
          T::st(out, oo, ew_apply<OP, DT>(x[u], y[u], alpha));
        }
      }
    }
  }
}

template <int ES, int CPL, int CPS>
__device__ __forceinline__ void copy_elem(rsrc_t dst, uint32_t i, rsrc_t src, uint32_t j) {
  if constexpr (ES == 4)
    st32<CPS>(dst, 4u * i, ld32<CPL>(src, 4u * j));
  else
    st16<CPS>(dst, 2u * i, ld16<CPL>(src, 2u * j));
}

// Bit copy of elements of ES bytes, with cyclic source (interleaved tiles).
template <int ES, int CPL, int CPS, class D>
__device__ __forceinline__ void copy_tile(D d, uint32_t t) {
  const uint32_t n = d(1), ntiles = d(6);
  const rsrc_t out = make_rsrc(d.q(18)), a = make_rsrc(d.q(20));
  const uint32_t ca = d(26);
  const uint32_t lane = lane_id();
  constexpr int V = 16 / ES;
  constexpr int U = 4;
  if (ca == 0 && aligned16(d.q(18)) && aligned16(d.q(20))) {
    const uint32_t nv = n / V, nrows = (nv + 63) / 64;
    const rsrc_t vo = make_rsrc_n(d.q(18), nv * 16u), va = make_rsrc_n(d.q(20), nv * 16u);
    const uint32_t ngroups = (nrows + U - 1) / U;
    u32x4 v[U];
    auto load = [&](uint32_t g) {
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = ld128<CPL>(va, vec_off((g * U + u) * 64 + lane));
    };
    if (t < ngroups) load(t);
    for (uint32_t g = t; g < ngroups; g += ntiles) {
      u32x4 c[U];
#pragma unroll
      for (int u = 0; u < U; ++u) c[u] = v[u];
      if (g + ntiles < ngroups) load(g + ntiles);
#pragma unroll
      for (int u = 0; u < U; ++u) st128<CPS>(vo, vec_off((g * U + u) * 64 + lane), c[u]);
    }
    if (t + 1 == ntiles)
      for (uint32_t i = nv * V + lane; i < n; i += 64) copy_elem<ES, CPL, CPS>(out, i, a, i);
    return;
  }
  for (uint32_t i = t * 64 + lane; i < n; i += 64 * ntiles)
    copy_elem<ES, CPL, CPS>(out, i, a, ca ? i % ca : i);
}

// out[k] = x[idx[k]]; returns an error code if any index is out of range.
template <int ES, int CPL, int CPS, class D>
__device__ __forceinline__ uint32_t gather_tile(D d, uint32_t t) {
  const uint32_t n = d(1), ntiles = d(6);
  const rsrc_t out = make_rsrc(d.q(18)), x = make_rsrc(d.q(20)), idx = make_rsrc(d.q(24));
  const int64_t bound = (int64_t)d(26);
  bool bad = false;
  for (uint32_t i = t * 64 + lane_id(); i < n; i += 64 * ntiles) {
    const int32_t j = (int32_t)ld32<CPL>(idx, 4u * i);
    if (j < 0 || (int64_t)j >= bound) {
      bad = true;
      continue;
    }
    copy_elem<ES, CPL, CPS>(out, i, x, (uint32_t)j);
  }
  return ballot(bad) ? (uint32_t)DERR_GATHER_RANGE : 0u;
}

// ---------------------------------------------------------------------------
// fused elementwise chain: acc = in[0]; for each step acc = op(acc, operand),
// rounded to the storage type after every step, optionally stored.  The
// intermediates stay in registers ("Launch Overhead and Fusion", "Fusion").

template <int V>
__device__ __forceinline__ void fused_step(uint32_t op, uint32_t fl, float scal, float (&acc)[V],
                                           const float (&opnd)[V]) {
  switch (op) {
    case FS_ADD:
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] = acc[e] + ((fl & FSF_SELF) ? acc[e] : opnd[e]);
      break;
    case FS_MUL:
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] = acc[e] * ((fl & FSF_SELF) ? acc[e] : opnd[e]);
      break;
    case FS_SCALE:
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] = scal * acc[e];
      break;
    case FS_RELU:
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] = acc[e] > 0.0f ? acc[e] : 0.0f;
      break;
    case FS_EXP:
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] = expf(acc[e]);
      break;
    default:  // FS_COPY
      break;
  }
}

// The step program of a fused descriptor, read once per tile.
struct FusedProg {
  uint32_t nsteps;
  uint32_t ops[2], fls[2];  // one byte per step
  uint32_t scal[kMaxSteps];
  uint64_t out[kMaxSteps];
  __device__ __forceinline__ uint32_t op(int s) const { return (ops[s / 4] >> (8 * (s % 4))) & 0xffu; }
  __device__ __forceinline__ uint32_t fl(int s) const { return (fls[s / 4] >> (8 * (s % 4))) & 0xffu; }
};

template <class D>
__device__ __forceinline__ FusedProg fused_prog(D d) {
  FusedProg p;
  p.nsteps = d(0) >> 24;
  p.ops[0] = d(42); p.ops[1] = d(43);
  p.fls[0] = d(44); p.fls[1] = d(45);
#pragma unroll
  for (int s = 0; s < kMaxSteps; ++s) {
    p.scal[s] = d(46 + s);
    p.out[s] = d.q(26 + 2 * s);
  }
  return p;
}

// Applies step s of the program to V values; returns the step's flags.
template <int V>
__device__ __forceinline__ uint32_t fused_apply(const FusedProg& P, int s, float (&acc)[V],
                                                const float (&v1)[V], const float (&v2)[V],
                                                const float (&v3)[V]) {
  const uint32_t sfl = P.fl(s);
  const uint32_t which = (sfl >> 4) & 3u;
  // operand = fused input `which`, selected with uniform bit masks (a select
  // between arrays would be lowered to a scratch-memory load)
  const uint32_t m1 = which == 1 ? ~0u : 0u, m2 = which == 2 ? ~0u : 0u, m3 = which == 3 ? ~0u : 0u;
  float opnd[V];
#pragma unroll
  for (int e = 0; e < V; ++e)
    opnd[e] = __uint_as_float((__float_as_uint(v1[e]) & m1) | (__float_as_uint(v2[e]) & m2) |
                              (__float_as_uint(v3[e]) & m3));
  fused_step<V>(P.op(s), sfl, __uint_as_float(P.scal[s]), acc, opnd);
  return sfl;
}

template <int DT, int CPL, int CPS, class D>
__device__ __forceinline__ void fused_tile(D d, uint32_t t) {
  static_assert(DT == GPUOS_F32, "fused chains are fp32");
  using T = DTr<DT, CPL, CPS>;
  constexpr int V = T::V;
  // rows of 64 vectors per group: with the next group in flight, 2 rows keep
  // 2 KiB per input per wave requested (4 rows measured 1-2% slower)
  constexpr int U = 2;
  const uint32_t n = d(1), ntiles = d(6);
  const uint64_t p0 = d.q(18), p1 = d.q(20), p2 = d.q(22), p3 = d.q(24);
  const FusedProg P = fused_prog(d);
  bool fast = aligned16(p0) && aligned16(p1) && aligned16(p2) && aligned16(p3);
#pragma unroll
  for (int s = 0; s < kMaxSteps; ++s) fast = fast && aligned16(P.out[s]);
  const uint32_t lane = lane_id();
  uint32_t scalar_from = t * 64, scalar_step = 64 * ntiles;  // per-element path
  if (fast) {
    // whole vectors only; rows past the end fall outside the resources, so
    // no load or store needs a bounds test; unused (null) inputs are not read
    const uint32_t nv = n / V, nrows = (nv + 63) / 64;
    const uint32_t vb = nv * 16u;
    const rsrc_t r0 = make_rsrc_n(p0, vb), r1 = make_rsrc_n(p1, vb), r2 = make_rsrc_n(p2, vb),
                 r3 = make_rsrc_n(p3, vb);
    const bool has1 = p1 != 0, has2 = p2 != 0, has3 = p3 != 0;
    const uint32_t ngroups = (nrows + U - 1) / U;
    float acc[U][V], v1[U][V], v2[U][V], v3[U][V];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < V; ++e) {
        v1[u][e] = 0.0f;
        v2[u][e] = 0.0f;
        v3[u][e] = 0.0f;
      }
    auto load = [&](uint32_t g) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t q = (g * U + u) * 64 + lane;
        T::ldq(r0, q, acc[u]);
        if (has1) T::ldq(r1, q, v1[u]);
        if (has2) T::ldq(r2, q, v2[u]);
        if (has3) T::ldq(r3, q, v3[u]);
      }
    };
    // software pipeline: group g + T is requested before group g is computed
    if (t < ngroups) load(t);
    for (uint32_t g = t; g < ngroups; g += ntiles) {
      float a[U][V], b1[U][V], b2[U][V], b3[U][V];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < V; ++e) {
          a[u][e] = acc[u][e];
          b1[u][e] = v1[u][e];
          b2[u][e] = v2[u][e];
          b3[u][e] = v3[u][e];
        }
      if (g + ntiles < ngroups) load(g + ntiles);
#pragma unroll
      for (int s = 0; s < kMaxSteps; ++s) {
        if ((uint32_t)s < P.nsteps) {
          uint32_t sfl = 0;
#pragma unroll
          for (int u = 0; u < U; ++u) sfl = fused_apply<V>(P, s, a[u], b1[u], b2[u], b3[u]);
          if (sfl & FSF_STORE) {
            const rsrc_t o = make_rsrc_n(P.out[s], vb);
#pragma unroll
            for (int u = 0; u < U; ++u) T::stq(o, (g * U + u) * 64 + lane, a[u]);
          }
        }
      }
    }
    if (t + 1 != ntiles) return;
    scalar_from = nv * V;  // leftover elements, last tile only
    scalar_step = 64;
  }
  const rsrc_t in0 = make_rsrc(p0), in1 = make_rsrc_n(p1, n * 4u), in2 = make_rsrc_n(p2, n * 4u),
               in3 = make_rsrc_n(p3, n * 4u);
  for (uint32_t i = scalar_from + lane; i < n; i += scalar_step) {
    float acc[1] = {T::ld(in0, i)};
    const float v1s[1] = {T::ld(in1, i)};
    const float v2s[1] = {T::ld(in2, i)};
    const float v3s[1] = {T::ld(in3, i)};
#pragma unroll
    for (int s = 0; s < kMaxSteps; ++s) {
      if ((uint32_t)s < P.nsteps) {
        const uint32_t sfl = fused_apply<1>(P, s, acc, v1s, v2s, v3s);
        if (sfl & FSF_STORE) T::st(make_rsrc(P.out[s]), i, acc[0]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// row reductions: one row at a time per wave.
//
// Vector path (16-byte aligned rows of whole vectors, no cyclic source): a
// row of up to 128 vectors (2 per lane) is loaded once and kept in
// registers; a longer row is swept in blocks of 16 values per lane with all
// of a block's loads issued before any is used.  Softmax keeps a running
// maximum and a sum rescaled to it (two sweeps: reduce, then write), RMSNORM
// a sum of squares (two sweeps), ROW_SUM a sum (one sweep).  Other rows take
// the per-element path (lane j reads elements j, j + 64, ...).

template <int DT, int CPL, int CPS>
struct RowReader {
  rsrc_t in;
  uint32_t base, ca;
  __device__ __forceinline__ float operator()(uint32_t j) const {
    const uint32_t e = base + j;
    return DTr<DT, CPL, CPS>::ld(in, ca ? e % ca : e);
  }
};

// Running softmax state of one lane: maximum m and sum of exp(x - m).  A
// -inf element adds nothing; NaN and +inf make the row NaN (as a
// max-subtracted softmax does).
struct SoftAcc {
  float m = -__builtin_inff();
  float s = 0.0f;
  __device__ __forceinline__ void add(float x) {
    if (x != x) {
      m = x;
      s = x;
      return;
    }
    if (x == -__builtin_inff()) return;
    if (x > m) {
      s = s * expf(m - x) + 1.0f;
      m = x;
    } else {
      s += expf(x - m);
    }
  }
};

// Combines the lanes' (m, s) into the row's maximum and sum.
__device__ __forceinline__ void soft_combine(SoftAcc a, float& M, float& S) {
  M = wave_max_nan(a.m);
  float part = a.s;
  if (a.m == -__builtin_inff())
    part = M == -__builtin_inff() ? __builtin_nanf("") : 0.0f;  // all -inf row: NaN
  else
    part = a.s * expf(a.m - M);
  S = wave_sum(part);
  if (M != M) S = M;
}

// One row on the vector path.  `in` / `out` cover exactly this row (whole
// vectors), so a lane's vectors past the row read as zeros and its stores are
// dropped; `g` covers the gain; ROW_SUM writes element r of `out`.
template <int OP, int DT, int CPL, int CPS>
__device__ __forceinline__ void row_vec(rsrc_t in, rsrc_t out, rsrc_t g, uint32_t r, uint32_t L,
                                        float eps) {
  using T = DTr<DT, CPL, CPS>;
  constexpr int V = T::V;
  const uint32_t lane = lane_id();
  const uint32_t nv = L / V;
  if (nv <= 128) {
    // the whole row in registers: 2 vectors per lane
    float x[2][V];
    const bool v0 = lane < nv, v1 = lane + 64 < nv;
    T::ldq(in, lane, x[0]);
    T::ldq(in, lane + 64, x[1]);
    if constexpr (OP == GPUOS_OP_ROW_SUM) {
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < V; ++e) s += x[0][e];
#pragma unroll
      for (int e = 0; e < V; ++e) s += x[1][e];
      s = wave_sum(s);
      if (lane == 0) T::st(out, r, s);
    } else if constexpr (OP == GPUOS_OP_ROW_SOFTMAX) {
      SoftAcc acc;
#pragma unroll
      for (int e = 0; e < V; ++e)
        if (v0) acc.add(x[0][e]);
#pragma unroll
      for (int e = 0; e < V; ++e)
        if (v1) acc.add(x[1][e]);
      float M, S;
      soft_combine(acc, M, S);
      float y[2][V];
#pragma unroll
      for (int e = 0; e < V; ++e) {
        y[0][e] = expf(x[0][e] - M) / S;
        y[1][e] = expf(x[1][e] - M) / S;
      }
      T::stq(out, lane, y[0]);
      T::stq(out, lane + 64, y[1]);
    } else {  // RMSNORM
      float q = 0.0f;
#pragma unroll
      for (int e = 0; e < V; ++e) q += x[0][e] * x[0][e];
#pragma unroll
      for (int e = 0; e < V; ++e) q += x[1][e] * x[1][e];
      const float ss = wave_sum(q);
      const float inv = 1.0f / sqrtf(ss / (float)L + eps);
      float w[2][V], y[2][V];
      T::ldq(g, lane, w[0]);
      T::ldq(g, lane + 64, w[1]);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        y[0][e] = x[0][e] * inv * w[0][e];
        y[1][e] = x[1][e] * inv * w[1][e];
      }
      T::stq(out, lane, y[0]);
      T::stq(out, lane + 64, y[1]);
    }
    return;
  }
  // long row: blocks of 16 values per lane (4 fp32 / 2 bf16 vectors)
  constexpr int B = 16 / V;
  float s = 0.0f;
  SoftAcc acc;
  for (uint32_t j0 = 0; j0 < nv; j0 += 64 * B) {
    float x[B][V];
#pragma unroll
    for (int u = 0; u < B; ++u) T::ldq(in, j0 + lane + 64 * u, x[u]);
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const bool v = j0 + lane + 64 * u < nv;
#pragma unroll
      for (int e = 0; e < V; ++e) {
        if constexpr (OP == GPUOS_OP_ROW_SUM) s += x[u][e];
        else if constexpr (OP == GPUOS_OP_RMSNORM) s += x[u][e] * x[u][e];
        else if (v) acc.add(x[u][e]);
      }
    }
  }
  if constexpr (OP == GPUOS_OP_ROW_SUM) {
    s = wave_sum(s);
    if (lane == 0) T::st(out, r, s);
    return;
  }
  float M = 0.0f, S = 0.0f, inv = 0.0f;
  if constexpr (OP == GPUOS_OP_ROW_SOFTMAX) soft_combine(acc, M, S);
  else inv = 1.0f / sqrtf(wave_sum(s) / (float)L + eps);
  for (uint32_t j0 = 0; j0 < nv; j0 += 64 * B) {
    float x[B][V], w[B][V];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      T::ldq(in, j0 + lane + 64 * u, x[u]);
      if constexpr (OP == GPUOS_OP_RMSNORM) T::ldq(g, j0 + lane + 64 * u, w[u]);
    }
#pragma unroll
    for (int u = 0; u < B; ++u) {
      float y[V];
#pragma unroll
      for (int e = 0; e < V; ++e) {
        if constexpr (OP == GPUOS_OP_ROW_SOFTMAX) y[e] = expf(x[u][e] - M) / S;
        else y[e] = x[u][e] * inv * w[u][e];
      }
      T::stq(out, j0 + lane + 64 * u, y);
    }
  }
}

template <int OP, int DT, int CPL, int CPS, class D>
__device__ __forceinline__ void row_tile(D d, uint32_t t) {
  using T = DTr<DT, CPL, CPS>;
  constexpr int V = T::V;
  const uint32_t rows = d(2), L = d(3), tile = d(7);
  const uint32_t r0 = t * tile;
  const uint32_t r1 = r0 + tile < rows ? r0 + tile : rows;
  const uint64_t pout = d.q(18), pin = d.q(20), pg = d.q(24);
  const uint32_t ca = d(26);
  const float eps = __uint_as_float(d(29));
  const uint32_t lane = lane_id();
  const bool vec = ca == 0 && L % V == 0 && aligned16(pin) &&
                   (OP == GPUOS_OP_ROW_SUM || aligned16(pout)) &&
                   (OP != GPUOS_OP_RMSNORM || aligned16(pg));
  if (vec) {
    const uint32_t rowbytes = L / V * 16u;
    const rsrc_t vg = make_rsrc_n(OP == GPUOS_OP_RMSNORM ? pg : 0, rowbytes);
    const rsrc_t sums = make_rsrc(pout);
    for (uint32_t r = r0; r < r1; ++r) {
      const uint64_t off = (uint64_t)r * rowbytes;
      const rsrc_t vin = make_rsrc_n(pin + off, rowbytes);
      const rsrc_t vout = OP == GPUOS_OP_ROW_SUM ? sums : make_rsrc_n(pout + off, rowbytes);
      row_vec<OP, DT, CPL, CPS>(vin, vout, vg, r, L, eps);
    }
    return;
  }
  const rsrc_t out = make_rsrc(pout), in = make_rsrc(pin), g = make_rsrc(pg);
  for (uint32_t r = r0; r < r1; ++r) {
    const RowReader<DT, CPL, CPS> x{in, r * L, ca};
    if constexpr (OP == GPUOS_OP_ROW_SUM) {
      float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
      uint32_t j = lane;
      for (; j + 192 < L; j += 256) {
        s0 += x(j); s1 += x(j + 64); s2 += x(j + 128); s3 += x(j + 192);
      }
      for (; j < L; j += 64) s0 += x(j);
      const float s = wave_sum((s0 + s1) + (s2 + s3));
      if (lane == 0) T::st(out, r, s);
    } else if constexpr (OP == GPUOS_OP_ROW_SOFTMAX) {
      SoftAcc acc;
      for (uint32_t j = lane; j < L; j += 64) acc.add(x(j));
      float M, S;
      soft_combine(acc, M, S);
      for (uint32_t jj = lane; jj < L; jj += 64) T::st(out, r * L + jj, expf(x(jj) - M) / S);
    } else {  // RMSNORM
      float q0 = 0.0f, q1 = 0.0f;
      uint32_t j = lane;
      for (; j + 64 < L; j += 128) {
        const float a = x(j), b = x(j + 64);
        q0 += a * a;
        q1 += b * b;
      }
      for (; j < L; j += 64) {
        const float a = x(j);
        q0 += a * a;
      }
      const float ss = wave_sum(q0 + q1);
      const float inv = 1.0f / sqrtf(ss / (float)L + eps);
      for (uint32_t jj = lane; jj < L; jj += 64) T::st(out, r * L + jj, x(jj) * inv * T::ld(g, jj));
    }
  }
}

// ---------------------------------------------------------------------------
// rotate-half rotary embedding, rows = heads of row_len = head_dim; each lane
// owns whole (i, i + h/2) pairs, so the op may run in place.  With 16-byte
// aligned operands and h/2 a multiple of 8, a lane takes 8 consecutive pairs
// with 128-bit loads (all of its loads in flight at once).

template <int DT, int CPL, int CPS, class D>
__device__ __forceinline__ void rope_tile(D d, uint32_t) {
  using T = DTr<DT, CPL, CPS>;
  const uint32_t heads = d(2), hd = d(3), half = hd / 2;
  const uint64_t pout = d.q(18), pin = d.q(20), ptab = d.q(24);
  const rsrc_t out = make_rsrc(pout), in = make_rsrc(pin), tab = make_rsrc(ptab);
  const uint32_t lane = lane_id();
  if (half % 8 == 0 && aligned16(pout) && aligned16(pin) && aligned16(ptab)) {
    const uint32_t per_head = half / 8, units = heads * per_head;
    for (uint32_t u = lane; u < units; u += 64) {
      const uint32_t h = u / per_head, i0 = (u - h * per_head) * 8;
      const uint32_t e1 = h * hd + i0, e2 = e1 + half;
      float x1[8], x2[8], c[8], s[8];
      if constexpr (T::ES == 2) {
        T::ldv(in, e1, x1);
        T::ldv(in, e2, x2);
      } else {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const u32x4 a = ld128<CPL>(in, 4u * (e1 + 4 * k)), b = ld128<CPL>(in, 4u * (e2 + 4 * k));
          x1[4 * k] = __uint_as_float(a.x); x1[4 * k + 1] = __uint_as_float(a.y);
          x1[4 * k + 2] = __uint_as_float(a.z); x1[4 * k + 3] = __uint_as_float(a.w);
          x2[4 * k] = __uint_as_float(b.x); x2[4 * k + 1] = __uint_as_float(b.y);
          x2[4 * k + 2] = __uint_as_float(b.z); x2[4 * k + 3] = __uint_as_float(b.w);
        }
      }
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const u32x4 a = ld128<CPL>(tab, 4u * (i0 + 4 * k)), b = ld128<CPL>(tab, 4u * (half + i0 + 4 * k));
        c[4 * k] = __uint_as_float(a.x); c[4 * k + 1] = __uint_as_float(a.y);
        c[4 * k + 2] = __uint_as_float(a.z); c[4 * k + 3] = __uint_as_float(a.w);
        s[4 * k] = __uint_as_float(b.x); s[4 * k + 1] = __uint_as_float(b.y);
        s[4 * k + 2] = __uint_as_float(b.z); s[4 * k + 3] = __uint_as_float(b.w);
      }
      float y1[8], y2[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float a1 = x1[k] * c[k], b1 = x2[k] * s[k];
        const float a2 = x2[k] * c[k], b2 = x1[k] * s[k];
        y1[k] = a1 - b1;
        y2[k] = a2 + b2;
      }
      if constexpr (T::ES == 2) {
        T::stv(out, e1, y1);
        T::stv(out, e2, y2);
      } else {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          u32x4 a, b;
          a.x = __float_as_uint(y1[4 * k]); a.y = __float_as_uint(y1[4 * k + 1]);
          a.z = __float_as_uint(y1[4 * k + 2]); a.w = __float_as_uint(y1[4 * k + 3]);
          b.x = __float_as_uint(y2[4 * k]); b.y = __float_as_uint(y2[4 * k + 1]);
          b.z = __float_as_uint(y2[4 * k + 2]); b.w = __float_as_uint(y2[4 * k + 3]);
          st128<CPS>(out, 4u * (e1 + 4 * k), a);
          st128<CPS>(out, 4u * (e2 + 4 * k), b);
        }
      }
    }
    return;
  }
  const uint32_t pairs = heads * half;
  for (uint32_t p = lane; p < pairs; p += 64) {
    const uint32_t h = p / half, i = p - h * half;
    const float x1 = T::ld(in, h * hd + i);
    const float x2 = T::ld(in, h * hd + half + i);
    const float c = __uint_as_float(ld32<CPL>(tab, 4u * i));
    const float s = __uint_as_float(ld32<CPL>(tab, 4u * (half + i)));
    const float a1 = x1 * c, b1 = x2 * s;
    const float a2 = x2 * c, b2 = x1 * s;
    T::st(out, h * hd + i, a1 - b1);
    T::st(out, h * hd + half + i, a2 + b2);
  }
}

// ---------------------------------------------------------------------------
// GEMV: out[i] = sum_k W[i, k] x[k]; `tile` rows per tile.  Lanes split K in
// 16-byte chunks of W (8 bf16); a step loads several chunks per lane (and up
// to 4 rows) with every load issued before the first FMA.

template <int DT, int CPL>
__device__ __forceinline__ void load_x8(rsrc_t x, uint32_t k, float (&v)[8]) {
  if constexpr (DT == GPUOS_BF16) {
    unpack_bf16x8(ld128<CPL>(x, 2u * k), v);
  } else {
    const u32x4 a = ld128<CPL>(x, 4u * k), b = ld128<CPL>(x, 4u * k + 16u);
    v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y);
    v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
    v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y);
    v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
  }
}

// Called where a GEMV tile may start reading x; the default does nothing.
struct NoWait {
  __device__ __forceinline__ void operator()() const {}
};

// GEMV epilogues: `load(i, nr)` runs on every lane once per step of rows
// i .. i + nr - 1, after the step's x loads (so after `ready()`);
// `store(i, r, s)` runs on lane 0 with the wave sum s of row i (= step row r).
template <int DT, int CPL, int CPS>
struct GemvStore {  // the plain op: round and store the row
  rsrc_t out;
  __device__ __forceinline__ void load(uint32_t, uint32_t) {}
  __device__ __forceinline__ void store(uint32_t i, int, float s) { DTr<DT, CPL, CPS>::st(out, i, s); }
};

// GEMV followed by ADD with a residual: the row is rounded as the GEMV stores
// it (and stored if the GEMV output is kept), then added to the residual
// element in the ADD's operand order and rounded as the ADD stores it.
template <int DT, int CPL, int CPS, int R>
struct GemvResAdd {
  using T = DTr<DT, CPL, CPS>;
  rsrc_t out, res, sum;
  bool keep, res_first;
  float rv[R];
  __device__ __forceinline__ void load(uint32_t i, uint32_t nr) {
#pragma unroll
    for (int r = 0; r < R; ++r) rv[r] = (uint32_t)r < nr ? T::ld(res, i + r) : 0.0f;
  }
  __device__ __forceinline__ void store(uint32_t i, int r, float s) {
    const float v = T::round(s);
    if (keep) T::st(out, i, v);
    T::st(sum, i, res_first ? rv[r] + v : v + rv[r]);
  }
};

// R rows at a time, C chunks per lane per step (x kept packed until used).
// `ready()` runs once, after the first step's weight loads are issued and
// before any load of x: a tile whose weights are already final can stream
// them while it waits for the op that produces x.
template <int R, int C, int DT, int CPL, int CPS, class Ready, class Epi>
__device__ __forceinline__ void gemv_rows(Epi& epi, uint64_t px, uint64_t pw, uint32_t K,
                                          uint32_t i0, uint32_t i1, Ready& ready) {
  using T = DTr<DT, CPL, CPS>;
  const uint32_t lane = lane_id();
  const uint32_t chunks = K / 8;
  // x and W clipped to whole chunks / the step's rows: anything past reads zeros
  const rsrc_t xv = make_rsrc_n(px, chunks * 8u * T::ES);
  bool waiting = true;
  for (uint32_t i = i0; i < i1; i += R) {
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.0f;
    const uint32_t nr = i1 - i < (uint32_t)R ? i1 - i : (uint32_t)R;
    const rsrc_t Wr = make_rsrc_n(pw + (uint64_t)i * K * 2u, nr * K * 2u);
    for (uint32_t c0 = 0; c0 < chunks; c0 += 64 * C) {
      u32x4 wr[R][C];
      u32x4 xp[C][T::ES / 2];  // 8 elements: one (bf16) or two (fp32) vectors
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const uint32_t ch = c0 + lane + 64 * c;
#pragma unroll
        for (int r = 0; r < R; ++r)
          wr[r][c] = ld128<CPL>(Wr, ch < chunks ? 2u * (r * K + ch * 8) : 0xFFF00000u);
      }
      if (waiting) {
        compiler_fence();
        ready();
        compiler_fence();
        waiting = false;
      }
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const uint32_t ch = c0 + lane + 64 * c;
        const uint32_t xo = ch < chunks ? ch * 8u * T::ES : 0xFFF00000u;
#pragma unroll
        for (int k = 0; k < T::ES / 2; ++k) xp[c][k] = ld128<CPL>(xv, xo + 16u * k);
      }
      if (c0 == 0) epi.load(i, nr);
#pragma unroll
      for (int c = 0; c < C; ++c) {
        float xf[8];
        if constexpr (DT == GPUOS_BF16) {
          unpack_bf16x8(xp[c][0], xf);
        } else {
          xf[0] = __uint_as_float(xp[c][0].x); xf[1] = __uint_as_float(xp[c][0].y);
          xf[2] = __uint_as_float(xp[c][0].z); xf[3] = __uint_as_float(xp[c][0].w);
          xf[4] = __uint_as_float(xp[c][1].x); xf[5] = __uint_as_float(xp[c][1].y);
          xf[6] = __uint_as_float(xp[c][1].z); xf[7] = __uint_as_float(xp[c][1].w);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float w[8];
          unpack_bf16x8(wr[r][c], w);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[r] = __builtin_fmaf(w[e], xf[e], acc[r]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float s = wave_sum(acc[r]);
      if (lane == 0 && (uint32_t)r < nr) epi.store(i + r, r, s);
    }
  }
  if (waiting) ready();
}

// Rows [t * tile, (t + 1) * tile) of a GEMV (or of a GEMV-ADD: `fused`).
template <int DT, int CPL, int CPS, class D, class Ready = NoWait>
__device__ __forceinline__ void gemv_tile(D d, uint32_t t, Ready ready = Ready(), bool fused = false) {
  using T = DTr<DT, CPL, CPS>;
  const uint32_t M = d(30), K = d(31), tile = d(7);
  const uint64_t px = d.q(20), pw = d.q(24);
  const rsrc_t x = make_rsrc(px), W = make_rsrc(pw);
  const uint32_t i0 = t * tile;
  const uint32_t i1 = i0 + tile < M ? i0 + tile : M;
  const uint32_t lane = lane_id();
  auto run = [&](auto& epi) {
    if ((K % 8 == 0) && aligned16(px) && aligned16(pw)) {
      // short rows: 4 rows per step, K <= 1,024 in one step; bf16 rows up to
      // 5,120: one row, all of K in one step; longer rows: one row per step,
      // 4,096 (bf16 x) or 2,048 (fp32 x) of K per step
      if (K <= 1024)
        gemv_rows<4, 2, DT, CPL, CPS>(epi, px, pw, K, i0, i1, ready);
      else if (DT == GPUOS_BF16 && K <= 5120)
        gemv_rows<1, 10, DT, CPL, CPS>(epi, px, pw, K, i0, i1, ready);  // one step
      else
        gemv_rows<1, DT == GPUOS_F32 ? 4 : 8, DT, CPL, CPS>(epi, px, pw, K, i0, i1, ready);
      return;
    }
    ready();
    for (uint32_t i = i0; i < i1; ++i) {
      float acc = 0.0f;
      for (uint32_t k = lane; k < K; k += 64)
        acc = __builtin_fmaf(bf2f(ld16<CPL>(W, 2u * (i * K + k))), T::ld(x, k), acc);
      acc = wave_sum(acc);
      epi.load(i, 1);
      if (lane == 0) epi.store(i, 0, acc);
    }
  };
  if (!fused) {
    GemvStore<DT, CPL, CPS> epi{make_rsrc(d.q(18))};
    run(epi);
  } else {
    GemvResAdd<DT, CPL, CPS, 4> epi;
    epi.out = make_rsrc(d.q(18));
    epi.res = make_rsrc(d.q(22));
    epi.sum = make_rsrc(d.q(32));
    epi.keep = d.q(18) != 0;
    epi.res_first = d(26) != 0;
    run(epi);
  }
}

// RMSNORM -> GEMV (-> SILU_MUL, or -> ROPE q, ROPE k, COPY v), bf16,
// K <= 1,024 (the normalised row is two 16-byte vectors per lane, in the
// GEMV's chunk layout).  Each value is the one the separate ops would store:
// the norm is summed in the same order as RMSNORM's in-register path and
// rounded to bf16, the GEMV accumulates in the same order as gemv_rows<4, 2>,
// its outputs are rounded to bf16, and the gate, or the rotation (with
// rope_tile's products and sums) and the copy, are applied to those rounded
// values.  A unit is one output row, a gate/up pair, or in rotary mode a
// pair of rows (i, i + hd/2) of one q or k head or two adjacent v rows.  Up
// to 4 output rows per step, two steps' weights requested together (the
// tile's first two before `ready()`).
template <int CPL, int CPS, class D, class Ready = NoWait>
__device__ __forceinline__ void norm_gemv_tile(D d, uint32_t t, Ready ready = Ready()) {
  using T = DTr<GPUOS_BF16, CPL, CPS>;
  const uint64_t pW = d.q(18), pout = d.q(20), px = d.q(22), pg = d.q(24), ph = d.q(26),
                 pact = d.q(28);
  const uint32_t M = d(30), K = d(31), F = d(33), tile = d(7);
  const float eps = __uint_as_float(d(32));
  const bool gate = pact != 0;
  const uint64_t prq = d.q(34), prk = d.q(36), prv = d.q(38), ptq = d.q(40), ptk = d.q(42);
  const bool rope = prq != 0;
  const uint32_t hd = rope ? d(44) : 2u, half = hd / 2;
  const uint32_t Dq = M / 3, hh = Dq / 2;  // rotary mode: rows per section, units per section
  const uint32_t units = gate ? F : rope ? M / 2 : M;
  const uint32_t u0 = t * tile;
  const uint32_t u1 = u0 + tile < units ? u0 + tile : units;
  const uint32_t lane = lane_id();
  const uint32_t chunks = K / 8;
  const rsrc_t xr = make_rsrc_n(px, chunks * 16u), gr = make_rsrc_n(pg, chunks * 16u);
  const rsrc_t W = make_rsrc_n(pW, M * K * 2u);
  const rsrc_t out = make_rsrc(pout), act = make_rsrc(pact);
  constexpr int R = 4;
  const bool paired = gate || rope;
  const uint32_t step = paired ? 2u : 4u;  // units per step
  // row `which` (0, 1) of rotary unit u
  auto pair_row = [&](uint32_t u, uint32_t which) -> uint32_t {
    const uint32_t sec = u / hh, w = u - sec * hh;
    if (sec >= 2) return 2 * Dq + 2 * w + which;
    const uint32_t h = w / half, p = w - h * half;
    return sec * Dq + h * hd + p + which * half;
  };
  // a step's rows: i .. i + 3; or units i, i + 1 as rows 0, 1 and their
  // partners (up rows F + i, F + i + 1, or the rotation partners) as rows 2, 3
  auto rows_of = [&](uint32_t i, uint32_t (&row)[R], bool (&ok)[R]) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t k = paired ? (uint32_t)(r & 1) : (uint32_t)r;
      ok[r] = i + k < u1;
      if (rope)
        row[r] = ok[r] ? pair_row(i + k, (uint32_t)r >> 1) : 0u;
      else
        row[r] = (gate && r >= 2 ? F : 0u) + i + k;
    }
  };
  // rotary mode: cos / sin of the 4 units from i on (0 for v units)
  float tc[4], ts[4];
  auto load_tab = [&](uint32_t i) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      tc[k] = 0.0f;
      ts[k] = 0.0f;
      const uint32_t u = i + k, sec = u / hh;
      if (u < u1 && sec < 2) {
        const uint32_t w = u - sec * hh, p = w - (w / half) * half;
        const rsrc_t tab = make_rsrc(sec == 0 ? ptq : ptk);
        tc[k] = __uint_as_float(ld32<CPL>(tab, 4u * p));
        ts[k] = __uint_as_float(ld32<CPL>(tab, 4u * (half + p)));
      }
    }
  };
  auto load_w = [&](const uint32_t (&row)[R], const bool (&ok)[R], u32x4 (&wr)[R][2]) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint32_t ch = lane + 64 * c;
#pragma unroll
      for (int r = 0; r < R; ++r)
        wr[r][c] = ld128<CPL>(W, ok[r] && ch < chunks ? 2u * (row[r] * K + ch * 8) : 0xFFF00000u);
    }
  };
  float hx[2][8];
  auto finish = [&](uint32_t i, uint32_t toff, const uint32_t (&row)[R], const bool (&ok)[R],
                    const u32x4 (&wr)[R][2]) {
    float acc[R] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float w[8];
        unpack_bf16x8(wr[r][c], w);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r] = __builtin_fmaf(w[e], hx[c][e], acc[r]);
      }
    }
    float v[R];
#pragma unroll
    for (int r = 0; r < R; ++r) v[r] = T::round(wave_sum(acc[r]));
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (ok[r] && pout) T::st(out, row[r], v[r]);
      if (gate) {
#pragma unroll
        for (int k = 0; k < 2; ++k)
          if (ok[k]) T::st(act, i + k, ew_apply<GPUOS_OP_SILU_MUL>(v[k], v[k + 2], 0.0f));
      }
      if (rope) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          if (!ok[k]) continue;
          const uint32_t u = i + k, sec = u / hh, w = u - sec * hh;
          const float x1 = v[k], x2 = v[k + 2];
          if (sec < 2) {
            const float c = tc[toff + k], sn = ts[toff + k];
            const float a1 = x1 * c, b1 = x2 * sn;
            const float a2 = x2 * c, b2 = x1 * sn;
            const uint32_t h = w / half, e1 = h * hd + (w - h * half);
            const rsrc_t dst = make_rsrc(sec == 0 ? prq : prk);
            T::st(dst, e1, a1 - b1);
            T::st(dst, e1 + half, a2 + b2);
          } else {
            const rsrc_t dst = make_rsrc(prv);
            T::st(dst, 2 * w, x1);
            T::st(dst, 2 * w + 1, x2);
          }
        }
      }
    }
  };
  bool waiting = true;
  // two steps at a time: both steps' weights are requested before the first
  // use (and, for the tile's first pair, before `ready()`)
  for (uint32_t i = u0; i < u1; i += 2 * step) {
    uint32_t rowA[R], rowB[R];
    bool okA[R], okB[R];
    rows_of(i, rowA, okA);
    rows_of(i + step, rowB, okB);
    u32x4 wA[R][2], wB[R][2];
    load_w(rowA, okA, wA);
    load_w(rowB, okB, wB);
    if (waiting) {
      compiler_fence();
      ready();
      compiler_fence();
      waiting = false;
      // the normalised row, as RMSNORM computes and stores it
      float xv[2][8], gv[2][8];
      T::ldq(xr, lane, xv[0]);
      T::ldq(xr, lane + 64, xv[1]);
      T::ldq(gr, lane, gv[0]);
      T::ldq(gr, lane + 64, gv[1]);
      float q = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) q += xv[0][e] * xv[0][e];
#pragma unroll
      for (int e = 0; e < 8; ++e) q += xv[1][e] * xv[1][e];
      const float ss = wave_sum(q);
      const float inv = 1.0f / sqrtf(ss / (float)K + eps);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        hx[0][e] = T::round(xv[0][e] * inv * gv[0][e]);
        hx[1][e] = T::round(xv[1][e] * inv * gv[1][e]);
      }
      if (t == 0 && ph) {
        const rsrc_t hr = make_rsrc_n(ph, chunks * 16u);
        T::stq(hr, lane, hx[0]);
        T::stq(hr, lane + 64, hx[1]);
      }
    }
    if (rope) load_tab(i);
    finish(i, 0, rowA, okA, wA);
    if (i + step < u1) finish(i + step, 2, rowB, okB, wB);
  }
  if (waiting) ready();
}

// ---------------------------------------------------------------------------
// attention scores: out[h*S + j] = alpha * <q_h, K[j, h]>, `tile` key rows per
// tile.  Lanes walk the key rows in 16-byte chunks; the Dh/8 lanes holding
// one (j, h) pair reduce together.

template <int DT, int CPL, int CPS, int CPH, class D>
__device__ __forceinline__ void score_rows_fast(D d, uint32_t j0, uint32_t j1) {
  const uint32_t H = d(30), Dh = d(31), S = d(32);
  const uint32_t HD = H * Dh, cpr = HD / 8;  // 16-byte chunks per key row
  const rsrc_t out = make_rsrc(d.q(18)), q = make_rsrc(d.q(20)), Kc = make_rsrc(d.q(24));
  const float alpha = __uint_as_float(d(28));
  const uint32_t lane = lane_id();
  const uint32_t total = (j1 - j0) * cpr;
  // two 64-chunk groups per step, both groups' loads issued first
  for (uint32_t f0 = 0; f0 < total; f0 += 128) {
    float qv[2][8];
    u32x4 kv[2];
    uint32_t j[2], c[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint32_t f = f0 + 64 * u + lane;
      const uint32_t fc = f < total ? f : 0;
      j[u] = j0 + fc / cpr;
      c[u] = fc - (j[u] - j0) * cpr;
      load_x8<DT, CPL>(q, c[u] * 8, qv[u]);
      kv[u] = ld128<CPL>(Kc, 2u * (j[u] * HD + c[u] * 8));
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint32_t f = f0 + 64 * u + lane;
      float k8[8];
      unpack_bf16x8(kv[u], k8);
      float part = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) part = __builtin_fmaf(qv[u][e], k8[e], part);
      part = group_sum<CPH>(part);
      const uint32_t h = c[u] / CPH;
      if (f < total && (c[u] % CPH) == 0)
        st32<CPS>(out, 4u * (h * S + j[u]), __float_as_uint(alpha * part));
    }
    (void)Dh;
  }
}

template <int DT, int CPL, int CPS, class D>
__device__ __forceinline__ void attn_score_tile(D d, uint32_t t) {
  using T = DTr<DT, CPL, CPS>;
  const uint32_t H = d(30), Dh = d(31), S = d(32), tile = d(7);
  const uint32_t j0 = t * tile;
  const uint32_t j1 = j0 + tile < S ? j0 + tile : S;
  const bool aligned = aligned16(d.q(20)) && aligned16(d.q(24));
  if (aligned && Dh == 64) {
    score_rows_fast<DT, CPL, CPS, 8>(d, j0, j1);
    return;
  }
  if (aligned && Dh == 128) {
    score_rows_fast<DT, CPL, CPS, 16>(d, j0, j1);
    return;
  }
  // general head size: one (j, h) pair per lane
  const rsrc_t out = make_rsrc(d.q(18)), q = make_rsrc(d.q(20)), Kc = make_rsrc(d.q(24));
  const float alpha = __uint_as_float(d(28));
  const uint32_t HD = H * Dh;
  const uint32_t pairs = (j1 - j0) * H;
  for (uint32_t p = lane_id(); p < pairs; p += 64) {
    const uint32_t j = j0 + p / H, h = p % H;
    float acc = 0.0f;
    for (uint32_t e = 0; e < Dh; ++e)
      acc = __builtin_fmaf(T::ld(q, h * Dh + e), bf2f(ld16<CPL>(Kc, 2u * (j * HD + h * Dh + e))), acc);
    st32<CPS>(out, 4u * (h * S + j), __float_as_uint(alpha * acc));
  }
}

// attention output: out[h*Dh + c] = sum_j p[h, j] V[j, h*Dh + c]; a tile is
// `tile` 8-column chunks; lanes split the key positions.
template <int DT, int CPL, int CPS, class D>
__device__ __forceinline__ void attn_av_tile(D d, uint32_t t) {
  using T = DTr<DT, CPL, CPS>;
  const uint32_t H = d(30), Dh = d(31), S = d(32), tile = d(7);
  const uint32_t HD = H * Dh;
  const rsrc_t out = make_rsrc(d.q(18)), p = make_rsrc(d.q(20)), Vc = make_rsrc(d.q(24));
  const uint32_t lane = lane_id();
  if ((Dh % 8) == 0 && aligned16(d.q(24))) {
    const uint32_t nchunks = HD / 8;
    const uint32_t c0 = t * tile;
    const uint32_t c1 = c0 + tile < nchunks ? c0 + tile : nchunks;
    // p and V clipped to the S key positions: positions past S read zeros
    const rsrc_t pv = make_rsrc_n(d.q(20), H * S * 4u);
    const rsrc_t Vv = make_rsrc_n(d.q(24), S * HD * 2u);
    for (uint32_t c = c0; c < c1; ++c) {
      const uint32_t h = (c * 8) / Dh;
      float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      // 8 key positions per lane per step, every load of a step issued first
      for (uint32_t jb = 0; jb < S; jb += 64 * 8) {
        float w[8];
        u32x4 vr[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const uint32_t j = jb + 64 * u + lane;
          const bool ok = j < S;
          w[u] = __uint_as_float(ld32<CPL>(pv, ok ? 4u * (h * S + j) : 0xFFF00000u));
          vr[u] = ld128<CPL>(Vv, ok ? 2u * (j * HD + c * 8) : 0xFFF00000u);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          float v[8];
          unpack_bf16x8(vr[u], v);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(w[u], v[e], acc[e]);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = wave_sum(acc[e]);
      if (lane < 8) {
        float mine = acc[0];
#pragma unroll
        for (int e = 1; e < 8; ++e)
          if (lane == (uint32_t)e) mine = acc[e];
        T::st(out, c * 8 + lane, mine);
      }
    }
  } else {
    // general: `tile` counts single columns
    const uint32_t c0 = t * tile;
    const uint32_t c1 = c0 + tile < HD ? c0 + tile : HD;
    for (uint32_t c = c0; c < c1; ++c) {
      const uint32_t h = c / Dh;
      float acc = 0.0f;
      for (uint32_t j = lane; j < S; j += 64)
        acc = __builtin_fmaf(__uint_as_float(ld32<CPL>(p, 4u * (h * S + j))),
                             bf2f(ld16<CPL>(Vc, 2u * (j * HD + c))), acc);
      acc = wave_sum(acc);
      if (lane == 0) T::st(out, c, acc);
    }
  }
}

// ROW_SOFTMAX -> ATTN_AV (fp32 score rows of S <= 512 elements, Dh % 8 == 0,
// 16-byte aligned scores, probabilities and V).  Tile t is AV chunk t (8
// output columns of head h).  The wave computes the softmax of score row h
// itself, with ROW_SOFTMAX's in-register arithmetic (the head's first chunk
// also stores the row when it is kept), hands the probabilities to the AV
// lanes through its LDS scratch (`kWaveScratch` floats) and sums them against
// V in attn_av_tile's order, so every stored value matches the separate ops.
// V and the score row are requested together.
template <int DT, int CPL, int CPS, class D>
__device__ __forceinline__ void softmax_av_tile(D d, uint32_t t, lds_f32* scr) {
  using T = DTr<DT, CPL, CPS>;
  using F = DTr<GPUOS_F32, CPL, CPS>;
  const uint32_t H = d(30), Dh = d(31), S = d(32);
  const uint32_t HD = H * Dh;
  const uint64_t pout = d.q(18), pp = d.q(20), px = d.q(22), pV = d.q(24);
  const uint32_t lane = lane_id();
  const uint32_t c = t;
  const uint32_t h = (c * 8) / Dh;
  const uint32_t rowbytes = S * 4u;
  const rsrc_t Vv = make_rsrc_n(pV, S * HD * 2u);
  u32x4 vr[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const uint32_t j = 64 * u + lane;
    vr[u] = ld128<CPL>(Vv, j < S ? 2u * (j * HD + c * 8) : 0xFFF00000u);
  }
  const rsrc_t vin = make_rsrc_n(px + (uint64_t)h * rowbytes, rowbytes);
  float x[2][4];
  F::ldq(vin, lane, x[0]);
  F::ldq(vin, lane + 64, x[1]);
  const uint32_t nv = S / 4;
  const bool v0 = lane < nv, v1 = lane + 64 < nv;
  SoftAcc acc;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (v0) acc.add(x[0][e]);
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (v1) acc.add(x[1][e]);
  float M, Ssum;
  soft_combine(acc, M, Ssum);
  float y[2][4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    y[0][e] = expf(x[0][e] - M) / Ssum;
    y[1][e] = expf(x[1][e] - M) / Ssum;
  }
  if (pp && (c * 8) % Dh == 0) {
    const rsrc_t vout = make_rsrc_n(pp + (uint64_t)h * rowbytes, rowbytes);
    F::stq(vout, lane, y[0]);
    F::stq(vout, lane + 64, y[1]);
  }
  // element 4k + e of the row sits in lane k (k < 64) or k - 64 (k >= 64);
  // a wave's LDS accesses complete in issue order
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    scr[4 * lane + e] = y[0][e];
    scr[256 + 4 * lane + e] = y[1][e];
  }
  float w[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const uint32_t j = 64 * u + lane;
    w[u] = j < S ? scr[j] : 0.0f;
  }
  float a8[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    float v[8];
    unpack_bf16x8(vr[u], v);
#pragma unroll
    for (int e = 0; e < 8; ++e) a8[e] = __builtin_fmaf(w[u], v[e], a8[e]);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) a8[e] = wave_sum(a8[e]);
  if (lane < 8) {
    float mine = a8[0];
#pragma unroll
    for (int e = 1; e < 8; ++e)
      if (lane == (uint32_t)e) mine = a8[e];
    T::st(make_rsrc(pout), c * 8 + lane, mine);
  }
}

// ---------------------------------------------------------------------------
// debug op: spin for aux[0] nanoseconds (s_memrealtime ticks at 100 MHz),
// bounded to 10 ms.
template <class D>
__device__ __forceinline__ void spin_tile(D d, uint32_t) {
  uint64_t ns = d(30);
  if (ns > 10000000u) ns = 10000000u;
  const uint64_t t0 = now_ticks();
  const uint64_t ticks = ns / 10u;
  while (now_ticks() - t0 < ticks) __builtin_amdgcn_s_sleep(8);
}

// ---------------------------------------------------------------------------
// opcode switch over the fixed op table (uniform per wave: a scalar branch,
// no indirect call).  Returns a device error code, 0 on success.

// One elementwise opcode in each dtype it takes (int32 only where INT).
template <int OP, bool INT, int CPL, int CPS, class D>
__device__ __forceinline__ void ew_any(uint32_t dt, D d, uint32_t t) {
  if (dt == GPUOS_BF16) ew_tile<OP, GPUOS_BF16, CPL, CPS>(d, t);
  else if (dt == GPUOS_F16) ew_tile<OP, GPUOS_F16, CPL, CPS>(d, t);
  else if constexpr (INT) {
    if (dt == GPUOS_I32) ew_tile<OP, GPUOS_I32, CPL, CPS>(d, t);
    else ew_tile<OP, GPUOS_F32, CPL, CPS>(d, t);
  } else ew_tile<OP, GPUOS_F32, CPL, CPS>(d, t);
}

template <int OP, bool INT, int CPL, int CPS, class D>
__device__ __forceinline__ void ew_view_any(uint32_t dt, D d, uint32_t t) {
  if (dt == GPUOS_BF16) ew_view_tile<OP, GPUOS_BF16, CPL, CPS>(d, t);
  else if (dt == GPUOS_F16) ew_view_tile<OP, GPUOS_F16, CPL, CPS>(d, t);
  else if constexpr (INT) {
    if (dt == GPUOS_I32) ew_view_tile<OP, GPUOS_I32, CPL, CPS>(d, t);
    else ew_view_tile<OP, GPUOS_F32, CPL, CPS>(d, t);
  } else ew_view_tile<OP, GPUOS_F32, CPL, CPS>(d, t);
}

// Elementwise ops over a view (DF_VIEW).
template <int CPL, int CPS, class D>
__device__ __forceinline__ uint32_t exec_view(uint32_t op, uint32_t dt, D d, uint32_t t) {
  switch (op) {
    case GPUOS_OP_COPY:  // bits: the 2- or 4-byte move of any dtype
      if ((d(0) >> 16) & DF_VIEW_T) {
        if (dt == GPUOS_BF16 || dt == GPUOS_F16) copy_transposed_tile<2, CPL, CPS>(d, t);
        else copy_transposed_tile<4, CPL, CPS>(d, t);
      } else if (dt == GPUOS_BF16 || dt == GPUOS_F16) {
        ew_view_tile<GPUOS_OP_COPY, GPUOS_BF16, CPL, CPS>(d, t);
      } else {
        ew_view_tile<GPUOS_OP_COPY, GPUOS_F32, CPL, CPS>(d, t);
      }
      return 0;
    case GPUOS_OP_ADD: ew_view_any<GPUOS_OP_ADD, true, CPL, CPS>(dt, d, t); return 0;
    case GPUOS_OP_MUL: ew_view_any<GPUOS_OP_MUL, true, CPL, CPS>(dt, d, t); return 0;
    case GPUOS_OP_RELU: ew_view_any<GPUOS_OP_RELU, true, CPL, CPS>(dt, d, t); return 0;
    case GPUOS_OP_SCALE: ew_view_any<GPUOS_OP_SCALE, false, CPL, CPS>(dt, d, t); return 0;
    case GPUOS_OP_EXP: ew_view_any<GPUOS_OP_EXP, false, CPL, CPS>(dt, d, t); return 0;
    case GPUOS_OP_SILU_MUL: ew_view_any<GPUOS_OP_SILU_MUL, false, CPL, CPS>(dt, d, t); return 0;
    default: return (uint32_t)DERR_BAD_OPCODE;
  }
}

// Streaming ops (elementwise, copy, fused chains) under cache policies CPL /
// CPS; returns false for any other opcode.
template <int CPL, int CPS, class D>
__device__ __forceinline__ bool exec_stream(uint32_t op, uint32_t dt, D d, uint32_t t, uint32_t& err) {
  err = 0;
  switch (op) {
    case GPUOS_OP_COPY:
      if (dt == GPUOS_BF16 || dt == GPUOS_F16) copy_tile<2, CPL, CPS>(d, t); else copy_tile<4, CPL, CPS>(d, t);
      return true;
    case GPUOS_OP_ADD: ew_any<GPUOS_OP_ADD, true, CPL, CPS>(dt, d, t); return true;
    case GPUOS_OP_MUL: ew_any<GPUOS_OP_MUL, true, CPL, CPS>(dt, d, t); return true;
    case GPUOS_OP_RELU: ew_any<GPUOS_OP_RELU, true, CPL, CPS>(dt, d, t); return true;
    case GPUOS_OP_SCALE: ew_any<GPUOS_OP_SCALE, false, CPL, CPS>(dt, d, t); return true;
    case GPUOS_OP_EXP: ew_any<GPUOS_OP_EXP, false, CPL, CPS>(dt, d, t); return true;
    case GPUOS_OP_SILU_MUL: ew_any<GPUOS_OP_SILU_MUL, false, CPL, CPS>(dt, d, t); return true;
    case GPUOS_OP_PROGRAM:
      if (dt == GPUOS_BF16) prog_tile<GPUOS_BF16, CPL, CPS>(d, t);
      else if (dt == GPUOS_F16) prog_tile<GPUOS_F16, CPL, CPS>(d, t);
      else prog_tile<GPUOS_F32, CPL, CPS>(d, t);
      return true;
    case OP_FUSED_EW:  // fp32 chains only (the fusion pass leaves other dtypes unfused)
      if (dt != GPUOS_F32) err = (uint32_t)DERR_BAD_OPCODE;
      else fused_tile<GPUOS_F32, CPL, CPS>(d, t);
      return true;
    default:
      return false;
  }
}

// Cache-policy bit that marks an access non-temporal (streamed: its lines
// are the first to be evicted).
constexpr int CP_NT = 2;

template <int CPL, int CPS, class D>
__device__ __forceinline__ uint32_t exec_tile(D d, uint32_t t, lds_f32* scr) {
  const uint32_t w0 = d(0);
  const uint32_t op = w0 & 0xffu, dt = (w0 >> 8) & 0xffu, fl = (w0 >> 16) & 0xffu;
  const bool bf = dt == GPUOS_BF16, hf = dt == GPUOS_F16;
  constexpr int F = GPUOS_F32, B = GPUOS_BF16, H = GPUOS_F16;
  uint32_t err = 0;
  if (fl & DF_VIEW) return exec_view<CPL, CPS>(op, dt, d, t);
  if (fl & GPUOS_FLAG_NONTEMPORAL) {
    if (exec_stream<CPL | CP_NT, CPS | CP_NT>(op, dt, d, t, err)) return err;
  } else {
    if (exec_stream<CPL, CPS>(op, dt, d, t, err)) return err;
  }
  switch (op) {
    case GPUOS_OP_NOP:
      return 0;
    case GPUOS_OP_GATHER:
      return bf ? gather_tile<2, CPL, CPS>(d, t) : gather_tile<4, CPL, CPS>(d, t);
    case GPUOS_OP_ROW_SUM:
      if (bf) row_tile<GPUOS_OP_ROW_SUM, B, CPL, CPS>(d, t);
      else if (hf) row_tile<GPUOS_OP_ROW_SUM, H, CPL, CPS>(d, t);
      else row_tile<GPUOS_OP_ROW_SUM, F, CPL, CPS>(d, t);
      return 0;
    case GPUOS_OP_ROW_SOFTMAX:
      if (bf) row_tile<GPUOS_OP_ROW_SOFTMAX, B, CPL, CPS>(d, t);
      else if (hf) row_tile<GPUOS_OP_ROW_SOFTMAX, H, CPL, CPS>(d, t);
      else row_tile<GPUOS_OP_ROW_SOFTMAX, F, CPL, CPS>(d, t);
      return 0;
    case GPUOS_OP_RMSNORM:
      if (bf) row_tile<GPUOS_OP_RMSNORM, B, CPL, CPS>(d, t);
      else if (hf) row_tile<GPUOS_OP_RMSNORM, H, CPL, CPS>(d, t);
      else row_tile<GPUOS_OP_RMSNORM, F, CPL, CPS>(d, t);
      return 0;
    case GPUOS_OP_ROPE:
      if (bf) rope_tile<B, CPL, CPS>(d, t);
      else if (hf) rope_tile<H, CPL, CPS>(d, t);
      else rope_tile<F, CPL, CPS>(d, t);
      return 0;
    case GPUOS_OP_GEMV:
      if (bf) gemv_tile<B, CPL, CPS>(d, t); else gemv_tile<F, CPL, CPS>(d, t);
      return 0;
    case GPUOS_OP_ATTN_SCORE:
      if (bf) attn_score_tile<B, CPL, CPS>(d, t); else attn_score_tile<F, CPL, CPS>(d, t);
      return 0;
    case GPUOS_OP_ATTN_AV:
      if (bf) attn_av_tile<B, CPL, CPS>(d, t); else attn_av_tile<F, CPL, CPS>(d, t);
      return 0;
    case GPUOS_OP_SPIN:
      spin_tile(d, t);
      return 0;
    case OP_NORM_GEMV:
      if (!bf) return (uint32_t)DERR_BAD_OPCODE;
      norm_gemv_tile<CPL, CPS>(d, t);
      return 0;
    case OP_GEMV_ADD:
      if (bf) gemv_tile<B, CPL, CPS>(d, t, NoWait(), true);
      else gemv_tile<F, CPL, CPS>(d, t, NoWait(), true);
      return 0;
    case OP_SOFTMAX_AV:
      if (bf) softmax_av_tile<B, CPL, CPS>(d, t, scr); else softmax_av_tile<F, CPL, CPS>(d, t, scr);
      return 0;
    default:
      return (uint32_t)DERR_BAD_OPCODE;
  }
}

}  // namespace gpuos
