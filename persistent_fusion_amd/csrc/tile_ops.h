// Tile bodies of the op table, shared by the resident kernel and the per-op
// launch comparator.  A body runs on one wave64 and processes one tile of one
// descriptor; `d(i)` returns dword i of the descriptor (uniform), `d.q(i)` the
// 64-bit value at dwords i, i+1.
//
// Memory-bound ops stream with 128-bit loads and stores (4 fp32 or 8 bf16 per
// lane); reductions keep a row in registers and reduce across the wave.  No op
// here is a dense contraction (batch-1 GEMV moves ~2 bytes per flop), so
// nothing uses MFMA.  Exact-class ops (COPY, GATHER, ADD, MUL, SCALE, RELU,
// ROPE) are single IEEE operations per element; the library is compiled with
// contraction off so a*b+c is never fused into an FMA.
#pragma once

#include "device_common.h"
#include "gpuos_internal.h"
#include "../../include/gpuos.h"

namespace gpuos {

// ---------------------------------------------------------------------------
// element types

template <int DT>
struct DTr;

template <>
struct DTr<GPUOS_F32> {
  static constexpr int V = 4;  // elements per 16-byte access
  __device__ static __forceinline__ float ld(uint64_t p, uint32_t i) {
    return ldg<float>(p + 4ull * i);
  }
  __device__ static __forceinline__ void st(uint64_t p, uint32_t i, float v) {
    stg<float>(p + 4ull * i, v);
  }
  __device__ static __forceinline__ void ldv(uint64_t p, uint32_t i, float (&x)[4]) {
    const u32x4 t = ldg<u32x4>(p + 4ull * i);
    x[0] = __uint_as_float(t.x); x[1] = __uint_as_float(t.y);
    x[2] = __uint_as_float(t.z); x[3] = __uint_as_float(t.w);
  }
  __device__ static __forceinline__ void stv(uint64_t p, uint32_t i, const float (&x)[4]) {
    u32x4 t;
    t.x = __float_as_uint(x[0]); t.y = __float_as_uint(x[1]);
    t.z = __float_as_uint(x[2]); t.w = __float_as_uint(x[3]);
    stg<u32x4>(p + 4ull * i, t);
  }
  __device__ static __forceinline__ float round(float v) { return v; }
};

__device__ __forceinline__ void unpack_bf16x8(const u32x4& t, float (&w)[8]) {
  w[0] = bf2f(t.x & 0xffffu); w[1] = bf2f(t.x >> 16);
  w[2] = bf2f(t.y & 0xffffu); w[3] = bf2f(t.y >> 16);
  w[4] = bf2f(t.z & 0xffffu); w[5] = bf2f(t.z >> 16);
  w[6] = bf2f(t.w & 0xffffu); w[7] = bf2f(t.w >> 16);
}

template <>
struct DTr<GPUOS_BF16> {
  static constexpr int V = 8;
  __device__ static __forceinline__ float ld(uint64_t p, uint32_t i) {
    return bf2f(ldg<uint16_t>(p + 2ull * i));
  }
  __device__ static __forceinline__ void st(uint64_t p, uint32_t i, float v) {
    stg<uint16_t>(p + 2ull * i, (uint16_t)f2bf(v));
  }
  __device__ static __forceinline__ void ldv(uint64_t p, uint32_t i, float (&x)[8]) {
    unpack_bf16x8(ldg<u32x4>(p + 2ull * i), x);
  }
  __device__ static __forceinline__ void stv(uint64_t p, uint32_t i, const float (&x)[8]) {
    u32x4 t;
    t.x = f2bf(x[0]) | (f2bf(x[1]) << 16);
    t.y = f2bf(x[2]) | (f2bf(x[3]) << 16);
    t.z = f2bf(x[4]) | (f2bf(x[5]) << 16);
    t.w = f2bf(x[6]) | (f2bf(x[7]) << 16);
    stg<u32x4>(p + 2ull * i, t);
  }
  // value after a round trip through bf16 storage
  __device__ static __forceinline__ float round(float v) { return bf2f(f2bf(v)); }
};

// ---------------------------------------------------------------------------
// elementwise semantics (one IEEE operation each; see gpuos.h)

template <int OP>
__device__ __forceinline__ float ew_apply(float x, float y, float alpha) {
  if constexpr (OP == GPUOS_OP_ADD) return x + y;
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

// Elements [lo, hi) of tile t of an elementwise op.
template <class D>
__device__ __forceinline__ void tile_range(const D& d, uint32_t t, uint32_t& lo, uint32_t& hi) {
  const uint32_t n = d(1), tile = d(7);
  lo = t * tile;
  hi = lo + tile < n ? lo + tile : n;
}

template <int OP, int DT, class D>
__device__ __forceinline__ void ew_tile(const D& d, uint32_t t) {
  using T = DTr<DT>;
  constexpr int V = T::V;
  constexpr bool BIN = ew_binary<OP>();
  constexpr int U = DT == GPUOS_F32 ? 4 : 2;
  uint32_t lo, hi;
  tile_range(d, t, lo, hi);
  const uint64_t out = d.q(18), a = d.q(20), b = d.q(22);
  const uint32_t ca = d(26), cb = d(27);
  const float alpha = __uint_as_float(d(28));
  const uint32_t lane = lane_id();
  const bool fast = ca == 0 && (!BIN || cb == 0) && aligned16(out) && aligned16(a) &&
                    (!BIN || aligned16(b));
  uint32_t vend = lo;
  if (fast) {
    vend = lo + ((hi - lo) / V) * V;
    for (uint32_t base = lo; base < vend; base += 64 * V * U) {
      float x[U][V], y[U][V];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t i = base + (u * 64 + lane) * V;
        if (i < vend) {
          T::ldv(a, i, x[u]);
          if constexpr (BIN) T::ldv(b, i, y[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t i = base + (u * 64 + lane) * V;
        if (i < vend) {
          float r[V];
#pragma unroll
          for (int e = 0; e < V; ++e) r[e] = ew_apply<OP>(x[u][e], BIN ? y[u][e] : 0.0f, alpha);
          T::stv(out, i, r);
        }
      }
    }
  }
  for (uint32_t i = vend + lane; i < hi; i += 64) {
    const float x = T::ld(a, ca ? i % ca : i);
    const float y = BIN ? T::ld(b, cb ? i % cb : i) : 0.0f;
    T::st(out, i, ew_apply<OP>(x, y, alpha));
  }
}

template <int ES>
__device__ __forceinline__ void copy_elem(uint64_t dst, uint64_t src) {
  if constexpr (ES == 4)
    stg<uint32_t>(dst, ldg<uint32_t>(src));
  else
    stg<uint16_t>(dst, ldg<uint16_t>(src));
}

// Bit copy of elements of ES bytes, with cyclic source.
template <int ES, class D>
__device__ __forceinline__ void copy_tile(const D& d, uint32_t t) {
  uint32_t lo, hi;
  tile_range(d, t, lo, hi);
  const uint64_t out = d.q(18), a = d.q(20);
  const uint32_t ca = d(26);
  const uint32_t lane = lane_id();
  constexpr int V = 16 / ES;
  uint32_t vend = lo;
  if (ca == 0 && aligned16(out) && aligned16(a)) {
    vend = lo + ((hi - lo) / V) * V;
    for (uint32_t base = lo; base < vend; base += 64 * V * 4) {
      u32x4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t i = base + (u * 64 + lane) * V;
        if (i < vend) v[u] = ldg<u32x4>(a + (uint64_t)i * ES);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t i = base + (u * 64 + lane) * V;
        if (i < vend) stg<u32x4>(out + (uint64_t)i * ES, v[u]);
      }
    }
  }
  for (uint32_t i = vend + lane; i < hi; i += 64) {
    const uint32_t j = ca ? i % ca : i;
    copy_elem<ES>(out + (uint64_t)i * ES, a + (uint64_t)j * ES);
  }
}

// out[k] = x[idx[k]]; returns an error code if any index is out of range.
template <int ES, class D>
__device__ __forceinline__ uint32_t gather_tile(const D& d, uint32_t t) {
  uint32_t lo, hi;
  tile_range(d, t, lo, hi);
  const uint64_t out = d.q(18), x = d.q(20), idx = d.q(24);
  const int64_t bound = (int64_t)d(26);
  bool bad = false;
  for (uint32_t i = lo + lane_id(); i < hi; i += 64) {
    const int32_t j = ldg<int32_t>(idx + 4ull * i);
    if (j < 0 || (int64_t)j >= bound) {
      bad = true;
      continue;
    }
    copy_elem<ES>(out + (uint64_t)i * ES, x + (uint64_t)j * ES);
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

template <int DT, class D>
__device__ __forceinline__ void fused_tile(const D& d, uint32_t t) {
  using T = DTr<DT>;
  constexpr int V = T::V;
  constexpr int U = DT == GPUOS_F32 ? 2 : 1;
  uint32_t lo, hi;
  tile_range(d, t, lo, hi);
  const uint32_t nsteps = d(0) >> 24;
  const uint64_t in0 = d.q(18), in1 = d.q(20), in2 = d.q(22), in3 = d.q(24);
  bool fast = aligned16(in0) && aligned16(in1) && aligned16(in2) && aligned16(in3);
#pragma unroll
  for (int s = 0; s < kMaxSteps; ++s) fast = fast && aligned16(d.q(26 + 2 * s));
  const uint32_t lane = lane_id();
  uint32_t vend = lo;
  if (fast) {
    vend = lo + ((hi - lo) / V) * V;
    for (uint32_t base = lo; base < vend; base += 64 * V * U) {
      float acc[U][V], v1[U][V], v2[U][V], v3[U][V];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t i = base + (u * 64 + lane) * V;
        if (i < vend) {
          T::ldv(in0, i, acc[u]);
          if (in1) T::ldv(in1, i, v1[u]);
          if (in2) T::ldv(in2, i, v2[u]);
          if (in3) T::ldv(in3, i, v3[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t i = base + (u * 64 + lane) * V;
        if (i < vend) {
#pragma unroll
          for (int s = 0; s < kMaxSteps; ++s) {
            if ((uint32_t)s < nsteps) {
              const uint32_t sop = (d(42 + s / 4) >> (8 * (s % 4))) & 0xffu;
              const uint32_t sfl = (d(44 + s / 4) >> (8 * (s % 4))) & 0xffu;
              const uint32_t which = (sfl >> 4) & 3u;
              float opnd[V];
#pragma unroll
              for (int e = 0; e < V; ++e)
                opnd[e] = which == 1 ? v1[u][e] : (which == 2 ? v2[u][e] : v3[u][e]);
              fused_step<V>(sop, sfl, __uint_as_float(d(46 + s)), acc[u], opnd);
              if constexpr (DT == GPUOS_BF16) {
#pragma unroll
                for (int e = 0; e < V; ++e) acc[u][e] = T::round(acc[u][e]);
              }
              if (sfl & FSF_STORE) T::stv(d.q(26 + 2 * s), i, acc[u]);
            }
          }
        }
      }
    }
  }
  for (uint32_t i = vend + lane; i < hi; i += 64) {
    float acc[1] = {T::ld(in0, i)};
    const float v1s = in1 ? T::ld(in1, i) : 0.0f;
    const float v2s = in2 ? T::ld(in2, i) : 0.0f;
    const float v3s = in3 ? T::ld(in3, i) : 0.0f;
#pragma unroll
    for (int s = 0; s < kMaxSteps; ++s) {
      if ((uint32_t)s < nsteps) {
        const uint32_t sop = (d(42 + s / 4) >> (8 * (s % 4))) & 0xffu;
        const uint32_t sfl = (d(44 + s / 4) >> (8 * (s % 4))) & 0xffu;
        const uint32_t which = (sfl >> 4) & 3u;
        const float opnd[1] = {which == 1 ? v1s : (which == 2 ? v2s : v3s)};
        fused_step<1>(sop, sfl, __uint_as_float(d(46 + s)), acc, opnd);
        acc[0] = T::round(acc[0]);
        if (sfl & FSF_STORE) T::st(d.q(26 + 2 * s), i, acc[0]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// row reductions: one row at a time per wave.  A pass over the row is a
// coalesced sweep (lane j reads elements j, j + 64, ...); multi-pass ops
// (softmax: max, sum of exponentials, write; RMSNORM: sum of squares, write)
// re-read the row while it is still in L2.

template <int DT>
struct RowReader {
  uint64_t in;
  uint32_t base, ca;
  __device__ __forceinline__ float operator()(uint32_t j) const {
    const uint32_t e = base + j;
    return DTr<DT>::ld(in, ca ? e % ca : e);
  }
};

template <int OP, int DT, class D>
__device__ __forceinline__ void row_tile(const D& d, uint32_t t) {
  using T = DTr<DT>;
  const uint32_t rows = d(2), L = d(3), tile = d(7);
  const uint32_t r0 = t * tile;
  const uint32_t r1 = r0 + tile < rows ? r0 + tile : rows;
  const uint64_t out = d.q(18), in = d.q(20), g = d.q(24);
  const uint32_t ca = d(26);
  const float eps = __uint_as_float(d(29));
  const uint32_t lane = lane_id();
  for (uint32_t r = r0; r < r1; ++r) {
    const RowReader<DT> x{in, r * L, ca};
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
      float m = -__builtin_inff();
      for (uint32_t j = lane; j < L; j += 64) m = nan_max(m, x(j));
      m = wave_max_nan(m);
      float s0 = 0.0f, s1 = 0.0f;
      uint32_t j = lane;
      for (; j + 64 < L; j += 128) {
        s0 += expf(x(j) - m);
        s1 += expf(x(j + 64) - m);
      }
      for (; j < L; j += 64) s0 += expf(x(j) - m);
      const float s = wave_sum(s0 + s1);
      for (uint32_t jj = lane; jj < L; jj += 64) T::st(out, r * L + jj, expf(x(jj) - m) / s);
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
      const float ms = ss / (float)L;
      const float inv = 1.0f / sqrtf(ms + eps);
      for (uint32_t jj = lane; jj < L; jj += 64) T::st(out, r * L + jj, x(jj) * inv * T::ld(g, jj));
    }
  }
}

// ---------------------------------------------------------------------------
// rotate-half rotary embedding, rows = heads of row_len = head_dim; each lane
// owns whole (i, i + h/2) pairs, so the op may run in place.

template <int DT, class D>
__device__ __forceinline__ void rope_tile(const D& d, uint32_t) {
  using T = DTr<DT>;
  const uint32_t heads = d(2), hd = d(3), half = hd / 2;
  const uint64_t out = d.q(18), in = d.q(20), tab = d.q(24);
  const uint32_t pairs = heads * half;
  for (uint32_t p = lane_id(); p < pairs; p += 64) {
    const uint32_t h = p / half, i = p - h * half;
    const float x1 = T::ld(in, h * hd + i);
    const float x2 = T::ld(in, h * hd + half + i);
    const float c = ldg<float>(tab + 4ull * i), s = ldg<float>(tab + 4ull * (half + i));
    const float a1 = x1 * c, b1 = x2 * s;
    const float a2 = x2 * c, b2 = x1 * s;
    T::st(out, h * hd + i, a1 - b1);
    T::st(out, h * hd + half + i, a2 + b2);
  }
}

// ---------------------------------------------------------------------------
// GEMV: out[i] = sum_k W[i, k] x[k]; `tile` rows per tile, up to 4 rows in
// flight per wave; lanes split K in 16-byte chunks of W (8 bf16).

template <int DT>
__device__ __forceinline__ void load_x8(uint64_t x, uint32_t k, float (&v)[8]) {
  if constexpr (DT == GPUOS_BF16) {
    unpack_bf16x8(ldg<u32x4>(x + 2ull * k), v);
  } else {
    const u32x4 a = ldg<u32x4>(x + 4ull * k), b = ldg<u32x4>(x + 4ull * k + 16);
    v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y);
    v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
    v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y);
    v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
  }
}

template <int DT, class D>
__device__ __forceinline__ void gemv_tile(const D& d, uint32_t t) {
  using T = DTr<DT>;
  const uint32_t M = d(30), K = d(31), tile = d(7);
  const uint64_t out = d.q(18), x = d.q(20), W = d.q(24);
  const uint32_t i0 = t * tile;
  const uint32_t i1 = i0 + tile < M ? i0 + tile : M;
  const uint32_t lane = lane_id();
  const bool fast = (K % 8 == 0) && aligned16(x) && aligned16(W);
  if (fast) {
    const uint32_t chunks = K / 8;
    constexpr int R = 4;
    for (uint32_t i = i0; i < i1; i += R) {
      float acc[R] = {0.0f, 0.0f, 0.0f, 0.0f};
      for (uint32_t c = lane; c < chunks; c += 64) {
        float xv[8];
        load_x8<DT>(x, c * 8, xv);
        u32x4 wr[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
          if (i + r < i1) wr[r] = ldg<u32x4>(W + 2ull * ((uint64_t)(i + r) * K + c * 8));
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if (i + r < i1) {
            float w[8];
            unpack_bf16x8(wr[r], w);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[r] = __builtin_fmaf(w[e], xv[e], acc[r]);
          }
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (i + r < i1) {
          const float s = wave_sum(acc[r]);
          if (lane == 0) T::st(out, i + r, s);
        }
      }
    }
  } else {
    for (uint32_t i = i0; i < i1; ++i) {
      float acc = 0.0f;
      for (uint32_t k = lane; k < K; k += 64)
        acc = __builtin_fmaf(bf2f(ldg<uint16_t>(W + 2ull * ((uint64_t)i * K + k))), T::ld(x, k), acc);
      acc = wave_sum(acc);
      if (lane == 0) T::st(out, i, acc);
    }
  }
}

// ---------------------------------------------------------------------------
// attention scores: out[h*S + j] = alpha * <q_h, K[j, h]>, `tile` key rows per
// tile.  Lanes walk the key rows in 16-byte chunks; the Dh/8 lanes holding
// one (j, h) pair reduce together.

template <int DT, int CPH, class D>
__device__ __forceinline__ void score_rows_fast(const D& d, uint32_t j0, uint32_t j1) {
  const uint32_t H = d(30), Dh = d(31), S = d(32);
  const uint32_t HD = H * Dh, cpr = HD / 8;  // 16-byte chunks per key row
  const uint64_t out = d.q(18), q = d.q(20), Kc = d.q(24);
  const float alpha = __uint_as_float(d(28));
  const uint32_t lane = lane_id();
  const uint32_t total = (j1 - j0) * cpr;
  for (uint32_t f0 = 0; f0 < total; f0 += 64) {
    const uint32_t f = f0 + lane;
    float part = 0.0f;
    uint32_t j = 0, h = 0, c = 0;
    if (f < total) {
      j = j0 + f / cpr;
      c = f - (j - j0) * cpr;
      h = c / CPH;
      float qv[8], kv[8];
      load_x8<DT>(q, c * 8, qv);
      unpack_bf16x8(ldg<u32x4>(Kc + 2ull * ((uint64_t)j * HD + c * 8)), kv);
#pragma unroll
      for (int e = 0; e < 8; ++e) part = __builtin_fmaf(qv[e], kv[e], part);
    }
    part = group_sum<CPH>(part);
    if (f < total && (c % CPH) == 0) stg<float>(out + 4ull * ((uint64_t)h * S + j), alpha * part);
    (void)Dh;
  }
}

template <int DT, class D>
__device__ __forceinline__ void attn_score_tile(const D& d, uint32_t t) {
  using T = DTr<DT>;
  const uint32_t H = d(30), Dh = d(31), S = d(32), tile = d(7);
  const uint32_t j0 = t * tile;
  const uint32_t j1 = j0 + tile < S ? j0 + tile : S;
  const bool aligned = aligned16(d.q(20)) && aligned16(d.q(24));
  if (aligned && Dh == 64) {
    score_rows_fast<DT, 8>(d, j0, j1);
    return;
  }
  if (aligned && Dh == 128) {
    score_rows_fast<DT, 16>(d, j0, j1);
    return;
  }
  // general head size: one (j, h) pair per lane
  const uint64_t out = d.q(18), q = d.q(20), Kc = d.q(24);
  const float alpha = __uint_as_float(d(28));
  const uint32_t HD = H * Dh;
  const uint32_t pairs = (j1 - j0) * H;
  for (uint32_t p = lane_id(); p < pairs; p += 64) {
    const uint32_t j = j0 + p / H, h = p % H;
    float acc = 0.0f;
    for (uint32_t e = 0; e < Dh; ++e)
      acc = __builtin_fmaf(T::ld(q, h * Dh + e),
                           bf2f(ldg<uint16_t>(Kc + 2ull * ((uint64_t)j * HD + h * Dh + e))), acc);
    stg<float>(out + 4ull * ((uint64_t)h * S + j), alpha * acc);
  }
}

// attention output: out[h*Dh + c] = sum_j p[h, j] V[j, h*Dh + c]; a tile is
// `tile` 8-column chunks; lanes split the key positions.
template <int DT, class D>
__device__ __forceinline__ void attn_av_tile(const D& d, uint32_t t) {
  using T = DTr<DT>;
  const uint32_t H = d(30), Dh = d(31), S = d(32), tile = d(7);
  const uint32_t HD = H * Dh;
  const uint64_t out = d.q(18), p = d.q(20), Vc = d.q(24);
  const uint32_t lane = lane_id();
  if ((Dh % 8) == 0 && aligned16(Vc)) {
    const uint32_t nchunks = HD / 8;
    const uint32_t c0 = t * tile;
    const uint32_t c1 = c0 + tile < nchunks ? c0 + tile : nchunks;
    for (uint32_t c = c0; c < c1; ++c) {
      const uint32_t h = (c * 8) / Dh;
      float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (uint32_t j = lane; j < S; j += 64) {
        const float w = ldg<float>(p + 4ull * ((uint64_t)h * S + j));
        float v[8];
        unpack_bf16x8(ldg<u32x4>(Vc + 2ull * ((uint64_t)j * HD + c * 8)), v);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(w, v[e], acc[e]);
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
        acc = __builtin_fmaf(ldg<float>(p + 4ull * ((uint64_t)h * S + j)),
                             bf2f(ldg<uint16_t>(Vc + 2ull * ((uint64_t)j * HD + c))), acc);
      acc = wave_sum(acc);
      if (lane == 0) T::st(out, c, acc);
    }
  }
}

// ---------------------------------------------------------------------------
// debug op: spin for aux[0] nanoseconds (s_memrealtime ticks at 100 MHz),
// bounded to 10 ms.
template <class D>
__device__ __forceinline__ void spin_tile(const D& d, uint32_t) {
  uint64_t ns = d(30);
  if (ns > 10000000u) ns = 10000000u;
  const uint64_t t0 = now_ticks();
  const uint64_t ticks = ns / 10u;
  while (now_ticks() - t0 < ticks) __builtin_amdgcn_s_sleep(8);
}

// ---------------------------------------------------------------------------
// opcode switch over the fixed op table (uniform per wave: a scalar branch,
// no indirect call).  Returns a device error code, 0 on success.

template <class D>
__device__ uint32_t exec_tile(const D& d, uint32_t t) {
  const uint32_t w0 = d(0);
  const uint32_t op = w0 & 0xffu, dt = (w0 >> 8) & 0xffu;
  const bool bf = dt == GPUOS_BF16;
  switch (op) {
    case GPUOS_OP_NOP:
      return 0;
    case GPUOS_OP_COPY:
      if (bf) copy_tile<2>(d, t); else copy_tile<4>(d, t);
      return 0;
    case GPUOS_OP_GATHER:
      return bf ? gather_tile<2>(d, t) : gather_tile<4>(d, t);
    case GPUOS_OP_ADD:
      if (bf) ew_tile<GPUOS_OP_ADD, GPUOS_BF16>(d, t); else ew_tile<GPUOS_OP_ADD, GPUOS_F32>(d, t);
      return 0;
    case GPUOS_OP_MUL:
      if (bf) ew_tile<GPUOS_OP_MUL, GPUOS_BF16>(d, t); else ew_tile<GPUOS_OP_MUL, GPUOS_F32>(d, t);
      return 0;
    case GPUOS_OP_SCALE:
      if (bf) ew_tile<GPUOS_OP_SCALE, GPUOS_BF16>(d, t); else ew_tile<GPUOS_OP_SCALE, GPUOS_F32>(d, t);
      return 0;
    case GPUOS_OP_RELU:
      if (bf) ew_tile<GPUOS_OP_RELU, GPUOS_BF16>(d, t); else ew_tile<GPUOS_OP_RELU, GPUOS_F32>(d, t);
      return 0;
    case GPUOS_OP_EXP:
      if (bf) ew_tile<GPUOS_OP_EXP, GPUOS_BF16>(d, t); else ew_tile<GPUOS_OP_EXP, GPUOS_F32>(d, t);
      return 0;
    case GPUOS_OP_SILU_MUL:
      if (bf) ew_tile<GPUOS_OP_SILU_MUL, GPUOS_BF16>(d, t);
      else ew_tile<GPUOS_OP_SILU_MUL, GPUOS_F32>(d, t);
      return 0;
    case GPUOS_OP_ROW_SUM:
      if (bf) row_tile<GPUOS_OP_ROW_SUM, GPUOS_BF16>(d, t);
      else row_tile<GPUOS_OP_ROW_SUM, GPUOS_F32>(d, t);
      return 0;
    case GPUOS_OP_ROW_SOFTMAX:
      if (bf) row_tile<GPUOS_OP_ROW_SOFTMAX, GPUOS_BF16>(d, t);
      else row_tile<GPUOS_OP_ROW_SOFTMAX, GPUOS_F32>(d, t);
      return 0;
    case GPUOS_OP_RMSNORM:
      if (bf) row_tile<GPUOS_OP_RMSNORM, GPUOS_BF16>(d, t);
      else row_tile<GPUOS_OP_RMSNORM, GPUOS_F32>(d, t);
      return 0;
    case GPUOS_OP_ROPE:
      if (bf) rope_tile<GPUOS_BF16>(d, t); else rope_tile<GPUOS_F32>(d, t);
      return 0;
    case GPUOS_OP_GEMV:
      if (bf) gemv_tile<GPUOS_BF16>(d, t); else gemv_tile<GPUOS_F32>(d, t);
      return 0;
    case GPUOS_OP_ATTN_SCORE:
      if (bf) attn_score_tile<GPUOS_BF16>(d, t); else attn_score_tile<GPUOS_F32>(d, t);
      return 0;
    case GPUOS_OP_ATTN_AV:
      if (bf) attn_av_tile<GPUOS_BF16>(d, t); else attn_av_tile<GPUOS_F32>(d, t);
      return 0;
    case GPUOS_OP_SPIN:
      spin_tile(d, t);
      return 0;
    case OP_FUSED_EW:
      if (bf) fused_tile<GPUOS_BF16>(d, t); else fused_tile<GPUOS_F32>(d, t);
      return 0;
    default:
      return (uint32_t)DERR_BAD_OPCODE;
  }
}

}  // namespace gpuos
