// Resident scheduler kernel and per-op comparator kernel (gfx950).
//
// The resident kernel is the persistent worker of "GPUOS: A GPU Operating
// System Primitive for Transparent Operation Fusion" (section "The Paper"):
// it is launched once and drains a host-managed work queue instead of taking
// one launch per op.  Wave 0 is the doorbell/tracker wave: it polls the ring
// tails the host publishes in pinned memory (the user-space form of the
// doorbell in "Kernel Launch and Host-Device Interaction", section "The launch
// path"), makes new descriptors claimable, and retires completed descriptors in
// order, publishing the retire cursor back to host memory.  Every other wave is
// a worker: it claims tiles with an atomic ticket, maps the ticket to its
// descriptor, waits for the descriptor's dependencies, runs the tile through
// the opcode switch and counts it done.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "gpuos_internal.h"
#include "kernels.h"
#include "tile_ops.h"

namespace gpuos {

// Descriptor held in one VGPR: lane i keeps dword i.
struct VDesc {
  uint32_t v;
  __device__ __forceinline__ uint32_t operator()(int i) const {
    return (uint32_t)__builtin_amdgcn_readlane((int)v, i);
  }
  __device__ __forceinline__ uint64_t q(int i) const {
    return (uint64_t)(*this)(i) | ((uint64_t)(*this)(i + 1) << 32);
  }
};

// Per-wave cache of the descriptor the wave last worked on, per ring.
struct Cached {
  uint64_t seq;    // 0 = none
  uint64_t start;  // first ticket
  uint64_t end;    // one past the last ticket
  uint32_t dw;     // this lane's descriptor dword
  uint32_t deps_ok;
};

__device__ __forceinline__ uint32_t slot_of(uint64_t seq, uint32_t mask) {
  return (uint32_t)((seq - 1) & mask);
}

__device__ void report_error(const KArgs& a, uint32_t ring, uint64_t seq, uint64_t code) {
  if (lane_id() == 0) {
    st_rlx_sys(&a.hctl->error_seq, ((uint64_t)ring << 62) | seq);
    st_rel_sys(&a.hctl->error, code);
  }
}

// ---------------------------------------------------------------------------
// ticket -> descriptor

// Finds the descriptor owning `ticket` among sequences (lo, hi]:
// ends(s) = dends[(s - 1) mod 2C] is the first ticket after descriptor s
// (C = ring slots).  A 64-way search: every lane probes one sequence, a ballot
// picks the first probe past the ticket; each round shrinks the range 64-fold.
//
// Probes stay inside (hi - C, hi], and no probed entry can be overwritten
// while the search runs: the ticket's own descriptor X (>= retired + 1, with
// hi <= retired + C at publication) cannot retire before this wave runs it, so
// the host can publish at most up to X - 1 + C < s + 2C for any probed s.
template <int RING>
__device__ uint64_t find_seq(const KArgs& a, uint64_t ticket, uint64_t lo, uint64_t hi) {
  const uint32_t lane = lane_id();
  const uint32_t mask = a.cap_mask;
  if (hi > (uint64_t)mask + 1 && lo < hi - mask - 1) lo = hi - mask - 1;
  while (hi - lo > 1) {
    const uint64_t span = hi - lo;
    const uint64_t step = (span + 63) / 64;
    uint64_t s = lo + step * (lane + 1);
    if (s > hi) s = hi;
    const uint64_t e = ld_rlx_agent(&a.dends[RING][slot_of(s, a.ends_mask)]);
    const uint64_t past = ballot(e > ticket);
    // the probe at hi is always past the ticket, so `past` is non-empty
    const uint32_t f = (uint32_t)__builtin_ctzll(past);
    const uint64_t nhi = lo + step * (f + 1) > hi ? hi : lo + step * (f + 1);
    const uint64_t nlo = f == 0 ? lo : lo + step * f;
    lo = nlo;
    hi = nhi;
  }
  return hi;
}

template <int RING>
__device__ void fetch_desc(const KArgs& a, uint64_t seq, Cached& c) {
  const uint32_t* src = reinterpret_cast<const uint32_t*>(&a.hdesc[RING][slot_of(seq, a.cap_mask)]);
  c.dw = ld_rlx_sys(src + lane_id());
  VDesc d{c.dw};
  c.seq = seq;
  c.start = d.q(60);
  c.end = c.start + d(6);
  c.deps_ok = 0;
  if (d(63) != ((uint32_t)seq ^ kDescMagic)) report_error(a, RING, seq, DERR_DESC_CHECK);
}

template <int RING>
__device__ void wait_deps(const KArgs& a, const Cached& c) {
  VDesc d{c.dw};
  const uint32_t mask = a.cap_mask;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint64_t dep = d.q(8 + 2 * i);
    if (dep) {
      const uint64_t* w = &a.done_id[RING][slot_of(dep, mask)];
      while (bcast64(ld_rlx_agent(w)) < dep) __builtin_amdgcn_s_sleep(2);
    }
  }
  const uint64_t wr = d.q(16);
  if (wr) {
    while (bcast64(ld_rlx_agent(&a.dctl->ring[RING].retired)) < wr) __builtin_amdgcn_s_sleep(4);
  }
  fence_acq_agent();
}

// Counts one tile done; the wave finishing the last tile publishes the
// descriptor's completion (done_id) for dependents and the doorbell wave.
template <int RING>
__device__ void finish_tile(const KArgs& a, const Cached& c, uint64_t t_start) {
  const uint32_t slot = slot_of(c.seq, a.cap_mask);
  VDesc d{c.dw};
  const uint32_t ntiles = d(6);
  fence_rel_agent();
  uint32_t old = 0;
  if (lane_id() == 0)
    old = __hip_atomic_fetch_add(&a.tiles_done[RING][slot], 1u, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
  old = bcast(old);
  if (old + 1 == ntiles) {
    fence_acq_agent();
    if (lane_id() == 0) {
      a.tiles_done[RING][slot] = 0;
      if (a.trace[RING]) {
        TraceRec* tr = &a.trace[RING][slot];
        tr->seq = c.seq;
        tr->t_done = now_ticks();
        tr->opcode = d(0) & 0xffu;
        tr->ntiles = ntiles;
      }
    }
    if (lane_id() == 0) st_rel_agent(&a.done_id[RING][slot], c.seq);
  }
  (void)t_start;
}

template <int RING>
__device__ void run_ticket(const KArgs& a, uint64_t ticket, Cached& c) {
  if (!c.deps_ok) {
    wait_deps<RING>(a, c);
    c.deps_ok = 1;
  }
  const uint32_t tile = (uint32_t)(ticket - c.start);
  VDesc d{c.dw};
  if (a.trace[RING] && tile == 0 && lane_id() == 0)
    a.trace[RING][slot_of(c.seq, a.cap_mask)].t_claim = now_ticks();
  const uint32_t err = exec_tile(d, tile);
  if (err) report_error(a, RING, c.seq, err);
  finish_tile<RING>(a, c, 0);
}

// Maps a claimable ticket to its descriptor (refreshing the cache if needed).
template <int RING>
__device__ void map_ticket(const KArgs& a, uint64_t ticket, uint64_t avail_ops, Cached& c) {
  if (c.seq != 0 && ticket < c.end) return;
  const uint64_t seq = find_seq<RING>(a, ticket, c.seq, avail_ops);
  fetch_desc<RING>(a, seq, c);
}

// Latency-critical ring: claims with compare-and-swap so a wave never holds a
// priority ticket that has no work behind it.  Priority tiles are drained
// before the wave returns to its best-effort ticket.
__device__ void service_lc(const KArgs& a, Cached& c) {
  DevRing* R = &a.dctl->ring[1];
  for (;;) {
    uint64_t nxt = 0, av = 0, avops = 0;
    if (lane_id() == 0) {
      av = ld_acq_agent(&R->avail_tiles);
      nxt = ld_rlx_agent(&R->next);
    }
    av = bcast64(av);
    nxt = bcast64(nxt);
    if (nxt >= av) return;
    uint32_t ok = 0;
    if (lane_id() == 0) {
      uint64_t expect = nxt;
      ok = __hip_atomic_compare_exchange_strong(&R->next, &expect, nxt + 1, __ATOMIC_RELAXED,
                                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
               ? 1u
               : 0u;
      avops = ld_acq_agent(&R->avail_ops);
    }
    ok = bcast(ok);
    avops = bcast64(avops);
    if (!ok) continue;
    map_ticket<1>(a, nxt, avops, c);
    run_ticket<1>(a, nxt, c);
  }
}

__device__ void worker_loop(const KArgs& a) {
  DevRing* R = &a.dctl->ring[0];
  Cached c0{0, 0, 0, 0, 0}, c1{0, 0, 0, 0, 0};
  uint64_t avail = 0, avail_ops = 0;
  uint32_t idle = 0;
  uint64_t ticket = 0;
  if (lane_id() == 0)
    ticket = __hip_atomic_fetch_add(&R->next, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  ticket = bcast64(ticket);
  for (;;) {
    if (a.lc_enabled) service_lc(a, c1);
    if (ticket >= avail) {
      uint64_t av = 0, ao = 0;
      if (lane_id() == 0) {
        av = ld_acq_agent(&R->avail_tiles);
        ao = ld_acq_agent(&R->avail_ops);
      }
      avail = bcast64(av);
      avail_ops = bcast64(ao);
      if (ticket >= avail) {
        // nothing published for this ticket yet: back off
        if (idle < 64) {
          ++idle;
          __builtin_amdgcn_s_sleep(2);
        } else {
          __builtin_amdgcn_s_sleep(16);
        }
        continue;
      }
    }
    idle = 0;
    map_ticket<0>(a, ticket, avail_ops, c0);
    if ((VDesc{c0.dw}(0) & 0xffu) == OP_STOP) {
      finish_tile<0>(a, c0, 0);
      return;
    }
    run_ticket<0>(a, ticket, c0);
    if (lane_id() == 0)
      ticket = __hip_atomic_fetch_add(&R->next, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ticket = bcast64(ticket);
  }
}

// ---------------------------------------------------------------------------
// doorbell / tracker wave

template <int RING>
__device__ bool publish_ring(const KArgs& a, uint64_t tail, uint64_t& avail) {
  if (tail <= avail) return false;
  const uint32_t mask = a.cap_mask;
  const uint32_t lane = lane_id();
  for (uint64_t s0 = avail + 1; s0 <= tail; s0 += 64) {
    const uint64_t s = s0 + lane;
    if (s <= tail)
      a.dends[RING][slot_of(s, a.ends_mask)] = ld_rlx_sys(&a.hends[RING][slot_of(s, mask)]);
  }
  uint64_t end_tiles = 0;
  if (lane == 0) end_tiles = ld_rlx_sys(&a.hends[RING][slot_of(tail, mask)]);
  end_tiles = bcast64(end_tiles);
  fence_rel_agent();
  if (lane == 0) {
    st_rlx_agent(&a.dctl->ring[RING].avail_ops, tail);
    st_rel_agent(&a.dctl->ring[RING].avail_tiles, end_tiles);
  }
  avail = tail;
  return true;
}

template <int RING>
__device__ bool retire_ring(const KArgs& a, uint64_t avail, uint64_t& retired) {
  const uint32_t mask = a.cap_mask;
  const uint32_t lane = lane_id();
  bool moved = false;
  while (retired < avail) {
    const uint64_t s = retired + 1 + lane;
    bool done = true;
    if (s <= avail) done = ld_rlx_agent(&a.done_id[RING][slot_of(s, mask)]) >= s;
    const uint64_t notdone = ballot(!done);
    uint64_t adv = notdone ? (uint64_t)__builtin_ctzll(notdone) : 64;
    if (retired + adv > avail) adv = avail - retired;
    if (adv == 0) break;
    retired += adv;
    moved = true;
  }
  if (moved) {
    fence_acq_agent();
    if (lane == 0) {
      st_rel_agent(&a.dctl->ring[RING].retired, retired);
      st_rel_sys(&a.hctl->completed[RING], retired);
    }
  }
  return moved;
}

__device__ void doorbell_loop(const KArgs& a) {
  uint64_t avail0 = 0, avail1 = 0, ret0 = 0, ret1 = 0;
  uint64_t beats = 0;
  for (;;) {
    uint64_t t0 = 0, t1 = 0, stop = 0;
    if (lane_id() == 0) {
      t0 = ld_rlx_sys(&a.hctl->tail[0]);
      t1 = ld_rlx_sys(&a.hctl->tail[1]);
      stop = ld_rlx_sys(&a.hctl->stop_seq);
    }
    t0 = bcast64(t0);
    t1 = bcast64(t1);
    stop = bcast64(stop);
    fence_acq_sys();
    bool work = publish_ring<0>(a, t0, avail0);
    work |= publish_ring<1>(a, t1, avail1);
    work |= retire_ring<0>(a, avail0, ret0);
    work |= retire_ring<1>(a, avail1, ret1);
    ++beats;
    if ((beats & 1023) == 0 && lane_id() == 0) st_rlx_sys(&a.hctl->heartbeat, beats);
    if (stop && ret0 >= stop) {
      if (lane_id() == 0) {
        st_rel_agent(&a.dctl->stop, 1u);
        st_rel_sys(&a.hctl->heartbeat, beats);
      }
      return;
    }
    if (!work) __builtin_amdgcn_s_sleep(1);
  }
}

__global__ __launch_bounds__(256) void gpuos_resident(KArgs a) {
  const uint32_t wave = (blockIdx.x * blockDim.x + threadIdx.x) / 64;
  if (wave == 0)
    doorbell_loop(a);
  else
    worker_loop(a);
}

// ---------------------------------------------------------------------------
// per-op comparator: one launch per descriptor, every wave runs tiles
// wave, wave + waves, ... of that descriptor.

__global__ __launch_bounds__(256) void gpuos_single(DevDesc d, uint32_t* err) {
  const uint32_t wave = (blockIdx.x * blockDim.x + threadIdx.x) / 64;
  const uint32_t waves = gridDim.x * blockDim.x / 64;
  // same register layout as the resident kernel: lane i holds dword i
  const VDesc v{reinterpret_cast<const uint32_t*>(&d)[lane_id()]};
  const uint32_t ntiles = v(6);
  for (uint32_t t = wave; t < ntiles; t += waves) {
    const uint32_t e = exec_tile(v, t);
    if (e && lane_id() == 0 && err) *err = e;
  }
}

hipError_t launch_resident(const KArgs& a, uint32_t blocks, hipStream_t s) {
  hipLaunchKernelGGL(gpuos_resident, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_single(const DevDesc& d, uint32_t* err, hipStream_t s) {
  uint32_t waves = d.ntiles;
  uint32_t blocks = (waves + 3) / 4;
  if (blocks > 8192) blocks = 8192;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(gpuos_single, dim3(blocks), dim3(256), 0, s, d, err);
  return hipGetLastError();
}

const void* resident_kernel() { return reinterpret_cast<const void*>(&gpuos_resident); }

}  // namespace gpuos
