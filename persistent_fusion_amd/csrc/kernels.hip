// Resident scheduler kernel (gfx950).  The per-op comparator kernel is in
// single_kernel.hip: each kernel is its own translation unit so that the two
// large, fully inlined kernels compile in parallel.
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
//
// The same source also builds the run-time compiled variant of the kernel
// (GPUOS_RTC_VARIANT, compiled with hipRTC): its opcode switch is the one in
// rtc_exec.h, which adds program bodies compiled to straight-line code.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "gpuos_internal.h"
#include "tile_ops.h"
#ifdef GPUOS_RTC_VARIANT
#include "rtc_exec.h"
#else
#include "kernels.h"
#endif

namespace gpuos {

// Cache policies of tensor data in the resident kernel.  Results must be
// visible to waves on other XCDs once an op completes: stores write through
// to the device coherence point and loads read it (see device_common.h).
constexpr int kResidentLoadCP = CP_DEVICE;
constexpr int kResidentStoreCP = CP_DEVICE;
// Acquire: invalidate this XCD's L2 before a wave reads a new descriptor's
// inputs (needed only when loads use the default policy).
constexpr bool kAcquireInvalidate = false;
// Release: write back this XCD's L2 after each tile (needed only when stores
// use the default policy).
constexpr bool kReleaseWriteback = false;

// Descriptor as just loaded, one dword per lane (lane i keeps dword i).  Read
// with readlane only where every lane is active (right after the load);
// everything after that reads the wave's LDS copy.
struct VDesc {
  uint32_t v;
  __device__ __forceinline__ uint32_t operator()(int i) const {
    return (uint32_t)__builtin_amdgcn_readlane((int)v, i);
  }
  __device__ __forceinline__ uint64_t q(int i) const {
    return (uint64_t)(*this)(i) | ((uint64_t)(*this)(i + 1) << 32);
  }
};

// Per-wave cache of the descriptor the wave last worked on, per ring; the
// descriptor itself is in the wave's LDS slot for that ring.
struct Cached {
  uint64_t seq;    // 0 = none
  uint64_t start;  // first ticket
  uint64_t end;    // one past the last ticket
  lds_u32* slot;   // 64 dwords
  uint32_t deps_ok;
  lds_f32* scr;    // the wave's tile scratch (kWaveScratch floats)
  uint32_t rep;    // which copy of the completion words this wave polls
  __device__ __forceinline__ SDesc desc() const { return SDesc{slot}; }
};

__device__ __forceinline__ uint32_t slot_of(uint64_t seq, uint32_t mask) {
  return (uint32_t)((seq - 1) & mask);
}

__device__ __forceinline__ void report_error(const KArgs& a, uint32_t ring, uint64_t seq, uint64_t code) {
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
// picks the first probe past the ticket, and the range shrinks to the gap
// before it.  On a wide first round, lanes 0-31 probe the 32 sequences right
// after lo (where a wave's next ticket lies when the ops are large, so one
// round finds it exactly) and lanes 32-63 split the rest of the range.
//
// Probes stay inside (hi - C, hi], and no probed entry can be overwritten
// while the search runs: the ticket's own descriptor X (>= retired + 1, with
// hi <= retired + C at publication) cannot retire before this wave runs it, so
// the host can publish at most up to X - 1 + C < s + 2C for any probed s.
template <int RING>
__device__ __forceinline__ uint64_t find_seq(const KArgs& a, uint64_t ticket, uint64_t lo, uint64_t hi) {
  const uint32_t lane = lane_id();
  const uint32_t mask = a.cap_mask;
  if (hi > (uint64_t)mask + 1 && lo < hi - mask - 1) lo = hi - mask - 1;
  bool first = true;
  while (hi - lo > 1) {
    const uint64_t span = hi - lo;
    uint64_t s;
    if (first && span > 64) {
      const uint64_t step = (span - 32 + 31) / 32;
      s = lane < 32 ? lo + 1 + lane : lo + 32 + step * (lane - 31);
    } else {
      const uint64_t step = (span + 63) / 64;
      s = lo + step * (lane + 1);
    }
    if (s > hi) s = hi;  // probes are non-decreasing and the last one is hi
    const uint64_t e = ld_rlx_agent(&a.dends[RING][slot_of(s, a.ends_mask)]);
    const uint64_t past = ballot(e > ticket);
    // the probe at hi is always past the ticket, so `past` is non-empty; the
    // probe before the first past one is not past, hence strictly smaller
    const uint32_t f = (uint32_t)__builtin_ctzll(past);
    const uint64_t nhi = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(s >> 32), f) << 32) |
                         (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)s, f);
    uint64_t nlo = lo;
    if (f > 0)
      nlo = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(s >> 32), f - 1) << 32) |
            (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)s, f - 1);
    lo = nlo;
    hi = nhi;
    first = false;
  }
  return hi;
}

// Descriptors of at most this many tiles may be read from the pinned host
// ring before the doorbell wave has copied them; larger ones wait for the
// copy (so that one op's many waves never read it over the host link).
constexpr uint64_t kHostReadMaxTiles = 4;

// Loads descriptor `seq` (lane i gets dword i).  A descriptor the doorbell
// wave has already copied (seq <= `copied`) comes from the device ring: read
// through the caches first, and if that copy is the slot's previous occupant
// (recognised by the seq field in the first 128-byte line and the check word
// in the second) again from the device coherence point.  A newer small one
// comes straight from the pinned host ring, whose slot does not change before
// the descriptor retires; a newer large one is waited for.
// Makes descriptor `seq` (lane i holds dword i in dw) the wave's cached one.
__device__ __forceinline__ void install_desc(Cached& c, uint64_t seq, uint32_t dw) {
  const VDesc e{dw};
  c.slot[lane_id()] = dw;
  c.seq = seq;
  c.start = e.q(60);
  c.end = c.start + e(6);
  c.deps_ok = 0;
}

template <int RING>
__device__ __forceinline__ void fetch_desc(const KArgs& a, uint64_t seq, uint64_t copied,
                                           const AvailLine* line, Cached& c) {
  const uint32_t slot = slot_of(seq, a.cap_mask);
  const uint32_t off = 4u * lane_id();
  if (seq > copied) {
    uint64_t lo = 0, hi = 0;
    if (lane_id() == 0) {
      lo = ld_rlx_agent(&a.dends[RING][slot_of(seq - 1, a.ends_mask)]);
      hi = ld_rlx_agent(&a.dends[RING][slot_of(seq, a.ends_mask)]);
    }
    if (bcast64(hi) - bcast64(lo) > kHostReadMaxTiles) {
      while (seq > copied) {
        __builtin_amdgcn_s_sleep(1);
        uint64_t k = 0;
        if (lane_id() == 0) k = ld_rlx_agent(&line->copied_ops);
        copied = bcast64(k);
      }
    }
  }
  uint32_t dw;
  if (seq <= copied) {
    const rsrc_t r = make_rsrc(reinterpret_cast<uint64_t>(&a.ddesc[RING][slot]));
    dw = ld32<CP_DEFAULT>(r, off);
    const VDesc d{dw};
    if (d.q(4) != seq || d(63) != ((uint32_t)seq ^ kDescMagic)) {
      dw = ld32<CP_DEVICE>(r, off);
      const VDesc f{dw};
      if (f.q(4) != seq || f(63) != ((uint32_t)seq ^ kDescMagic)) report_error(a, RING, seq, DERR_DESC_CHECK);
    }
  } else {
    const rsrc_t r = make_rsrc(reinterpret_cast<uint64_t>(&a.hdesc[RING][slot]));
    dw = ld32<CP_SYSTEM>(r, off);
    const VDesc f{dw};
    if (f.q(4) != seq || f(63) != ((uint32_t)seq ^ kDescMagic)) report_error(a, RING, seq, DERR_DESC_CHECK);
  }
  install_desc(c, seq, dw);
}

// Waits until every dependency of the cached descriptor has completed.
// Polls are device-scope loads (coherent without invalidating L2); tensor data
// is read with device-coherent loads, so no acquire fence is needed after.
template <int RING>
__device__ __forceinline__ void wait_deps(const KArgs& a, const Cached& c) {
  const SDesc d = c.desc();
  const uint32_t mask = a.cap_mask;
  for (int i = 0; i < kMaxDeps; ++i) {
    const uint32_t delta = d(i < 8 ? 8 + i : 54 + (i - 8));
    if (delta) {
      const uint64_t dep = c.seq - delta;
      const uint64_t* w = &a.done_id[RING][(uint64_t)c.rep * (mask + 1) + slot_of(dep, mask)];
      while (bcast64(ld_rlx_agent(w)) < dep) __builtin_amdgcn_s_sleep(1);
    }
  }
  const uint64_t wr = d.q(16);
  if (wr) {
    while (bcast64(ld_rlx_agent(&a.dctl->ring[RING].retired)) < wr) __builtin_amdgcn_s_sleep(2);
  }
  if constexpr (kAcquireInvalidate) fence_acq_agent();
  compiler_fence();
}

// Counts one tile done; the wave completing the descriptor publishes
// done_id for dependents and the doorbell wave.  The tile's stores are
// device-coherent write-through stores, so waiting for their acknowledgement
// makes them visible on every XCD before the count moves (no L2 writeback).
template <int RING>
__device__ __forceinline__ void finish_tile(const KArgs& a, const Cached& c, uint32_t tile,
                                            uint64_t ticket) {
  const uint32_t slot = slot_of(c.seq, a.cap_mask);
  const uint32_t cap = a.cap_mask + 1;
  const SDesc d = c.desc();
  const uint32_t ntiles = d(6);
  if ((a.debug & kDebugCount) && lane_id() == 0) {
    uint32_t* cnt = a.dctl->tile_exec[RING];
    if (ticket < a.dctl->tile_exec_n)
      __hip_atomic_fetch_add(&cnt[ticket], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if constexpr (kReleaseWriteback) fence_rel_agent();
  const bool traced = a.trace[RING] != nullptr;
  const uint64_t t_end = traced ? now_ticks() : 0;
  wait_mem();
  const uint64_t t_ack = traced ? now_ticks() : 0;
  if (lane_id() != 0) return;
  bool complete;
  const uint32_t S = ntiles <= kTilesPerSub ? 1u
                     : ((ntiles + kTilesPerSub - 1) / kTilesPerSub < kSubCounters
                            ? (ntiles + kTilesPerSub - 1) / kTilesPerSub : kSubCounters);
  if (ntiles == 1) {
    complete = true;  // the only tile: no count needed
  } else if (S == 1) {
    uint32_t* ctr = &a.tiles_done[RING][slot];
    const uint32_t old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    complete = old + 1 == ntiles;
    if (complete) st_rlx_agent(ctr, 0u);
  } else {
    const uint32_t sub = tile % S;
    const uint32_t need = ntiles / S + (sub < ntiles % S ? 1u : 0u);
    uint32_t* ctr = &a.tiles_done[RING][sub * cap + slot];
    const uint32_t old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    complete = false;
    if (old + 1 == need) {
      st_rlx_agent(ctr, 0u);
      uint32_t* top = &a.subs_done[RING][slot];
      const uint32_t o2 = __hip_atomic_fetch_add(top, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      complete = o2 + 1 == S;
      if (complete) st_rlx_agent(top, 0u);
    }
  }
  if (complete) {
    // every tile's stores were acknowledged before its count: publish at once
    const uint64_t t_done = now_ticks();
#pragma unroll
    for (uint32_t k = 0; k < kDoneReplicas; ++k) st_rlx_agent(&a.done_id[RING][(uint64_t)k * cap + slot], c.seq);
    if constexpr (RING == 1) st_rlx_sys(&a.dctl->hdone_lc[slot], c.seq);
    if (traced) {
      TraceRec* tr = &a.trace[RING][slot];
      st_rlx_agent(&tr->seq, c.seq);
      st_rlx_agent(&tr->t_done, t_done);
      st_rlx_agent(&tr->t_end, t_end);
      st_rlx_agent(&tr->t_ack, t_ack);
      st_rlx_agent(&tr->opcode, d(0) & 0xffu);
      st_rlx_agent(&tr->ntiles, ntiles);
    }
  }
}

// Debug schedule jitter: waits a pseudo-random 0..max steps of s_sleep 4
// (256 clocks, about 0.1 us), the count drawn from a hash of the ticket
// (splitmix64 finaliser), so that tiles start and finish in another order.
__device__ __forceinline__ void jitter_wait(uint64_t ticket, uint32_t max) {
  uint64_t h = ticket + 0x9E3779B97F4A7C15ull;
  h = (h ^ (h >> 30)) * 0xBF58476D1CE4E5B9ull;
  h = (h ^ (h >> 27)) * 0x94D049BB133111EBull;
  h ^= h >> 31;
  const uint32_t n = (uint32_t)(h % ((uint64_t)max + 1));
  for (uint32_t i = 0; i < n; ++i) __builtin_amdgcn_s_sleep(4);
}

template <int RING>
__device__ __forceinline__ void run_ticket(const KArgs& a, uint64_t ticket, Cached& c) {
  const uint32_t tile = (uint32_t)(ticket - c.start);
  const SDesc d = c.desc();
  if (a.debug >> 16) jitter_wait(ticket, a.debug >> 16);
  auto stamp = [&](uint64_t TraceRec::*field) {
    if (a.trace[RING] && tile == 0 && lane_id() == 0)
      st_rlx_agent(&(a.trace[RING][slot_of(c.seq, a.cap_mask)].*field), now_ticks());
  };
  auto claimed = [&]() { stamp(&TraceRec::t_claim); };
  if (!c.deps_ok) {
#ifndef GPUOS_RTC_VARIANT
    const uint32_t w0 = d(0);
    const uint32_t op = w0 & 0xffu;
    if ((op == GPUOS_OP_GEMV || op == OP_NORM_GEMV || op == OP_GEMV_ADD) &&
        ((w0 >> 16) & DF_AUX_READY)) {
      // the weights are final: start streaming them, then wait for x
      auto ready = [&]() {
        stamp(&TraceRec::t_wait);
        wait_deps<RING>(a, c);
        c.deps_ok = 1;
        claimed();
      };
      const bool bf = ((w0 >> 8) & 0xffu) == GPUOS_BF16;
      if (op == OP_NORM_GEMV && bf)
        norm_gemv_tile<kResidentLoadCP, kResidentStoreCP>(d, tile, ready);
      else if (op == GPUOS_OP_GEMV && bf)
        gemv_tile<GPUOS_BF16, kResidentLoadCP, kResidentStoreCP>(d, tile, ready);
      else if (op == GPUOS_OP_GEMV)
        gemv_tile<GPUOS_F32, kResidentLoadCP, kResidentStoreCP>(d, tile, ready);
      else if (op == OP_GEMV_ADD && bf)
        gemv_tile<GPUOS_BF16, kResidentLoadCP, kResidentStoreCP>(d, tile, ready, true);
      else if (op == OP_GEMV_ADD)
        gemv_tile<GPUOS_F32, kResidentLoadCP, kResidentStoreCP>(d, tile, ready, true);
      else
        report_error(a, RING, c.seq, DERR_BAD_OPCODE);
      finish_tile<RING>(a, c, tile, ticket);
      return;
    }
#endif
    stamp(&TraceRec::t_wait);
    wait_deps<RING>(a, c);
    c.deps_ok = 1;
  }
  claimed();
#ifdef GPUOS_RTC_VARIANT
  const uint32_t err = exec_rtc<kResidentLoadCP, kResidentStoreCP>(d, tile);
#else
  const uint32_t err = exec_tile<kResidentLoadCP, kResidentStoreCP>(d, tile, c.scr);
#endif
  if (err) report_error(a, RING, c.seq, err);
  finish_tile<RING>(a, c, tile, ticket);
}

// Maps a runnable ticket to its descriptor (refreshing the cache if needed).
template <int RING>
__device__ __forceinline__ void map_ticket(const KArgs& a, uint64_t ticket, uint64_t avail_ops,
                                           uint64_t copied, const AvailLine* line, Cached& c) {
  if (c.seq != 0 && ticket < c.end) return;
  // When ops are large the next descriptor usually owns the ticket: its copy
  // in the device ring is requested before the search, so both share one
  // round trip.  It is used only if the search agrees and it is the current
  // occupant of its slot (seq field and check word).
  const uint64_t nx = c.seq + 1;
  const bool spec = c.seq != 0 && nx <= copied && nx <= avail_ops;
  uint32_t sdw = 0;
  if (spec) {
    const rsrc_t r = make_rsrc(reinterpret_cast<uint64_t>(&a.ddesc[RING][slot_of(nx, a.cap_mask)]));
    sdw = ld32<CP_DEFAULT>(r, 4u * lane_id());
  }
  const uint64_t seq = find_seq<RING>(a, ticket, c.seq, avail_ops);
  if (spec && seq == nx) {
    const VDesc d{sdw};
    if (d.q(4) == nx && d(63) == ((uint32_t)nx ^ kDescMagic)) {
      install_desc(c, nx, sdw);
      return;
    }
  }
  fetch_desc<RING>(a, seq, copied, line, c);
}

// Reads a ring's published-work replica: avail_tiles first, then (after the
// first load has returned) avail_ops, which was stored before it, and the
// copied frontier (any value it held is a valid lower bound).
__device__ __forceinline__ void read_avail(const AvailLine* l, uint64_t& tiles, uint64_t& ops,
                                           uint64_t& copied) {
  uint64_t t = 0, o = 0, k = 0;
  if (lane_id() == 0) {
    t = ld_rlx_agent(&l->avail_tiles);
    wait_mem();
    o = ld_rlx_agent(&l->avail_ops);
    k = ld_rlx_agent(&l->copied_ops);
  }
  tiles = bcast64(t);
  ops = bcast64(o);
  copied = bcast64(k);
}

// Latency-critical ring: served only by the reserved waves, which take its
// descriptors straight from the host: a wave reads the host's ring tail
// (pinned memory; the copy on its own line, so that these polls stay off the
// line the host writes at every flush) and the claim cursor in one round trip, claims the next
// descriptor with one compare-and-swap, reading it from the pinned host ring
// in the same round trip (its slot does not change before it retires), and
// runs all its tiles
// itself (the host plans small latency-critical ops as one tile).  The
// doorbell wave still publishes and retires the ring in order, but is not on
// this path.  Drains the ring.
__device__ __forceinline__ bool service_lc(const KArgs& a, Cached& c) {
  DevRing* R = &a.dctl->ring[1];
  bool work = false;
  for (;;) {
    uint64_t tail = 0, nxt = 0;
    if (lane_id() == 0) {
      tail = ld_rlx_sys(&a.hctl->lc_tail);
      nxt = ld_rlx_agent(&R->next);
    }
    tail = bcast64(tail);
    nxt = bcast64(nxt);
    if (nxt >= tail) return work;
    // the descriptor is read in the same round trip as the claim (the host
    // stored it before the tail this wave has read); it is used only if the
    // claim succeeds
    const uint64_t seq = nxt + 1;
    const rsrc_t r = make_rsrc(reinterpret_cast<uint64_t>(&a.hdesc[1][slot_of(seq, a.cap_mask)]));
    const uint32_t dw = ld32<CP_SYSTEM>(r, 4u * lane_id());
    uint32_t ok = 0;
    if (lane_id() == 0) {
      uint64_t expect = nxt;
      ok = __hip_atomic_compare_exchange_strong(&R->next, &expect, nxt + 1, __ATOMIC_RELAXED,
                                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
               ? 1u
               : 0u;
    }
    if (!bcast(ok)) continue;
    const VDesc f{dw};
    if (f.q(4) != seq || f(63) != ((uint32_t)seq ^ kDescMagic)) report_error(a, 1, seq, DERR_DESC_CHECK);
    install_desc(c, seq, dw);
    for (uint64_t t = c.start; t < c.end; ++t) run_ticket<1>(a, t, c);
    work = true;
  }
}

// A reserved wave: serves the latency-critical ring until the launch ends
// (at which point every published descriptor has retired).  It takes no
// descriptor before the whole grid has checked in.  It polls back to back
// for 16 polls (about 30 us) after it last found work, then about every
// 3.5 us: eight waves polling host memory without pause slowed the
// best-effort waves' dependency chains by 13%, and while latency-critical ops
// keep coming the waves stay in the fast mode.
__device__ __forceinline__ void lc_loop(const KArgs& a, uint32_t w, lds_u32* slot1, lds_f32* scr) {
  const AvailLine* line0 = &a.dctl->avail[0][w % kReplicas];
  Cached c1{0, 0, 0, slot1, 0, scr, w % kDoneReplicas};
  const uint64_t want = (uint64_t)a.epoch * gridDim.x * 4u;
  for (;;) {
    uint64_t got = 0, se = 0;
    if (lane_id() == 0) {
      got = ld_rlx_agent(&a.dctl->arrived);
      se = ld_rlx_agent(&line0->stop_epoch);
    }
    if (bcast64(got) >= want) break;
    if (bcast64(se) == a.epoch) return;
    __builtin_amdgcn_s_sleep(8);
  }
  uint32_t idle = 0;
  for (;;) {
    if (service_lc(a, c1)) idle = 0;
    else if (idle < 16) ++idle;
    uint64_t se = 0;
    if (lane_id() == 0) se = ld_rlx_agent(&line0->stop_epoch);
    if (bcast64(se) == a.epoch) return;
    if (idle < 16) __builtin_amdgcn_s_sleep(1);
    else __builtin_amdgcn_s_sleep(127);
  }
}

// A best-effort wave: runs its round-robin share of the ring-0 tickets.
__device__ __forceinline__ void worker_loop(const KArgs& a, uint32_t w, lds_u32* slot0, lds_f32* scr) {
  const AvailLine* line0 = &a.dctl->avail[0][w % kReplicas];
  Cached c0{0, 0, 0, slot0, 0, scr, w % kDoneReplicas};
  uint64_t avail = 0, avail_ops = 0, copied = 0;
  uint32_t idle = 0;
  // tickets are dealt round-robin: this wave owns those = w (mod workers),
  // from the first one this launch has not inherited as done
  const uint64_t base = a.ticket_base;
  uint64_t ticket = base - base % a.workers + w;
  if (ticket < base) ticket += a.workers;
  for (;;) {
    if (ticket >= avail) {
      if (idle > 0) {
        // idle: watch avail_tiles alone until it moves past this ticket
        uint64_t t = 0;
        if (lane_id() == 0) t = ld_rlx_agent(&line0->avail_tiles);
        if (bcast64(t) > ticket) read_avail(line0, avail, avail_ops, copied);
      } else {
        read_avail(line0, avail, avail_ops, copied);
      }
      if (ticket >= avail) {
        if (idle >= 32 || (idle & 7) == 7) {
          uint64_t se = 0, stop = 0;
          if (lane_id() == 0) {
            se = ld_rlx_agent(&line0->stop_epoch);
            wait_mem();
            stop = ld_rlx_agent(&line0->stop_ticket);
          }
          if (bcast64(se) == a.epoch && ticket >= bcast64(stop)) return;
        }
        // nothing published for this ticket yet: back off, further the
        // longer the queue stays empty (about 0.03, 0.6, then 3.5 us)
        if (idle < 32) {
          __builtin_amdgcn_s_sleep(2);
        } else if (idle < 4096) {
          __builtin_amdgcn_s_sleep(20);
        } else {
          __builtin_amdgcn_s_sleep(127);
        }
        if (idle < 4096) ++idle;
        continue;
      }
    }
    idle = 0;
    map_ticket<0>(a, ticket, avail_ops, copied, line0, c0);
    run_ticket<0>(a, ticket, c0);
    ticket += a.workers;
  }
}

// ---------------------------------------------------------------------------
// doorbell / tracker wave

// Publishes the ticket ranges of descriptors (avail, tail]: their ends are
// copied from the pinned host ring into the device ring of ends (8 loads of
// 8 bytes per lane in flight, 512 descriptors per round trip over the host
// link), then every replica gets avail_ops and, after it, avail_tiles.
template <int RING>
__device__ __forceinline__ bool publish_ends(const KArgs& a, uint64_t tail, uint64_t& avail,
                                             uint64_t& avail_tiles) {
  if (tail <= avail) return false;
  const uint32_t mask = a.cap_mask;
  const uint32_t lane = lane_id();
  constexpr int B = 8;
  uint64_t last = 0;
  for (uint64_t s0 = avail + 1; s0 <= tail; s0 += 64 * B) {
    uint64_t e[B];
#pragma unroll
    for (int k = 0; k < B; ++k) {
      const uint64_t s = s0 + 64 * k + lane;
      e[k] = s <= tail ? ld_rlx_sys(&a.hends[RING][slot_of(s, mask)]) : 0;
    }
#pragma unroll
    for (int k = 0; k < B; ++k) {
      const uint64_t s = s0 + 64 * k + lane;
      if (s <= tail) st_rlx_agent(&a.dends[RING][slot_of(s, a.ends_mask)], e[k]);
      if (s == tail) last = e[k];
    }
  }
  // the lane that loaded ends(tail) shares it
  const uint64_t holder = ballot((tail - avail - 1) % 64 == lane);
  const uint32_t src = (uint32_t)__builtin_ctzll(holder);
  const uint64_t end_tiles = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)last, src) |
                             ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(last >> 32), src) << 32);
  wait_mem();
  // every replica: avail_ops, then avail_tiles (one replica per lane)
  if (lane < kReplicas) st_rlx_agent(&a.dctl->avail[RING][lane].avail_ops, tail);
  wait_mem();
  if (lane < kReplicas) st_rlx_agent(&a.dctl->avail[RING][lane].avail_tiles, end_tiles);
  avail = tail;
  avail_tiles = end_tiles;
  return true;
}

// Copies the next (at most kCopyChunk) published descriptors into the device
// ring: every 16-byte system-scope load of the chunk (four descriptors per
// wave-wide load) is issued before the first store; the stores write
// through to the device coherence point, and once they are acknowledged the
// copied frontier moves.  Retired descriptors are never copied.
constexpr uint32_t kCopyChunk = 64;

template <int RING>
__device__ __forceinline__ bool copy_some(const KArgs& a, uint64_t avail, uint64_t retired,
                                          uint64_t& copied) {
  if (copied < retired) copied = retired;
  if (copied >= avail) return false;
  const uint64_t from = copied;
  const uint64_t to = avail - from > kCopyChunk ? from + kCopyChunk : avail;
  constexpr int G = kCopyChunk / 4;  // wave-wide loads of 4 descriptors
  const uint32_t mask = a.cap_mask;
  const uint32_t lane = lane_id();
  const rsrc_t hr = make_rsrc(reinterpret_cast<uint64_t>(a.hdesc[RING]));
  const rsrc_t dr = make_rsrc(reinterpret_cast<uint64_t>(a.ddesc[RING]));
  const uint32_t sub = lane / 16, part = lane % 16;  // descriptor in group, 16-byte part
  u32x4 v[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint64_t s = from + 1 + 4 * g + sub;
    if (s <= to) v[g] = ld128<CP_SYSTEM>(hr, slot_of(s, mask) * kDescBytes + 16u * part);
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint64_t s = from + 1 + 4 * g + sub;
    if (s <= to) st128<CP_DEVICE>(dr, slot_of(s, mask) * kDescBytes + 16u * part, v[g]);
  }
  wait_mem();
  if (lane < kReplicas) st_rlx_agent(&a.dctl->avail[RING][lane].copied_ops, to);
  copied = to;
  return true;
}

template <int RING>
__device__ __forceinline__ bool retire_ring(const KArgs& a, uint64_t avail, uint64_t& retired) {
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
  if (moved && lane == 0) {
    st_rlx_agent(&a.dctl->ring[RING].retired, retired);
    st_rlx_sys(&a.hctl->completed[RING], retired);
  }
  return moved;
}

// Releases the workers (every ticket below `tiles0` has run) and reports the
// exit to the host.
__device__ __forceinline__ void release_workers(const KArgs& a, uint64_t tiles0) {
  const uint32_t lane = lane_id();
  if (lane < kReplicas) st_rlx_agent(&a.dctl->avail[0][lane].stop_ticket, tiles0);
  wait_mem();
  if (lane < kReplicas) st_rlx_agent(&a.dctl->avail[0][lane].stop_epoch, (uint64_t)a.epoch);
  if (lane == 0) st_rlx_sys(&a.hctl->exit_tiles, tiles0);
  wait_mem();
  if (lane == 0) st_rlx_sys(&a.hctl->exit_epoch, (uint64_t)a.epoch);
  wait_mem();
}

// Co-residency check: every wave of the grid counts itself in at start, and
// the doorbell wave publishes no work before the whole grid has arrived.  A
// worker only ever waits for tiles with smaller tickets, which resident waves
// hold, so once every wave is resident each wait ends; a grid that cannot be
// resident at once (another kernel holding compute units) takes no work, and
// the host sees no resident_epoch for this launch.  A stop request ends the
// wait.  Returns false when stopped before the grid was complete.
__device__ __forceinline__ bool await_grid(const KArgs& a) {
  const uint64_t want = (uint64_t)a.epoch * gridDim.x * 4u;
  for (;;) {
    uint64_t got = 0, stop = 0;
    if (lane_id() == 0) {
      got = ld_rlx_agent(&a.dctl->arrived);
      stop = ld_rlx_sys(&a.hctl->stop_req);
    }
    if (bcast64(got) >= want) break;
    if (bcast64(stop)) return false;
    __builtin_amdgcn_s_sleep(8);
  }
  if (lane_id() == 0) st_rel_sys(&a.hctl->resident_epoch, (uint64_t)a.epoch);
  return true;
}

__device__ __forceinline__ void doorbell_loop(const KArgs& a) {
  if (!await_grid(a)) {
    // stopped before the grid was resident: release whatever waves run
    uint64_t t0 = 0;
    if (lane_id() == 0) t0 = ld_rlx_agent(&a.dctl->avail[0][0].avail_tiles);
    release_workers(a, bcast64(t0));
    return;
  }
  // resume from what earlier launches published and retired
  uint64_t avail0 = 0, avail1 = 0, ret0 = 0, ret1 = 0, tiles0 = 0, tiles1 = 0, cp0 = 0, cp1 = 0;
  if (lane_id() == 0) {
    avail0 = ld_rlx_agent(&a.dctl->avail[0][0].avail_ops);
    avail1 = ld_rlx_agent(&a.dctl->avail[1][0].avail_ops);
    tiles0 = ld_rlx_agent(&a.dctl->avail[0][0].avail_tiles);
    tiles1 = ld_rlx_agent(&a.dctl->avail[1][0].avail_tiles);
    cp0 = ld_rlx_agent(&a.dctl->avail[0][0].copied_ops);
    cp1 = ld_rlx_agent(&a.dctl->avail[1][0].copied_ops);
    ret0 = ld_rlx_agent(&a.dctl->ring[0].retired);
    ret1 = ld_rlx_agent(&a.dctl->ring[1].retired);
  }
  avail0 = bcast64(avail0); avail1 = bcast64(avail1);
  tiles0 = bcast64(tiles0); tiles1 = bcast64(tiles1);
  cp0 = bcast64(cp0); cp1 = bcast64(cp1);
  ret0 = bcast64(ret0); ret1 = bcast64(ret1);
  uint64_t beats = 0;
  uint64_t last_work = now_ticks();
  for (;;) {
    uint64_t t0 = 0, t1 = 0, stop = 0;
    if (lane_id() == 0) {
      t0 = ld_rlx_sys(&a.hctl->tail[0]);
      t1 = ld_rlx_sys(&a.hctl->tail[1]);
      stop = ld_rlx_sys(&a.hctl->stop_req);
    }
    t0 = bcast64(t0);
    t1 = bcast64(t1);
    stop = bcast64(stop);
    compiler_fence();
    // ticket ranges first (cheap), then one chunk of descriptor copies
    bool work = publish_ends<1>(a, t1, avail1, tiles1);
    work |= publish_ends<0>(a, t0, avail0, tiles0);
    work |= copy_some<1>(a, avail1, ret1, cp1);
    work |= copy_some<0>(a, avail0, ret0, cp0);
    work |= retire_ring<0>(a, avail0, ret0);
    work |= retire_ring<1>(a, avail1, ret1);
    ++beats;
    if ((beats & 1023) == 0 && lane_id() == 0) st_rlx_sys(&a.hctl->heartbeat, beats);
    const bool drained = ret0 == t0 && ret1 == t1 && avail0 == t0 && avail1 == t1;
    if (work) last_work = now_ticks();
    if (drained && stop) {
      // every published descriptor has retired: release the workers
      if (lane_id() == 0) st_rlx_sys(&a.hctl->heartbeat, beats);
      release_workers(a, tiles0);
      return;
    }
    bool yield = false;  // the host asks the kernel to give the GPU back now
    if (drained) {
      uint64_t y = 0;
      if (lane_id() == 0) y = ld_rlx_sys(&a.hctl->yield_req);
      yield = bcast64(y) != 0;
    }
    if (drained && (yield || (a.idle_exit_ticks && now_ticks() - last_work > a.idle_exit_ticks))) {
      // idle for too long: announce the exit, then look at the tails again.
      // The re-read cannot overtake the announcement on its way to host
      // memory, and the host reads the announcement after storing a tail, so
      // either the host sees the announcement (and relaunches after the exit)
      // or this wave sees the new tail (and cancels).
      uint64_t n0 = 0, n1 = 0;
      if (lane_id() == 0) {
        st_rlx_sys(&a.hctl->exit_req, (uint64_t)a.epoch);
        wait_mem();
        n0 = ld_rlx_sys(&a.hctl->tail[0]);
        n1 = ld_rlx_sys(&a.hctl->tail[1]);
      }
      n0 = bcast64(n0);
      n1 = bcast64(n1);
      if (n0 == t0 && n1 == t1) {
        if (lane_id() == 0) st_rlx_sys(&a.hctl->heartbeat, beats);
        release_workers(a, tiles0);
        return;
      }
      if (lane_id() == 0) st_rlx_sys(&a.hctl->exit_req, (uint64_t)0);
      wait_mem();
      last_work = now_ticks();
      continue;
    }
    if (!work) __builtin_amdgcn_s_sleep(1);
  }
}

__device__ __forceinline__ void resident_main(const KArgs& a) {
  // one descriptor slot per wave and ring, and each wave's tile scratch
  __shared__ uint32_t sdesc[4][2][64];
  __shared__ float sscr[4][kWaveScratch];
  // Waves are numbered across workgroups first (wave j of workgroup b is
  // j * blocks + b), so consecutive tickets, dealt round-robin, land on
  // different CUs and XCDs (workgroups are dispatched round-robin over the
  // XCDs).  Number 0 is the doorbell wave; the next lc_waves (one per XCD for
  // up to 8) serve the latency-critical ring; the rest run best-effort tiles.
  const uint32_t wib = threadIdx.x / 64;
  const uint32_t num = wib * gridDim.x + blockIdx.x;
  if (lane_id() == 0)
    __hip_atomic_fetch_add(&a.dctl->arrived, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (num == 0)
    doorbell_loop(a);
  else if (num - 1 < a.lc_waves)
    lc_loop(a, num - 1, (lds_u32*)&sdesc[wib][1][0], (lds_f32*)&sscr[wib][0]);
  else
    worker_loop(a, num - 1 - a.lc_waves, (lds_u32*)&sdesc[wib][0][0], (lds_f32*)&sscr[wib][0]);
}

}  // namespace gpuos

#ifdef GPUOS_RTC_VARIANT
// Entry point of the compiled variant, found by name in the loaded module.
extern "C" __global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gpuos_resident_rtc(gpuos::KArgs a) {
  gpuos::resident_main(a);
}
#else
namespace gpuos {

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gpuos_resident(KArgs a) {
  resident_main(a);
}

hipError_t launch_resident(const KArgs& a, uint32_t blocks, hipStream_t s) {
  hipLaunchKernelGGL(gpuos_resident, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

const void* resident_kernel() { return reinterpret_cast<const void*>(&gpuos_resident); }

}  // namespace gpuos
#endif
