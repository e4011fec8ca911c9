// Host consumer: drives the host half of the gpuos runtime under concurrency.
//
// A producer thread submits and flushes a queue of int32 ADD / MUL / COPY ops
// over overlapping ranges of a few buffers into a host-only context with a
// small ring.  A consumer thread plays the resident kernel on the same ring
// protocol: it follows the published tails, reads descriptors from their ring
// slots, runs any descriptor whose published dependencies have run (chosen at
// random among the ready ones, so independent descriptors run out of order,
// as the device's waves may), and advances each ring's in-order retire
// cursor.  The ring fills and wraps, so the producer blocks on back-pressure,
// and latency-critical ops go to the second ring.  The buffers are host
// memory: a host-only context never dereferences the pointers it is given.
//
// Built with the sanitizers (address + undefined, or thread) by the test that
// runs it; the final buffers are compared with the oracle's program-order run
// of the same queue.
//
// usage: host_consumer OPS INIT OUT SLOTS BATCH FLUSH_EVERY SEED [AUTO_DEPS]
//   OPS    text: "buffers B L", then one line per op:
//          "op KIND LC OUTB OUTOFF IN0B IN0OFF IN1B IN1OFF N" (KIND 0 add,
//          1 mul, 2 copy; IN1 ignored by copy)
//   INIT   B*L int32, little endian (initial buffer contents)
//   OUT    written: B*L int32 (final buffer contents)
//   AUTO_DEPS  config.auto_deps (default 1: hazard dependencies on; 2 turns
//          them off, which the test uses to show that the comparison fails
//          when the runtime orders nothing)
// Prints one line of counters and exits 0, or prints the failure and exits 1.

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cinttypes>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <thread>
#include <vector>

#include "../../include/gpuos.h"
#include "../../include/gpuos_debug.h"
#include "../../persistent_fusion_amd/csrc/gpuos_internal.h"

namespace {

struct HostOp {
  int kind, lc;
  int ob, ib0, ib1;
  uint32_t oo, io0, io1, n;
};

[[noreturn]] void die(const char* what, int rc = 0) {
  std::fprintf(stderr, "host_consumer: %s (rc %d: %s)\n", what, rc, gpuos_last_error());
  std::exit(1);
}

std::atomic<bool> producer_done{false};
std::atomic<bool> consumer_failed{false};

struct Pending {
  gpuos::DevDesc d;
  bool ran = false;
};

struct Counters {
  uint64_t ran[gpuos::kRings] = {0, 0};
  uint64_t out_of_order = 0;   // descriptors run while an earlier one waited
  uint64_t max_ready = 0;      // most descriptors ready at once
  uint64_t deps_seen = 0;
};

void run_desc(const gpuos::DevDesc& d) {
  int32_t* out = reinterpret_cast<int32_t*>(d.p.ptr[0]);
  const int32_t* a = reinterpret_cast<const int32_t*>(d.p.ptr[1]);
  const int32_t* b = reinterpret_cast<const int32_t*>(d.p.ptr[2]);
  for (uint32_t i = 0; i < d.n; ++i) {
    const uint32_t x = (uint32_t)a[i];
    uint32_t v;
    if (d.opcode == GPUOS_OP_ADD) v = x + (uint32_t)b[i];
    else if (d.opcode == GPUOS_OP_MUL) v = x * (uint32_t)b[i];
    else v = x;
    out[i] = (int32_t)v;
  }
}

void consumer(gpuos_ctx* ctx, uint32_t cap, uint64_t seed, Counters* cnt) {
  std::mt19937_64 rng(seed);
  // per ring: descriptors read but not yet retired, indexed by seq - retired - 1
  std::vector<Pending> win[gpuos::kRings];
  uint64_t retired[gpuos::kRings] = {0, 0};
  uint64_t seen[gpuos::kRings] = {0, 0};
  uint32_t idle = 0;
  // let the producer fill the ring first, so that it has to wait for ring
  // space at least once whatever the two threads' speeds (after 200 ms the
  // consumer starts anyway: the producer may be waiting on the host for a
  // cross-ring dependency, which only this thread can end)
  const auto t0 = std::chrono::steady_clock::now();
  while (!producer_done.load() && gpuos_debug_consumer_tail(ctx, 0) < cap &&
         std::chrono::steady_clock::now() - t0 < std::chrono::milliseconds(200))
    std::this_thread::sleep_for(std::chrono::microseconds(100));
  for (;;) {
    bool progress = false;
    for (int r = 0; r < gpuos::kRings; ++r) {
      const uint64_t tail = gpuos_debug_consumer_tail(ctx, r);
      if (tail < seen[r] || tail - retired[r] > cap) {
        std::fprintf(stderr, "ring %d: tail %" PRIu64 " with %" PRIu64 " retired, %u slots\n", r,
                     tail, retired[r], cap);
        consumer_failed = true;
        return;
      }
      for (uint64_t s = seen[r] + 1; s <= tail; ++s) {
        Pending p;
        const int rc = gpuos_debug_consumer_read(ctx, r, s, &p.d);
        if (rc) {
          std::fprintf(stderr, "ring %d seq %" PRIu64 ": %s\n", r, s, gpuos_last_error());
          consumer_failed = true;
          return;
        }
        const uint8_t op = p.d.opcode;
        if ((op != GPUOS_OP_ADD && op != GPUOS_OP_MUL && op != GPUOS_OP_COPY) ||
            p.d.dtype != GPUOS_I32 || p.d.n == 0) {
          std::fprintf(stderr, "ring %d seq %" PRIu64 ": unexpected opcode %u dtype %u n %u\n", r,
                       s, op, p.d.dtype, p.d.n);
          consumer_failed = true;
          return;
        }
        win[r].push_back(p);
      }
      seen[r] = tail;
      // ready: every published dependency has run
      std::vector<size_t> ready;
      for (size_t k = 0; k < win[r].size(); ++k) {
        const Pending& p = win[r][k];
        if (p.ran) continue;
        const uint64_t s = retired[r] + 1 + k;
        bool ok = p.d.wait_retired <= retired[r] || p.d.wait_retired == 0;
        for (int j = 0; j < gpuos::kMaxDeps && ok; ++j) {
          const uint32_t delta = j < 8 ? p.d.deps_lo[j] : p.d.deps_hi[j - 8];
          if (!delta) continue;
          if (delta >= s) {
            std::fprintf(stderr, "ring %d seq %" PRIu64 ": dependency delta %u\n", r, s, delta);
            consumer_failed = true;
            return;
          }
          const uint64_t dep = s - delta;
          if (dep > retired[r] && !win[r][dep - retired[r] - 1].ran) ok = false;
        }
        if (ok) ready.push_back(k);
      }
      if (ready.empty()) continue;
      if (ready.size() > cnt->max_ready) cnt->max_ready = ready.size();
      // run a random half of the ready descriptors (at least one), in random order
      std::shuffle(ready.begin(), ready.end(), rng);
      const size_t take = 1 + rng() % ready.size();
      for (size_t t = 0; t < take; ++t) {
        Pending& p = win[r][ready[t]];
        for (int j = 0; j < gpuos::kMaxDeps; ++j)
          cnt->deps_seen += (j < 8 ? p.d.deps_lo[j] : p.d.deps_hi[j - 8]) != 0;
        run_desc(p.d);
        p.ran = true;
        ++cnt->ran[r];
        if (ready[t] != 0 && !win[r][0].ran) ++cnt->out_of_order;
      }
      size_t k = 0;
      while (k < win[r].size() && win[r][k].ran) ++k;
      if (k) {
        win[r].erase(win[r].begin(), win[r].begin() + k);
        retired[r] += k;
        const int rc = gpuos_debug_consumer_retire(ctx, r, retired[r]);
        if (rc) {
          std::fprintf(stderr, "retire: %s\n", gpuos_last_error());
          consumer_failed = true;
          return;
        }
      }
      progress = true;
    }
    if (progress) {
      // a device slower than the host: the producer runs ahead, so the ring
      // fills and descriptors accumulate with their dependencies pending
      idle = 0;
      std::this_thread::sleep_for(std::chrono::microseconds(50));
      continue;
    }
    if (producer_done.load() && win[0].empty() && win[1].empty() &&
        gpuos_debug_consumer_tail(ctx, 0) == seen[0] && gpuos_debug_consumer_tail(ctx, 1) == seen[1])
      return;
    if (++idle > 64) std::this_thread::yield();
  }
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 8 && argc != 9) {
    std::fprintf(stderr, "usage: host_consumer OPS INIT OUT SLOTS BATCH FLUSH_EVERY SEED [AUTO_DEPS]\n");
    return 2;
  }
  FILE* f = std::fopen(argv[1], "r");
  if (!f) die("cannot open the op list");
  int B = 0, L = 0;
  if (std::fscanf(f, " buffers %d %d", &B, &L) != 2 || B <= 0 || L <= 0) die("bad op list header");
  std::vector<HostOp> ops;
  HostOp o;
  while (std::fscanf(f, " op %d %d %d %u %d %u %d %u %u", &o.kind, &o.lc, &o.ob, &o.oo, &o.ib0,
                     &o.io0, &o.ib1, &o.io1, &o.n) == 9) {
    if (o.ob < 0 || o.ob >= B || o.ib0 < 0 || o.ib0 >= B || o.ib1 < 0 || o.ib1 >= B ||
        o.oo + (uint64_t)o.n > (uint64_t)L || o.io0 + (uint64_t)o.n > (uint64_t)L ||
        o.io1 + (uint64_t)o.n > (uint64_t)L || o.kind < 0 || o.kind > 2)
      die("op out of range");
    ops.push_back(o);
  }
  std::fclose(f);
  std::vector<int32_t> mem((size_t)B * L);
  f = std::fopen(argv[2], "rb");
  if (!f || std::fread(mem.data(), 4, mem.size(), f) != mem.size()) die("cannot read the initial buffers");
  std::fclose(f);
  const uint32_t slots = (uint32_t)std::strtoul(argv[4], nullptr, 10);
  const uint32_t batch = (uint32_t)std::strtoul(argv[5], nullptr, 10);
  const uint32_t flush_every = (uint32_t)std::strtoul(argv[6], nullptr, 10);
  const uint64_t seed = std::strtoull(argv[7], nullptr, 10);
  if (!batch || !flush_every) die("batch and flush interval must be positive");

  gpuos_config cfg;
  gpuos_config_default(&cfg);
  cfg.ring_slots = slots;
  cfg.block_on_full = 1;
  if (argc == 9) cfg.auto_deps = (uint32_t)std::strtoul(argv[8], nullptr, 10);
  gpuos_ctx* ctx = nullptr;
  int rc = gpuos_create(GPUOS_DEVICE_NONE, &cfg, &ctx);
  if (rc) die("gpuos_create", rc);
  rc = gpuos_debug_consumer_attach(ctx);
  if (rc) die("gpuos_debug_consumer_attach", rc);

  Counters cnt;
  std::thread cons(consumer, ctx, slots, seed, &cnt);
  int32_t* base = mem.data();
  auto at = [&](int b, uint32_t off) { return base + (size_t)b * L + off; };
  std::vector<gpuos_op> arr;
  uint32_t batches = 0;
  for (size_t i = 0; i < ops.size() && !consumer_failed; i += batch) {
    arr.clear();
    for (size_t j = i; j < ops.size() && j < i + batch; ++j) {
      const HostOp& h = ops[j];
      gpuos_op g;
      std::memset(&g, 0, sizeof g);
      g.opcode = h.kind == 0 ? GPUOS_OP_ADD : h.kind == 1 ? GPUOS_OP_MUL : GPUOS_OP_COPY;
      g.dtype = GPUOS_I32;
      g.flags = h.lc ? GPUOS_FLAG_LC : 0;
      g.n = h.n;
      g.out = at(h.ob, h.oo);
      g.in[0] = at(h.ib0, h.io0);
      if (h.kind != 2) g.in[1] = at(h.ib1, h.io1);
      arr.push_back(g);
    }
    rc = gpuos_submit(ctx, arr.data(), (uint32_t)arr.size(), nullptr);
    if (rc) die("gpuos_submit", rc);
    if (++batches % flush_every == 0) {
      rc = gpuos_flush(ctx);
      if (rc) die("gpuos_flush", rc);
    }
  }
  if (!consumer_failed) {
    rc = gpuos_sync(ctx, 0, 60ll * 1000 * 1000 * 1000);
    if (rc) die("gpuos_sync", rc);
  }
  producer_done = true;
  cons.join();
  if (consumer_failed) die("the consumer failed");
  gpuos_stats st;
  rc = gpuos_get_stats(ctx, &st);
  if (rc) die("gpuos_get_stats", rc);
  rc = gpuos_destroy(ctx, 1000ll * 1000 * 1000);
  if (rc) die("gpuos_destroy", rc);
  f = std::fopen(argv[3], "wb");
  if (!f || std::fwrite(mem.data(), 4, mem.size(), f) != mem.size()) die("cannot write the result");
  std::fclose(f);
  std::printf("ops %zu ran %" PRIu64 " + %" PRIu64 " out_of_order %" PRIu64 " max_ready %" PRIu64
              " deps %" PRIu64 " ring_full_waits %" PRIu64 "\n",
              ops.size(), cnt.ran[0], cnt.ran[1], cnt.out_of_order, cnt.max_ready, cnt.deps_seen,
              (uint64_t)st.ring_full_waits);
  return 0;
}
