// Internal layouts shared by the host runtime and the device kernels.
//
// Queue structure ("GPUOS: A GPU Operating System Primitive for Transparent
// Operation Fusion", section "The Paper": a host-managed work queue drained by
// one long-lived kernel with atomic task queues).  The hand-off mirrors the
// driver path of "Kernel Launch and Host-Device Interaction" (section "The
// launch path": packets written into a pinned ring in host memory, then a
// doorbell): here the host writes 256-byte descriptors into a pinned ring and
// the doorbell is a release store of the ring tail that one device wave polls.
//
// Tiles of every published descriptor form one dense ticket space per ring:
// descriptor `seq` owns tickets [ends[seq-1], ends[seq]).  In the best-effort
// ring, worker wave w runs tickets w, w + W, w + 2W, ... in increasing order
// (W = worker waves), so each tile runs exactly once without a shared claim
// counter, and the wave holding the smallest unfinished ticket can always
// proceed: every tile its op waits on has a smaller ticket and is finished.
// The latency-critical ring is claimed dynamically (compare-and-swap), so any
// wave can pick up priority work between its own tiles.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace gpuos {

// Internal opcodes beyond the public ones (gpuos_opcode).
enum : uint8_t {
  OP_FUSED_EW = 32,   // register-resident elementwise chain
  OP_NORM_GEMV = 33,  // RMSNORM -> GEMV (-> SILU_MUL, or -> ROPE q, ROPE k,
                      // COPY v): every GEMV tile normalises the input row
                      // itself (tile 0 also stores it); with the SiLU gate
                      // a tile computes gate row i and up row F + i
                      // together, in rotary mode the two rows a rotation
                      // pairs
  OP_GEMV_ADD = 34,   // GEMV -> ADD of a residual: each output row, rounded
                      // as the GEMV stores it, is added to the residual
                      // element and stored to the ADD's output
  OP_SOFTMAX_AV = 35, // ROW_SOFTMAX -> ATTN_AV: each AV tile computes the
                      // softmax of its head's score row itself
};
// Per-wave LDS scratch of the tile bodies, in floats.
constexpr uint32_t kWaveScratch = 512;

// Completion counting: a descriptor of up to 8 tiles counts its tiles in one
// counter.  A larger one spreads them over S = min(64, ceil(tiles / 8))
// sub-counters (tile t in sub-counter t % S); the wave that fills a
// sub-counter bumps the second-level counter, which completes the descriptor
// at S.  Same-address atomics serialise, so no address takes more than
// about 8 (sub-counters) or 64 (second level) increments.
constexpr uint32_t kSubCounters = 64;
constexpr uint32_t kTilesPerSub = 8;
// Replicas of the published-work words; wave w polls replica w % kReplicas.
constexpr uint32_t kReplicas = 16;

// Elementwise step codes inside a FUSED_EW micro-program.
enum : uint8_t {
  FS_ADD = 1,
  FS_MUL = 2,
  FS_SCALE = 3,
  FS_RELU = 4,
  FS_EXP = 5,
  FS_COPY = 6,  // identity (a COPY folded into a chain)
};

// Step flag bits.  Bits 4..5 hold the index (1..3) of the fused input pointer
// that supplies a binary step's second operand.
enum : uint8_t {
  FSF_OPERAND = 0x1,   // binary step: second operand is fused input in[idx]
  FSF_SELF = 0x2,      // binary step whose second operand is the accumulator
  FSF_STORE = 0x4,     // write the accumulator to out[s] after the step
};

constexpr int kMaxSteps = 8;
// Descriptor flag set by the runtime (user flags use the low bits): in[2]
// (GEMV weights) has no queued writer, so the kernel may read it before the
// op's dependencies have completed.
constexpr uint8_t DF_AUX_READY = 0x80;
// Descriptor flag set by the runtime: an elementwise op over a strided or
// broadcast view (shape and strides in the descriptor's view fields).
constexpr uint8_t DF_VIEW = 0x40;
// Descriptor flag set by the runtime with DF_VIEW: a COPY whose view is a
// 2-D transpose (output rows contiguous, the input contiguous down the output's
// columns).  Tiles are blocks of kTBlockBytes / element size rows (one 128-byte
// line of each input column) by kTCols columns, row blocks outer.
constexpr uint8_t DF_VIEW_T = 0x20;
constexpr uint32_t kTBlockBytes = 128, kTCols = 128;
constexpr int kMaxDeps = 14;  // dependencies a descriptor carries (more: wait
                              // for the retire cursor instead)
constexpr int kMaxFusedInputs = 4;
// Copies of each slot's completion word.  The completing wave writes all of
// them; a waiting wave polls the copy its number selects, so a descriptor
// with many tiles is not waited on by thousands of polls of one address.
constexpr uint32_t kDoneReplicas = 8;
constexpr int kRings = 2;      // 0 = best effort (default), 1 = latency critical
constexpr uint32_t kDescBytes = 256;
// Largest byte extent of one operand.  Tile bodies address tensors through
// buffer resources with 32-bit byte offsets; offsets of vectors past the end
// saturate at this value, which stays out of every resource's range with room
// for a 16-byte access.
constexpr uint64_t kMaxExtentBytes = 0xFFF00000ull;
constexpr uint32_t kDescMagic = 0x9e3779b9u;

// Device descriptor: 256 bytes = 64 dwords; lane i of a wave fetches dword i.
struct alignas(16) DevDesc {
  uint8_t opcode;     // dword 0: public opcode or OP_FUSED_EW
  uint8_t dtype;      //          gpuos_dtype
  uint8_t flags;      //          GPUOS_FLAG_*
  uint8_t nsteps;     //          FUSED_EW program length
  uint32_t n;         // 1: extent (see gpuos.h)
  uint32_t rows;      // 2
  uint32_t row_len;   // 3
  uint64_t seq;       // 4-5: 1-based sequence in its ring
  uint32_t ntiles;    // 6
  uint32_t tile;      // 7: units per tile (elements, rows, key rows, chunks)
  uint32_t deps_lo[8];  // 8-15: dependencies 0..7 as seq - dep_seq (same
                        // ring; 0 = none); 8..13 are dwords 54-59
  uint64_t wait_retired;  // 16-17: wait until the ring's in-order retire
                          // cursor reaches this sequence (0 = none)
  union {
    struct {
      uint64_t ptr[4];      // 18-25: out, in0, in1, in2
      uint32_t src_len[2];  // 26-27: readable length of in0 / in1 (0 = n)
      float alpha;          // 28
      float eps;            // 29
      int32_t aux[4];       // 30-33
      // DF_VIEW: 4 dimensions, outermost first (leading extents of 1), and
      // element strides of out, in0, in1 per dimension
      uint32_t vshape[4];   // 34-37
      int32_t vstride[3][4];  // 38-49
      uint8_t _pad[16];
    } p;
    struct {
      uint64_t W;           // 18-19: GEMV weights [M x K] bf16
      uint64_t out;         // 20-21: GEMV output [M] (0 = not stored)
      uint64_t x;           // 22-23: RMSNORM input [K]
      uint64_t g;           // 24-25: RMSNORM gain [K]
      uint64_t h;           // 26-27: RMSNORM output [K] (0 = not stored)
      uint64_t act;         // 28-29: SILU_MUL output [F] (0 = no SiLU gate)
      uint32_t M;           // 30
      uint32_t K;           // 31
      float eps;            // 32
      uint32_t F;           // 33: gate rows (M == 2F) when act != 0
      // rotary mode (q != 0): the GEMV output is q | k | v, D = M / 3 rows
      // each, heads of hd rows; ROPE of q and k and COPY of v follow
      uint64_t q;           // 34-35: rotated q [D]
      uint64_t k;           // 36-37: rotated k [D] (e.g. a K-cache slot)
      uint64_t v;           // 38-39: copy of v [D] (e.g. a V-cache slot)
      uint64_t tabq;        // 40-41: rotary table of q (fp32 cos[hd/2] | sin[hd/2])
      uint64_t tabk;        // 42-43: rotary table of k
      uint32_t hd;          // 44: head size (even)
      uint8_t _pad[36];
    } ng;
    struct {
      uint64_t out;         // 18-19: GEMV output [M] (0 = not stored)
      uint64_t x;           // 20-21: GEMV input [K]
      uint64_t res;         // 22-23: residual [M]
      uint64_t W;           // 24-25: weights [M x K] bf16
      uint32_t res_first;   // 26: 1 = the ADD reads the residual as in[0]
      uint32_t _u[3];       // 27-29
      uint32_t M;           // 30
      uint32_t K;           // 31
      uint64_t sum;         // 32-33: ADD output [M]
      uint8_t _pad[80];
    } ga;
    struct {
      uint64_t ptr[4];      // 18-25: out, in0, in1, in2
      uint32_t meta;        // 26: n_insns | result << 8 | n_inputs << 16
      uint32_t ins[16];     // 27-42: op | dst << 5 | a << 8 | b << 12 | c << 16
      float k[8];           // 43-50: registers 8..15
      uint32_t body;        // 51: compiled body + 1 in the compiled kernel
                            // variant (0 = none; the built-in kernel
                            // interprets the body above either way)
      uint8_t _pad[8];
    } pg;                   // GPUOS_OP_PROGRAM: the op's body, by value
    struct {
      uint64_t in[4];       // 18-25: in[0] = chain input, in[1..3] operands
      uint64_t out[8];      // 26-41: output pointer of step s (FSF_STORE)
      uint8_t step_op[8];   // 42-43
      uint8_t step_fl[8];   // 44-45
      float fscal[8];       // 46-53: SCALE factor of step s
    } f;
  };
  uint32_t deps_hi[6];  // 54-59: dependencies 8..13 (as deps_lo)
  uint64_t tstart;      // 60-61: first ticket of this descriptor
  uint32_t user_ops;    // 62: user ops folded into this descriptor
  uint32_t check;       // 63: (uint32)seq ^ kDescMagic
};
static_assert(sizeof(DevDesc) == kDescBytes, "descriptor must be 256 bytes");
static_assert(offsetof(DevDesc, deps_lo) == 8 * 4, "deps_lo at dword 8");
static_assert(offsetof(DevDesc, deps_hi) == 54 * 4, "deps_hi at dword 54");
static_assert(offsetof(DevDesc, wait_retired) == 16 * 4, "wait_retired at dword 16");
static_assert(offsetof(DevDesc, p.ptr) == 18 * 4, "ptr at dword 18");
static_assert(offsetof(DevDesc, p.src_len) == 26 * 4, "src_len at dword 26");
static_assert(offsetof(DevDesc, p.alpha) == 28 * 4, "alpha at dword 28");
static_assert(offsetof(DevDesc, p.aux) == 30 * 4, "aux at dword 30");
static_assert(offsetof(DevDesc, p.vshape) == 34 * 4 && offsetof(DevDesc, p.vstride) == 38 * 4,
              "view fields at dwords 34-49");
static_assert(offsetof(DevDesc, f.out) == 26 * 4, "fused out at dword 26");
static_assert(offsetof(DevDesc, ng.M) == 30 * 4, "norm-GEMV M at dword 30");
static_assert(offsetof(DevDesc, ng.q) == 34 * 4 && offsetof(DevDesc, ng.hd) == 44 * 4,
              "norm-GEMV rotary fields at dwords 34-44");
static_assert(offsetof(DevDesc, ga.W) == 24 * 4 && offsetof(DevDesc, ga.M) == 30 * 4 &&
                  offsetof(DevDesc, ga.sum) == 32 * 4,
              "GEMV-ADD keeps the GEMV fields where a GEMV descriptor has them");
static_assert(offsetof(DevDesc, pg.meta) == 26 * 4 && offsetof(DevDesc, pg.ins) == 27 * 4 &&
                  offsetof(DevDesc, pg.k) == 43 * 4 && offsetof(DevDesc, pg.body) == 51 * 4,
              "program fields at dwords 26-50");
static_assert(offsetof(DevDesc, f.step_op) == 42 * 4, "step_op at dword 42");
static_assert(offsetof(DevDesc, f.step_fl) == 44 * 4, "step_fl at dword 44");
static_assert(offsetof(DevDesc, f.fscal) == 46 * 4, "fscal at dword 46");
static_assert(offsetof(DevDesc, tstart) == 60 * 4, "tstart at dword 60");
static_assert(offsetof(DevDesc, user_ops) == 62 * 4, "user_ops at dword 62");
static_assert(offsetof(DevDesc, check) == 63 * 4, "check word is dword 63");

// Device-side scheduler state (device memory).  Hot words sit on their own
// 256-byte lines.
struct alignas(256) DevRing {
  uint64_t next;        // latency-critical ring: descriptors claimed (CAS)
  uint64_t _p0[31];
  uint64_t retired;     // in-order retire cursor
  uint64_t _p1[31];
};

// One replica of what the doorbell wave has published for a ring.  The
// doorbell stores avail_ops before avail_tiles; readers load avail_tiles
// first, so the descriptors below avail_tiles are always within avail_ops.
struct alignas(256) AvailLine {
  uint64_t avail_tiles;  // tickets below this value are runnable
  uint64_t avail_ops;    // descriptors whose ticket ranges are published
  uint64_t stop_ticket;  // ring 0: once stop_epoch is the running launch's
  uint64_t stop_epoch;   // epoch, waves whose next ticket is >= stop_ticket
                         // exit (stop_ticket is stored first)
  uint64_t copied_ops;   // descriptors (retired, copied_ops] are in the
                         // device ring; later ones are read from the host
  uint64_t _p[27];
};

struct alignas(256) DevCtl {
  DevRing ring[kRings];
  AvailLine avail[kRings][kReplicas];
  uint64_t arrived;     // waves that have started, summed over all launches:
                        // launch e of a grid of W waves is complete at e * W
  uint64_t _pa[31];
  // debug options (read only when KArgs::debug is nonzero)
  uint32_t* tile_exec[kRings];  // executions of ticket i of each ring, i < n
  uint64_t tile_exec_n;
  // latency-critical ring: the wave that completes descriptor s stores s into
  // hdone_lc[slot] (pinned host memory), so that the host sees an LC op done
  // without waiting for the in-order retire of the doorbell wave
  uint64_t* hdone_lc;
  uint64_t _pd[28];
};
constexpr uint32_t kDebugCount = 1u;

// Host-visible control block (pinned host memory, fine-grained).
struct alignas(256) HostCtl {
  uint64_t tail[kRings];      // host: last published sequence per ring
  uint64_t _p0[30];
  uint64_t completed[kRings]; // device: retire cursor per ring
  uint64_t heartbeat;         // device: doorbell loop iterations
  uint64_t exit_tiles;        // device: ring-0 tickets published when the
                              // kernel last exited (stored first)
  uint64_t exit_epoch;        // device: epoch of the launch that exited
  uint64_t exit_req;          // device: epoch of a launch about to leave
                              // after idling (0 = cancelled); between this
                              // store and the exit, the doorbell re-reads
                              // the tails and cancels if any moved
  uint64_t resident_epoch;    // device: epoch of the last launch whose waves
                              // have all started (before any work is taken)
  uint64_t _p1[25];
  uint64_t stop_req;          // host: nonzero asks the kernel to exit once
                              // every published descriptor has retired
  uint64_t error;             // device: first error code (0 = none)
  uint64_t error_seq;         // device: (ring << 62) | sequence that raised it
  uint64_t yield_req;         // host: nonzero asks a drained kernel to leave
                              // at once, as after its idle period
  uint64_t _p2[4];
  uint64_t lc_tail;           // host: tail[1] again, on a 64-byte line of its
                              // own: the reserved waves poll it, so the line
                              // the host writes at every flush and the
                              // doorbell polls is not also read by them
  uint64_t _p3[23];
};
static_assert(sizeof(HostCtl) == 768, "host control block is three 256-byte groups");
static_assert(offsetof(HostCtl, lc_tail) % 64 == 0 && offsetof(HostCtl, lc_tail) / 64 != 0 &&
                  offsetof(HostCtl, lc_tail) / 64 != offsetof(HostCtl, stop_req) / 64,
              "the latency-critical tail has a 64-byte line of its own");

// Per-descriptor trace record (device memory), one per ring slot.
struct TraceRec {
  uint64_t seq;
  uint64_t t_claim;  // first tile: dependencies met
  uint64_t t_done;   // completing wave: counted last, done_id about to be stored
  uint32_t opcode;
  uint32_t ntiles;
  uint64_t t_wait;   // first tile: its wave starts waiting on the dependencies
  uint64_t t_end;    // completing wave: its tile's stores issued
  uint64_t t_ack;    // completing wave: those stores acknowledged
};

// Device error codes (HostCtl::error).
enum : uint64_t {
  DERR_BAD_OPCODE = 1,
  DERR_GATHER_RANGE = 2,
  DERR_DESC_CHECK = 3,
};

// Host bytes of the pinned rings of a context with `slots` slots per ring:
// control block, then per ring the descriptor ring and its ends, then the
// latency-critical ring's completion words.
inline size_t align256(size_t b) { return (b + 255) / 256 * 256; }
inline size_t static_host_bytes(uint32_t slots) {
  return align256(sizeof(HostCtl)) +
         kRings * (align256((size_t)slots * kDescBytes) + align256((size_t)slots * 8)) +
         align256((size_t)slots * 8);
}

// Device scratch of gpuos_create_static: one array per device, sized for
// kStaticMaxSlots ring slots per ring.
constexpr size_t kStaticScratchBytes = 8u << 20;
constexpr uint32_t kStaticMaxSlots = 4096;
constexpr int kMaxStaticDevices = 64;
// Device bytes of a context's scheduler state with `slots` slots per ring:
// control block, then per ring the descriptor ring, ends, completion words,
// tile counters and their second level.
inline size_t static_device_bytes(uint32_t slots) {
  size_t b = align256(sizeof(DevCtl));
  for (int r = 0; r < kRings; ++r) {
    b += align256((size_t)slots * kDescBytes);
    b += align256((size_t)2 * slots * 8);
    b += align256((size_t)slots * kDoneReplicas * 8);
    b += align256((size_t)kSubCounters * slots * 4);
    b += align256((size_t)slots * 4);
  }
  return b;
}

// Everything the resident kernel needs, passed by value.
struct KArgs {
  const DevDesc* hdesc[kRings];   // pinned host ring (device-visible address)
  DevDesc* ddesc[kRings];         // device copy of the ring, filled by the
                                  // doorbell wave before it publishes
  const uint64_t* hends[kRings];  // pinned host: ends[slot] per descriptor
  HostCtl* hctl;                  // pinned host control block
  DevCtl* dctl;                   // device control block
  uint64_t* dends[kRings];        // device copy of ends[], 2 * ring_slots
                                  // entries indexed by (seq - 1) mod 2*slots
  uint64_t* done_id[kRings];      // device: last completed sequence per slot,
                                  // kDoneReplicas copies (copy k of slot s
                                  // at k * slots + s)
  uint32_t* tiles_done[kRings];   // device: kSubCounters x ring_slots tile
                                  // counters, sub-counter s of slot at
                                  // [s * ring_slots + slot]
  uint32_t* subs_done[kRings];    // device: filled sub-counters per slot
  TraceRec* trace[kRings];        // device trace ring (nullable)
  uint32_t cap_mask;              // ring_slots - 1
  uint32_t ends_mask;             // 2 * ring_slots - 1
  uint32_t workers;               // best-effort worker waves
  uint32_t lc_waves;              // waves reserved for the latency-critical
                                  // ring (0 = no priority ring)
  uint32_t epoch;                 // launch number of this context, from 1
  uint32_t debug;                 // 0, or the debug options of DevCtl::dbg
                                  // (bit 0: count tile executions; bits
                                  // 16-31: jitter steps)
  uint64_t ticket_base;           // ring-0 tickets below this ran in earlier
                                  // launches
  uint64_t idle_exit_ticks;       // exit after this long (100 MHz ticks) with
                                  // nothing queued; 0 = never
};

}  // namespace gpuos
