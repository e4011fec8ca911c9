/*
 * gpuos.h - C ABI of the persistent small-op runtime for AMD Instinct MI355X
 * (gfx950).
 *
 * One resident HIP kernel stays on the GPU and drains a queue of small tensor
 * operations that the host publishes through a ring of descriptors, so that a
 * stream of tiny ops costs one launch instead of one launch per op.  The
 * method is the one described in "GPUOS: A GPU Operating System Primitive for
 * Transparent Operation Fusion" (section "The Paper": a long-lived worker
 * kernel fed by a host-managed work queue with atomic task queues, micro-ops
 * batched into unified submissions, operators over a generic tensor view).
 * The host-to-device hand-off follows the launch path described in "Kernel
 * Launch and Host-Device Interaction" (section "The launch path": commands are
 * written into a pinned ring in host memory and a doorbell write tells the GPU
 * front end to fetch them), moved into user space and paid once per flush.
 * Elementwise chains such as y = relu(a*x + b) are merged into one
 * register-resident pass as in "Launch Overhead and Fusion" (section
 * "Fusion").
 *
 * Conventions shared by every entry point:
 *  - Every function returns a gpuos_status (0 on success, a negative code on
 *    failure) unless stated otherwise.  On failure a message is available from
 *    gpuos_last_error() in the calling thread.
 *  - Pointers inside a gpuos_op are DEVICE addresses owned by the caller
 *    (typically torch tensors' data_ptr()).  They must stay allocated, and no
 *    other agent may write them, until the op that uses them has completed.
 *  - Plain host pointers to gpuos_op / gpuos_config / gpuos_stats arrays are
 *    read or written during the call only; the library keeps no reference.
 *  - A context is single-producer: calls on one context must not overlap in
 *    time (like calls on one stream).  Different contexts are independent.
 *  - While a context is alive its resident kernel occupies part of every
 *    compute unit.  A device-wide synchronisation (hipDeviceSynchronize,
 *    torch.cuda.synchronize) waits for that kernel and therefore only returns
 *    after gpuos_destroy().  Synchronise on the caller's own streams instead.
 */
#ifndef GPUOS_H
#define GPUOS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GPUOS_ABI_VERSION 9

/* Status codes. */
typedef enum gpuos_status {
  GPUOS_OK = 0,
  GPUOS_EINVAL = -1,    /* a malformed argument or op descriptor */
  GPUOS_ENOMEM = -2,    /* device or pinned host allocation failed */
  GPUOS_EAGAIN = -3,    /* ring full and the context does not block */
  GPUOS_ETIMEDOUT = -4, /* gpuos_sync gave up before the ops completed */
  GPUOS_EDEVICE = -5,   /* HIP error, or the device raised its error word;
                           the context is poisoned and must be destroyed */
  GPUOS_ESTATE = -6,    /* call not allowed in the context's current state */
  GPUOS_ECOMPILE = -7   /* run-time compilation failed (gpuos_program_compile) */
} gpuos_status;

/*
 * Opcodes accepted by gpuos_submit.  Operand roles: in[0] and in[1] are the
 * data operands, in[2] the auxiliary operand (weight matrix, gain vector,
 * rotary table or index vector).  "x[k mod len]" means that a source whose
 * src_len is shorter than the op's extent is read cyclically; a longer one is
 * read as a prefix.  Element type: dtype applies to in[0], in[1] and out unless
 * the row says otherwise; BF16 operands are widened exactly to fp32, computed
 * in fp32 and rounded to bf16 with round-to-nearest-even.
 *
 *  NOP          nothing; completes once its dependencies have completed.
 *  COPY         out[k] = in0[k mod src_len0], k < n.  Bit copy.
 *  GATHER       out[k] = in0[idx[k]], idx = (int32*)in[2], k < n; an index
 *               outside [0, src_len0) sets the device error word.
 *  ADD          out[k] = in0[k] + in1[k]
 *  MUL          out[k] = in0[k] * in1[k]
 *  SCALE        out[k] = alpha * in0[k]
 *  RELU         out[k] = in0[k] > 0 ? in0[k] : +0   (-0 and NaN give +0)
 *  EXP          out[k] = exp(in0[k])
 *  ROW_SUM      out[r] = sum_j in0[r*row_len + j], r < rows; out has rows
 *               elements, n must equal rows*row_len.
 *  ROW_SOFTMAX  m = max_j x[r,j]; out[r,j] = exp(x[r,j]-m) / sum_j exp(x[r,j]-m)
 *  RMSNORM      out[r,j] = x[r,j] / sqrt(mean_j(x[r,j]^2) + eps) * g[j],
 *               g = in[2] (row_len elements of dtype).
 *  ROPE         rotate-half rotary embedding of rows = heads rows of row_len =
 *               head_dim (even): with c = in[2][0..h/2), s = in[2][h/2..h)
 *               (fp32 table for the token's position, h = head_dim):
 *               y[i] = x[i]*c[i] - x[i+h/2]*s[i],
 *               y[i+h/2] = x[i+h/2]*c[i] + x[i]*s[i],  i < h/2.
 *  GEMV         out[i] = sum_k W[i*K + k] * x[k], i < M; W = (bf16*)in[2] row
 *               major, x = in0 (dtype), aux[0] = M, aux[1] = K, n = M.
 *  ATTN_SCORE   out[h*S + j] = alpha * sum_d q[h*D + d] * Kc[j*(H*D) + h*D + d]
 *               q = in0 (dtype), Kc = (bf16*)in[2], out fp32;
 *               aux = {H, D, S}, n = H*S.
 *  ATTN_AV      out[h*D + d] = sum_j p[h*S + j] * Vc[j*(H*D) + h*D + d]
 *               p = (float*)in0, Vc = (bf16*)in[2], out dtype;
 *               aux = {H, D, S}, n = H*D.
 *  SILU_MUL     out[k] = g[k] / (1 + exp(-g[k])) * u[k], g = in0, u = in1.
 *  SPIN         debug op: the claiming wave spins for aux[0] nanoseconds
 *               (bounded to 10 ms) and completes; used to test time-outs.
 *  PROGRAM      an op defined at run time (gpuos_program_define): out[k] =
 *               P(in0[k], in1[k], in2[k]) for the register program P whose
 *               id is aux[0]; in[j] is given for j < P.n_inputs and null
 *               otherwise (in[2] is a data input here).  dtype F32, BF16 or
 *               F16 for every operand; src_len must be 0.
 *
 * Ops whose result is rounded once from an exact formula (COPY, GATHER, ADD,
 * MUL, SCALE, RELU, ROPE) give bit-identical results however the queue is
 * scheduled or fused.  Reductions and transcendentals (EXP, ROW_SUM,
 * ROW_SOFTMAX, RMSNORM, GEMV, ATTN_*, SILU_MUL) accumulate in fp32 and match
 * an exact evaluation to within rounding.  A PROGRAM op is bit-reproducible
 * like the first group unless its program uses EXP.
 */
typedef enum gpuos_opcode {
  GPUOS_OP_NOP = 0,
  GPUOS_OP_COPY = 1,
  GPUOS_OP_GATHER = 2,
  GPUOS_OP_ADD = 3,
  GPUOS_OP_MUL = 4,
  GPUOS_OP_SCALE = 5,
  GPUOS_OP_RELU = 6,
  GPUOS_OP_EXP = 7,
  GPUOS_OP_ROW_SUM = 8,
  GPUOS_OP_ROW_SOFTMAX = 9,
  GPUOS_OP_RMSNORM = 10,
  GPUOS_OP_ROPE = 11,
  GPUOS_OP_GEMV = 12,
  GPUOS_OP_ATTN_SCORE = 13,
  GPUOS_OP_ATTN_AV = 14,
  GPUOS_OP_SILU_MUL = 15,
  GPUOS_OP_SPIN = 16,
  GPUOS_OP_PROGRAM = 17,
  GPUOS_OP_COUNT = 18
} gpuos_opcode;

/*
 * Element types.  BF16 and F16 operands are widened exactly to fp32, computed
 * in fp32 and rounded back with round-to-nearest-even.  F16 is accepted by
 * COPY, ADD, MUL, SCALE, RELU, EXP, SILU_MUL, ROW_SUM, ROW_SOFTMAX, RMSNORM
 * and ROPE.  I32 is accepted by COPY and GATHER (bit moves) and by ADD, MUL
 * (two's-complement, wrapping modulo 2^32) and RELU (x > 0 ? x : 0).
 */
typedef enum gpuos_dtype {
  GPUOS_F32 = 0,
  GPUOS_BF16 = 1,
  GPUOS_I32 = 2,
  GPUOS_F16 = 3
} gpuos_dtype;

/* Op flags. */
#define GPUOS_FLAG_TRANSIENT 0x1u   /* the output is scratch: when the fusion
                                       pass merges this op with its consumer
                                       and no other queued op reads it, the
                                       store is elided and its contents are
                                       left undefined */
#define GPUOS_FLAG_LC 0x2u          /* latency-critical: goes to the priority
                                       ring, served by reserved waves that
                                       never run best-effort tiles.  An
                                       explicit dependency between an LC op
                                       and a best-effort op is rejected
                                       (EINVAL).  A byte-range hazard
                                       between them is honoured on the
                                       host: gpuos_flush waits, before
                                       publishing the dependent op, until
                                       the op it depends on has completed,
                                       which can block the flush for as
                                       long as that op runs */
#define GPUOS_FLAG_NONTEMPORAL 0x4u /* stream the op's operands: loads and
                                       stores are marked non-temporal so
                                       their cache lines are evicted first.
                                       Set automatically on elementwise,
                                       COPY and fused ops whose operands
                                       total config.stream_min_kib or more */

/*
 * User op descriptor (128 bytes).  Fields not used by an opcode must be zero.
 *  n        extent of the op: number of output elements for elementwise ops,
 *           rows*row_len for row ops, M for GEMV, H*S / H*D for attention.
 *  src_len  length in elements of in[0] / in[1]; 0 means "same as the op's
 *           extent".  A shorter source is read cyclically (elementwise ops,
 *           COPY, ROW_* inputs); GATHER uses src_len[0] as the bound check.
 *  deps     up to four ops this op must wait for: a value > 0 is an id
 *           returned by an earlier gpuos_submit; a value < 0 names the op
 *           -deps[i] positions earlier in the same gpuos_submit array; 0 is
 *           unused.  Read-after-write, write-after-read and write-after-write
 *           hazards between the byte ranges of queued ops are added
 *           automatically unless the context was created with auto_deps = 0.
 * All device pointers must be aligned to their element size; 16-byte aligned
 * operands take the 128-bit load path.  n, rows * row_len and src_len are at
 * most 2^30, and no operand may span more than 0xFFF00000 bytes (4 GiB minus
 * 1 MiB: kernels address an operand with 32-bit byte offsets).
 */
typedef struct gpuos_op {
  uint16_t opcode;   /* gpuos_opcode */
  uint8_t dtype;     /* gpuos_dtype */
  uint8_t flags;     /* GPUOS_FLAG_* */
  uint32_t n;
  uint32_t rows;
  uint32_t row_len;
  void* out;
  const void* in[3];
  uint64_t src_len[2];
  float alpha;
  float beta;
  float eps;
  int32_t aux[4];
  int32_t _pad;
  int64_t deps[4];
} gpuos_op;

/*
 * Context configuration.  gpuos_config_default() fills the defaults; zero in
 * a field of a config passed to gpuos_create also selects the default.  The
 * environment can replace a default when a context is created: GPUOS_<FIELD>
 * (the field's name in capitals, e.g. GPUOS_FUSION=2 or GPUOS_RING_SLOTS=
 * 0x1000) sets that field wherever the caller's config leaves it zero; a value
 * that is not a 32-bit unsigned number fails gpuos_create with EINVAL, and
 * the result is validated like the caller's own fields.
 */
typedef struct gpuos_config {
  uint32_t ring_slots;    /* descriptors per ring, power of two in
                             [64, 1<<18]; default 65536 */
  uint32_t waves_per_cu;  /* resident waves per compute unit, multiple of 4
                             in [4, 32]; default 8 */
  uint32_t tile_elems;    /* elementwise tile in elements, multiple of 256;
                             default 1024 (one memory round trip per wave) */
  uint32_t be_tile_elems; /* tile for ops of 1<<24 elements or more, multiple
                             of 256 in [256, 1<<22]; default 32768 */
  uint32_t fusion;        /* 1 = merge adjacent elementwise ops (default),
                             2 = off */
  uint32_t auto_deps;     /* 1 = add hazard dependencies (default), 2 = off */
  uint32_t trace;         /* 1 = record per-op device timestamps, 2 = off
                             (default) */
  uint32_t block_on_full; /* 1 = submit/flush wait for ring space (default),
                             2 = return GPUOS_EAGAIN */
  uint32_t max_fuse;      /* longest fused chain, 2..8; default 8 */
  uint32_t priority;      /* 1 = a latency-critical ring served by
                             lc_waves reserved waves (default), 2 = no
                             priority ring: GPUOS_FLAG_LC ops are rejected
                             and every wave runs best-effort tiles */
  uint32_t idle_exit_ms;  /* the resident kernel exits after this many
                             milliseconds with every published op retired and
                             nothing new, giving its compute units back; the
                             next flush (or a wait that finds work pending)
                             relaunches it.  Default 200; 0xFFFFFFFF = never */
  uint32_t stream_min_kib; /* elementwise / COPY / fused ops moving at least
                              this many KiB are streamed (non-temporal).
                              Default 32768 (32 MiB); 0xFFFFFFFF = only ops
                              flagged GPUOS_FLAG_NONTEMPORAL */
  uint32_t lc_waves;      /* waves reserved for the latency-critical ring
                             when priority == 1, in [1, 64]; default 8 (one
                             per XCD).  They never run best-effort tiles, so
                             a latency-critical op waits for no best-effort
                             tile */
  uint32_t tile_counts;   /* debug: count how many times each of the first
                             tile_counts tiles (tickets) of each ring runs,
                             in device memory that gpuos_debug_tile_counts
                             reads back (every count must be exactly 1);
                             0 = off (default) */
  uint32_t jitter;        /* debug: before running a tile, its wave waits a
                             pseudo-random 0..jitter steps of about 0.1 us
                             drawn from a hash of the tile's ticket, so tiles
                             start and finish in another order; results of
                             exact-class ops must not change.  0 = off
                             (default), at most 1000 */
  uint32_t reserved;      /* must be 0 */
} gpuos_config;

/* Counters returned by gpuos_get_stats. */
typedef struct gpuos_stats {
  uint64_t ops_submitted;      /* user ops accepted by gpuos_submit */
  uint64_t ops_fused;          /* user ops merged into a preceding descriptor */
  uint64_t descs_published;    /* device descriptors published (all rings) */
  uint64_t descs_completed;    /* device descriptors retired (all rings) */
  uint64_t flushes;
  uint64_t ring_full_waits;    /* times publishing had to wait for space */
  uint64_t deps_explicit;      /* dependencies given by the caller */
  uint64_t deps_auto;          /* hazard dependencies added by the runtime */
  uint64_t device_error;       /* device error word (0 = none) */
  uint64_t error_desc;         /* descriptor sequence that raised it */
  uint64_t worker_waves;       /* resident best-effort worker waves */
  uint64_t compute_units;
  uint64_t kernel_ns;          /* summed duration of the resident kernel's
                                  launches, from HIP events recorded on its
                                  stream just before and just after each
                                  launch; counts launches that have ended */
  uint64_t launches;           /* resident kernel launches (1 + relaunches
                                  after idle exits) */
  uint64_t lc_waves;           /* waves serving the latency-critical ring */
  uint64_t programs_lowered;   /* PROGRAM ops run as a built-in op or fused
                                  micro-program (their body is a chain the
                                  fused tile expresses; fusion on) */
  uint64_t programs_compiled;  /* PROGRAM ops published with a compiled body
                                  (gpuos_program_compile) */
  uint64_t kernel_switches;    /* hand-overs of the queue between the built-in
                                  kernel and the compiled variant */
} gpuos_stats;

/* Per-descriptor device timing, recorded when config.trace == 1.  Times are
 * s_memrealtime ticks (100 MHz).  They split a descriptor's critical path:
 * t_wait..t_claim is the first tile's dependency poll, t_claim..t_end its
 * work up to the completing wave's last store, t_end..t_ack that wave's
 * store acknowledgement, t_ack..t_done the completion count. */
typedef struct gpuos_trace_rec {
  uint64_t seq;       /* device descriptor sequence (1-based, per ring) */
  uint64_t t_claim;   /* the first tile's dependencies are met */
  uint64_t t_done;    /* the last tile is counted (done_id follows) */
  uint32_t opcode;    /* opcode executed (FUSED_EW = 32) */
  uint32_t ntiles;
  uint32_t ring;      /* 0 = best-effort ring, 1 = latency-critical ring */
  uint32_t first_ops; /* user ops folded into this descriptor */
  uint64_t t_wait;    /* the first tile's wave starts its dependency poll */
  uint64_t t_end;     /* the completing wave's tile has issued its stores */
  uint64_t t_ack;     /* those stores are acknowledged */
} gpuos_trace_rec;

typedef struct gpuos_ctx gpuos_ctx;

/* Fills *cfg with the defaults. */
void gpuos_config_default(gpuos_config* cfg);

/*
 * Creates a context on HIP device `device`: allocates the descriptor rings
 * (pinned host memory), the scheduler state (device memory) and launches the
 * resident kernel on a library-owned non-blocking stream ("The Paper": one
 * long-lived kernel instead of one launch per op).  The grid is sized to the
 * kernel's occupancy (waves_per_cu on every compute unit), and the kernel
 * takes no work before every one of its waves is running: each wave checks
 * in at start, and the call returns only once the whole grid has (a worker
 * waits only for tiles held by other waves, so a partly resident grid could
 * wait forever; "The Counter" on the GPUOS page notes the kernel holds the
 * GPU).  cfg may be NULL for the defaults.  *out receives the context (NULL
 * on failure).
 * Errors: EINVAL (bad device or config), ENOMEM, EDEVICE (HIP failure, or the
 * grid did not become resident within 10 s, for example because another
 * kernel holds compute units).
 */
int gpuos_create(int device, const gpuos_config* cfg, gpuos_ctx** out);

/*
 * gpuos_create for callers that cannot allocate memory (code that must not
 * call hipMalloc or hipHostMalloc: serving loops, harnesses that forbid it).
 * The context's device scheduler state (control block, device descriptor
 * ring, ticket ends, completion words, tile counters) lives in a static
 * device array the library holds on each device until the process ends
 * (8 MiB: at most GPUOS_STATIC_MAX_SLOTS ring slots per ring), and its pinned
 * rings live in host_ws, which the caller owns: host_ws_bytes >=
 * GPUOS_STATIC_HOST_BYTES(cfg->ring_slots), 256-byte aligned, from
 * hipHostMalloc with hipHostMallocMapped | hipHostMallocCoherent, untouched
 * by the caller until gpuos_destroy returns.  The call makes no device or
 * pinned allocation (host bookkeeping uses the C++ heap; the stream and the
 * two timing events are created as in gpuos_create).  Every other entry point
 * works on the context as on one from gpuos_create.
 * One static context per device at a time: they would share the device's
 * array, and calls on two of them would race; the second create returns
 * ESTATE.  A new static context clears what must start at zero.
 * Errors: EINVAL (ring_slots above GPUOS_STATIC_MAX_SLOTS, trace or
 * tile_counts requested, a workspace too small, misaligned or not pinned
 * that way, a bad device or config), ESTATE (a static context is alive on
 * the device), EDEVICE.
 */
#define GPUOS_STATIC_MAX_SLOTS 4096u
#define GPUOS_STATIC_HOST_BYTES(slots) \
  (768u + 2u * ((size_t)(slots) * 256u + (((size_t)(slots) * 8u + 255u) / 256u) * 256u) + \
   (((size_t)(slots) * 8u + 255u) / 256u) * 256u)
int gpuos_create_static(int device, const gpuos_config* cfg, void* host_ws, size_t host_ws_bytes,
                        gpuos_ctx** out);

/*
 * Validates and copies n ops into the context's staging area; the caller's
 * array may be reused on return.  ids_out (nullable, n entries) receives the
 * ids assigned to the ops: consecutive, monotone, starting at 1 for a new
 * context.  Nothing reaches the device before gpuos_flush (the "unified
 * submission" of "The Paper").  Dependencies are resolved here (explicit ones
 * plus byte-range hazards).
 * Errors: EINVAL (bad opcode, dtype, size, alignment, or a dependency on an
 * id not yet submitted); nothing from the call is staged then.  ESTATE if the
 * context is poisoned.
 */
int gpuos_submit(gpuos_ctx* ctx, const gpuos_op* ops, uint32_t n,
                 uint64_t* ids_out);

/*
 * A strided or broadcast view of an elementwise op's operands (the "generic
 * tensor abstraction" of arbitrary shapes, strides and broadcasting in the
 * GPUOS page, section "The Paper").  With a view, element (i0, .., i{d-1})
 * of the op's index space, shape[0] x .. x shape[ndim-1] (outermost first,
 * product = n), is
 *   out[sum_k i_k stride[0][k]] = f(in0[sum_k i_k stride[1][k]],
 *                                   in1[sum_k i_k stride[2][k]])
 * with strides in elements.  Input strides are >= 0 (0 broadcasts the input
 * along that dimension); output strides are >= 0 and must address every
 * element of the index space at a distinct position (checked).  src_len must
 * be 0.  ndim = 0 means no view (the plain contiguous op).
 */
typedef struct gpuos_view {
  uint32_t ndim;        /* 0..4 */
  uint32_t _reserved;   /* must be 0 */
  uint64_t shape[4];
  int64_t stride[3][4]; /* [0] out, [1] in[0], [2] in[1] */
} gpuos_view;

/*
 * gpuos_submit with views: views[i] (nullable array; NULL = no op has a
 * view) describes op i's index space and strides.  Views are accepted by
 * COPY, ADD, MUL, SCALE, RELU, EXP and SILU_MUL in every dtype those ops
 * take; an op with a view is never fused.  The byte ranges used for hazard
 * tracking cover each operand from its pointer to its largest offset.
 * Errors: as gpuos_submit, plus EINVAL for a malformed view (ndim > 4, an
 * extent product other than n, a negative stride, an output that addresses
 * an element twice, an operand past 0xFFF00000 bytes, or an output that
 * overlaps an input without being exactly that input under the same view).
 */
int gpuos_submit_views(gpuos_ctx* ctx, const gpuos_op* ops, const gpuos_view* views,
                       uint32_t n, uint64_t* ids_out);

/*
 * Runs the fusion pass over the staged ops, writes the resulting device
 * descriptors into the ring and rings the doorbell (a release store of the
 * ring tail the resident kernel polls).  This is the user-space form of the
 * last steps of a launch in "Kernel Launch and Host-Device Interaction"
 * (section "The launch path": the command packet is written into a ring and
 * a doorbell write tells the GPU to fetch it), paid once per flush instead of
 * once per op.  Returns without waiting for the ops to run, like a kernel
 * launch.  If the ring is full it waits for space when block_on_full = 1,
 * else returns EAGAIN with the unpublished ops still staged.  A staged op that
 * has a byte-range hazard on an op of the other ring makes the flush wait on
 * the host for that op (see GPUOS_FLAG_LC).
 * Errors: EDEVICE (context poisoned), EAGAIN.
 */
int gpuos_flush(gpuos_ctx* ctx);

/*
 * gpuos_submit followed by gpuos_flush in one call, for callers whose ops
 * must start at once (a latency-critical op submitted alone): the same
 * validation, ids and errors as gpuos_submit, then the flush's.  If the submit
 * fails nothing is flushed; if the flush fails the ops stay staged.
 */
int gpuos_submit_flush(gpuos_ctx* ctx, const gpuos_op* ops, uint32_t n, uint64_t* ids_out);

/*
 * Flushes, then blocks until every op with id <= upto has completed
 * (upto = 0: every op submitted so far).  timeout_ns < 0 waits forever.
 * Completion of an op implies its outputs are visible to later work on any
 * stream of the device and to device-to-host copies.  ("Synchronization
 * primitives": the blocking form of stream/event synchronisation.)
 * Errors: ETIMEDOUT, EDEVICE (device error word set or HIP failure).
 */
int gpuos_sync(gpuos_ctx* ctx, uint64_t upto, int64_t timeout_ns);

/*
 * Non-blocking completion test for op `id` (the event.query form of
 * "Synchronization primitives"): returns 1 if done, 0 if pending, or a
 * negative status (EINVAL for an id never submitted, EDEVICE if poisoned).
 * Does not flush.
 */
int gpuos_query(gpuos_ctx* ctx, uint64_t id);

/*
 * Copies the context's counters into *out (host memory, written during the
 * call only).  The counters are what "gpuopt-runtime 0.1.0" (section "What it
 * does") keeps for its replay path, recast for a work queue: how many ops were
 * accepted, fused and completed, how often publication waited, and how long
 * the resident kernel ran (HIP events, the timing method of "Kernel Launch and
 * Host-Device Interaction", section "CUDA events for timing").  Works on any
 * context, also a stopped or poisoned one.  Errors: EINVAL (null argument).
 * Named gpuos_get_stats rather than gpuos_stats because gpuos_stats is the
 * struct's name.
 */
int gpuos_get_stats(gpuos_ctx* ctx, gpuos_stats* out);

/*
 * Copies up to max trace records of the most recently retired descriptors
 * (oldest first, at most ring_slots of them) into out and stores the count
 * in *n_out.  Requires config.trace == 1 (else ESTATE).  Waits for no op.
 */
int gpuos_trace_read(gpuos_ctx* ctx, gpuos_trace_rec* out, uint32_t max,
                     uint32_t* n_out);

/*
 * Drains every submitted op, tells the resident kernel to exit (a STOP
 * descriptor with one tile per worker wave) and waits for it, bounded by
 * timeout_ns (< 0 = forever).  Afterwards the context accepts only
 * gpuos_get_stats, gpuos_trace_read, gpuos_query, gpuos_sync (which returns
 * at once) and gpuos_destroy; gpuos_stats.kernel_ns then holds the kernel's
 * lifetime.  Calling it twice is harmless.
 * Errors: ETIMEDOUT (ops did not drain or the kernel did not exit),
 * EDEVICE (device error word set or HIP failure; the kernel is still stopped).
 */
int gpuos_stop(gpuos_ctx* ctx, int64_t timeout_ns);

/*
 * Ends a context: drains every submitted op (or abandons unflushed ones when
 * the context is poisoned), tells the resident kernel to exit, waits for it
 * (bounded by timeout_ns, < 0 = forever) and frees all library memory.  The
 * long-lived worker kernel of "GPUOS: A GPU Operating System Primitive for
 * Transparent Operation Fusion" (section "The Paper") holds its compute units
 * until told to stop; this is that stop, with a bound so that a wedged kernel
 * cannot hang the caller.  The context pointer is invalid afterwards, also
 * when an error is returned.
 * Errors: ETIMEDOUT (kernel did not exit; its memory is then leaked, not
 * freed under it), EDEVICE.
 */
int gpuos_destroy(gpuos_ctx* ctx, int64_t timeout_ns);

/*
 * Message describing the last failing call made by this thread (on any
 * context); "" if none.  The pointer stays valid until the thread's next
 * failing call.  Errors are reported where the caller waits, as in "Kernel
 * Launch and Host-Device Interaction" (section "Synchronization primitives":
 * an asynchronous call returns at once and a failure surfaces at the next
 * synchronising call); the status code says that a call failed and this
 * message says why.  It is thread-local rather than per context because some
 * failures (gpuos_create, gpuos_baseline_run) have no context.
 */
const char* gpuos_last_error(void);

/*
 * Per-op launch comparator: runs the n ops on HIP stream `stream` (NULL = the
 * legacy default stream) as one kernel launch each, in order, with the same
 * tile code as the resident kernel; stream order provides every dependency
 * ("Under the hood": blocks of different kernels on one stream never
 * overlap).  With fuse = 1 the fusion pass runs first and each fused chain is
 * one launch (a stand-alone fused kernel).  Does not synchronise.
 * deps are ignored; PROGRAM ops are refused (their bodies belong to a
 * context).  Errors: EINVAL, EDEVICE.
 */
int gpuos_baseline_run(int device, const gpuos_op* ops, uint32_t n, int fuse,
                       void* stream);

/*
 * Ops defined at run time ("GPUOS: A GPU Operating System Primitive for
 * Transparent Operation Fusion", section "The Paper": operators injected into
 * the running persistent kernel and updated safely while it runs).  An op
 * body is a register program of up to GPUOS_PROG_MAX_INSNS instructions that
 * the resident kernel interprets per element; defining or updating one needs
 * no compilation and no relaunch.
 *
 * Registers hold fp32 values.  r0..r7 are per element: r0..r(n_inputs-1)
 * start as the op's inputs in0[k], in1[k], in2[k] (widened exactly from
 * BF16 / F16), the rest as +0.  r8..r15 are the constants consts[0..7].
 * Instructions run in order; each writes register dst (0..7) with one fp32
 * result rounded to nearest even (no fused multiply-add).  The op's output is
 * register `result` (0..15), rounded once to the op's dtype.  Operand fields
 * an instruction does not use, and every reserved field, must be 0.
 *
 *  MOV  a        EXP  exp(a) (within the EXP op's tolerance)
 *  ADD  a + b    NEG  -a (sign flip)        LT   a < b ? 1 : 0
 *  SUB  a - b    ABS  |a| (sign cleared)    SEL  a != 0 ? b : c (NaN != 0)
 *  MUL  a * b    RELU a > 0 ? a : +0
 *  DIV  a / b (correctly rounded)
 *  MIN  the smaller of a, b; MAX the larger: a NaN operand gives NaN, and -0
 *       counts as smaller than +0 (IEEE 754-2019 minimum / maximum).
 *
 * An op's body is fixed when the op is submitted: gpuos_program_update
 * changes the body of ops submitted after it and never of ops already
 * submitted, whether or not they have started.
 *
 * With fusion on, an fp32 PROGRAM op whose body is a chain over one
 * accumulator (each instruction reads the previous result, first an input,
 * and at most an unchanged input, the result itself or, for MUL, a
 * constant; ADD, MUL, RELU, EXP, MOV only) runs as the built-in op or fused
 * micro-program doing the same fp32 operations: the same result, at the
 * built-in ops' speed.  Other programs are interpreted.
 */
#define GPUOS_PROG_MAX_INSNS 16
#define GPUOS_PROG_MAX_PROGRAMS 4096
#define GPUOS_PROG_MAX_COMPILED 256  /* distinct bodies in one compile */

typedef enum gpuos_pop {
  GPUOS_P_MOV = 0,
  GPUOS_P_ADD = 1,
  GPUOS_P_SUB = 2,
  GPUOS_P_MUL = 3,
  GPUOS_P_DIV = 4,
  GPUOS_P_MIN = 5,
  GPUOS_P_MAX = 6,
  GPUOS_P_NEG = 7,
  GPUOS_P_ABS = 8,
  GPUOS_P_RELU = 9,
  GPUOS_P_EXP = 10,
  GPUOS_P_LT = 11,
  GPUOS_P_SEL = 12,
  GPUOS_P_COUNT = 13
} gpuos_pop;

typedef struct gpuos_insn {
  uint8_t op;        /* gpuos_pop */
  uint8_t dst;       /* 0..7 */
  uint8_t a, b, c;   /* source registers 0..15 (b for binary ops and LT,
                        b and c for SEL) */
  uint8_t _reserved[3];
} gpuos_insn;        /* 8 bytes */

typedef struct gpuos_program {
  uint32_t n_insns;   /* 1..GPUOS_PROG_MAX_INSNS */
  uint32_t n_inputs;  /* 1..3 */
  uint32_t result;    /* register holding the output, 0..15 */
  uint32_t _reserved;
  float consts[8];    /* registers 8..15 */
  gpuos_insn insns[GPUOS_PROG_MAX_INSNS];
} gpuos_program;      /* 176 bytes */

/*
 * Defines a program on the context and returns its id (0, 1, 2, ... in
 * definition order) in *id_out; PROGRAM ops name it in aux[0].  The program
 * is copied.  Errors: EINVAL for a null argument, an instruction or register
 * out of range, a nonzero reserved field, or more than
 * GPUOS_PROG_MAX_PROGRAMS programs; ESTATE on a stopped context.
 */
int gpuos_program_define(gpuos_ctx* ctx, const gpuos_program* prog, uint32_t* id_out);

/*
 * Replaces the body of program `id` for ops submitted from now on (see
 * above).  Errors: EINVAL for an unknown id or a malformed program (as
 * gpuos_program_define); ESTATE on a stopped context.
 */
int gpuos_program_update(gpuos_ctx* ctx, uint32_t id, const gpuos_program* prog);

/*
 * Compiled program bodies ("GPUOS: A GPU Operating System Primitive for
 * Transparent Operation Fusion", section "The Paper": operators compiled at
 * run time and installed into the running persistent kernel, with two slots
 * so that an operator can be replaced while the kernel runs).
 *
 * gpuos_program_compile writes the current bodies of programs ids[0, n_ids)
 * (ids = NULL: every program defined so far) as straight-line code, builds
 * with hipRTC a variant of the resident kernel whose op table holds them,
 * and loads it on the context's device.  The call blocks for the compile
 * (seconds) and leaves the queue alone: the running kernel goes on.  It
 * allocates device memory for the code (refused on a static context).
 *
 * Two kernels can then serve the queue.  The built-in kernel runs every op
 * (PROGRAM ops interpreted).  The compiled variant runs PROGRAM ops whose
 * body, as of their submission, is one it compiled (in a dtype of `dtypes`),
 * and the fp32 streaming ops: NOP, COPY of 4-byte elements, ADD, MUL, RELU,
 * SCALE, EXP, SILU_MUL and fused chains of them, without views.  At a flush,
 * the context hands the queue to the compiled variant before a PROGRAM op
 * with a compiled body when every descriptor left in that flush can run
 * there, and back to the built-in kernel before a descriptor that cannot.  A
 * hand-over waits until every published op has completed, lets the running
 * kernel leave as gpuos_yield does, and launches the other kernel on the same
 * rings, so such a flush blocks for that drain.  A new compile's variant
 * replaces the previous one at the next hand-over (the previous one stays
 * loaded while it runs: two slots).  Which kernel runs an op never changes
 * its result: a compiled body performs the interpreter's fp32 operations in
 * the same order, each rounded to nearest even.
 *
 * dtypes: a mask of 1u << GPUOS_F32, 1u << GPUOS_BF16, 1u << GPUOS_F16 to
 * compile the bodies for (0 = all three).  log: if not NULL, receives the
 * compiler's messages, NUL-terminated and cut to log_bytes (empty when there
 * are none).  On a host-only context (GPUOS_DEVICE_NONE) the variant is
 * compiled for gfx950 and not loaded; flushes then count hand-overs without
 * running anything.
 * Errors: EINVAL (null context, an unknown id, no program to compile, more
 * than GPUOS_PROG_MAX_COMPILED distinct bodies, a bad mask); ESTATE (stopped or static context); ECOMPILE (hipRTC failed, or the
 * variant would not fit the resident grid: see log and gpuos_last_error);
 * EDEVICE (loading the module failed).
 */
int gpuos_program_compile(gpuos_ctx* ctx, const uint32_t* ids, uint32_t n_ids, uint32_t dtypes,
                          char* log, size_t log_bytes);

/*
 * Graph-replay comparator ("Launch Overhead and Fusion", section "Graph
 * capture": a fixed sequence of launches recorded once and replayed with a
 * single submission).  gpuos_graph_create captures into a HIP graph the
 * launches gpuos_baseline_run would issue for ops[0, n) (same tile code; with
 * fuse = 1 the same fusion pass), on device `device`; the ops' pointers,
 * sizes and scalars are fixed in the graph, the caller's array may be freed
 * on return.  gpuos_graph_launch replays the whole graph on HIP stream
 * `stream` (NULL = the legacy default stream) without synchronising; the
 * buffers must stay allocated while a replay may run.  gpuos_graph_destroy
 * frees the graph (no replay may be pending).  Errors: EINVAL (bad op, null
 * argument), EDEVICE (HIP failure).
 */
typedef struct gpuos_graph gpuos_graph;
int gpuos_graph_create(int device, const gpuos_op* ops, uint32_t n, int fuse, gpuos_graph** out);
int gpuos_graph_launch(gpuos_graph* g, void* stream);
int gpuos_graph_destroy(gpuos_graph* g);

/*
 * Launch-rate measurement ("Kernel Launch and Host-Device Interaction",
 * section "The launch path": each launch writes a packet into a queue and
 * rings a doorbell, a few microseconds per launch).  On device `device`, an
 * empty kernel (one workgroup of one wave) is launched n times back to back
 * on a new stream and then waited for once (*async_us: host time per launch),
 * then n times each followed by hipStreamSynchronize (*sync_us: time per
 * launch-and-wait round trip); both from std::chrono::steady_clock, after 100
 * untimed launches.  Errors: EINVAL (n = 0 or a null output), EDEVICE.
 */
int gpuos_launch_overhead(int device, uint32_t n, double* async_us, double* sync_us);

/*
 * Gives the GPU back to other work: waits (up to timeout_ns, < 0 = forever)
 * until every submitted op has completed, then lets the resident kernel leave
 * at once instead of after idle_exit_ms, and returns once its launch has
 * ended.  While the kernel is resident it holds the register files of every
 * compute unit, so kernels launched by other code (PyTorch included) cannot
 * start; the pages' critique of persistent kernels ("The Counter" on the
 * GPUOS page) is exactly that.  The next gpuos_flush with work relaunches
 * the kernel.  Returns 0 at once on a host-only or already parked context.
 * Errors: ESTATE (stopped), ETIMEDOUT, EDEVICE.
 */
int gpuos_yield(gpuos_ctx* ctx, int64_t timeout_ns);

/* ABI version of the loaded library (GPUOS_ABI_VERSION). */
int gpuos_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif
