/*
 * gpuos_debug.h - host-only inspection hooks of the gpuos runtime.
 *
 * These entry points let the host half of the runtime (validation, hazard
 * dependencies, the fusion pass, ring publication and back-pressure) be
 * exercised without a GPU: a context created with device = GPUOS_DEVICE_NONE
 * keeps its rings in ordinary host memory, launches nothing, and never
 * completes an op unless the caller retires it with gpuos_debug_retire.  The
 * rings and their publication protocol are the ones described in gpuos.h
 * (after "Kernel Launch and Host-Device Interaction", section "The launch
 * path": commands written into a ring in host memory, then a doorbell).
 */
#ifndef GPUOS_DEBUG_H
#define GPUOS_DEBUG_H

#include "gpuos.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Device id that creates a host-only context (no HIP call is made). */
#define GPUOS_DEVICE_NONE (-1)

/*
 * Copies the 256-byte device descriptor published with sequence `seq` in ring
 * `ring` (0 = best effort, 1 = latency critical) into out (256 bytes, caller
 * owned).  Errors: EINVAL if seq was never published or its slot has been
 * reused.  Works on any context.
 */
int gpuos_debug_read_desc(gpuos_ctx* ctx, int ring, uint64_t seq, void* out);

/* Last sequence published in `ring` (0 if none). */
uint64_t gpuos_debug_published(gpuos_ctx* ctx, int ring);

/* Device sequence (in *ring_out / *seq_out) that carries user op `id`.
 * Errors: EINVAL if id is unknown, EAGAIN if it is still staged. */
int gpuos_debug_seq_of(gpuos_ctx* ctx, uint64_t id, int* ring_out, uint64_t* seq_out);

/*
 * Host-only contexts: marks every descriptor of `ring` up to sequence `upto`
 * as retired, as the resident kernel would.  Errors: ESTATE on a device
 * context, EINVAL if upto is beyond the last published sequence.
 */
int gpuos_debug_retire(gpuos_ctx* ctx, int ring, uint64_t upto);

/*
 * Host consumer: a thread that plays the resident kernel on a host-only
 * context, for tests of the host runtime under concurrency (back-pressure on
 * a full ring, ring wraparound, the order dependencies impose).  After
 * gpuos_debug_consumer_attach, a full ring or a pending cross-ring dependency
 * blocks the producer until the consumer retires enough (30 s at most, then
 * ETIMEDOUT) instead of failing with EAGAIN, and gpuos_sync waits for the
 * consumer.  The three consumer calls may run on another thread, concurrently
 * with the producer's calls, and touch only what the device would:
 *  - gpuos_debug_consumer_tail: the ring's published tail (acquire load; 0
 *    for a device context or a bad argument);
 *  - gpuos_debug_consumer_read: copies the 256-byte descriptor of sequence
 *    seq from its ring slot into out (caller owned), after checking the
 *    slot's sequence and check words (EINVAL if the slot holds another
 *    sequence); seq must be at or below the tail, and not yet retired;
 *  - gpuos_debug_consumer_retire: advances the ring's in-order retire cursor
 *    to upto (release store; EINVAL beyond the published tail).
 * Errors: ESTATE on a device context.  One consumer thread per context.
 */
int gpuos_debug_consumer_attach(gpuos_ctx* ctx);
uint64_t gpuos_debug_consumer_tail(gpuos_ctx* ctx, int ring);
int gpuos_debug_consumer_read(gpuos_ctx* ctx, int ring, uint64_t seq, void* out);
int gpuos_debug_consumer_retire(gpuos_ctx* ctx, int ring, uint64_t upto);

/*
 * Copies the execution counts of tickets [0, n) of `ring` into out (n
 * uint32 entries, caller owned), for a context created with
 * config.tile_counts >= n.  Ticket i is the i-th tile published to the ring
 * (descriptor s owns the tickets from the sum of the tile counts of the
 * descriptors before it); each count is the number of times a wave ran that
 * tile, which the scheduler's claim rule makes exactly 1 ("LithOS", section
 * 5.4, Algorithm 1: non-overlapping block ranges, so every block runs once).
 * Call after gpuos_sync; reads device memory while the kernel may run.
 * Errors: EINVAL (bad argument, n above tile_counts), ESTATE (counting off
 * or host-only context), EDEVICE.
 */
int gpuos_debug_tile_counts(gpuos_ctx* ctx, int ring, uint32_t* out, uint32_t n);

/*
 * The program-body source that the last gpuos_program_compile call wrote
 * (the generated gpuos_rtc_bodies.h): copies it, NUL-terminated and cut to
 * n bytes, into buf (may be NULL) and returns its length plus 1 (1 if there
 * has been no compile, 0 for a null context).
 */
size_t gpuos_debug_rtc_source(gpuos_ctx* ctx, char* buf, size_t n);

#ifdef __cplusplus
}
#endif
#endif
