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

#ifdef __cplusplus
}
#endif
#endif
