"""GPU: gpuos_create_static, the context for callers that cannot allocate.

Its scheduler state lives in the library's static device scratch and its
rings in a pinned workspace the caller brings.  Two calls in a row (create,
run a queue, destroy), the second with a smaller ring and a smaller input,
each checked against the same queues run on a context from gpuos_create
(bit for bit) and against the oracle; a second static context while one is
alive is refused, as is a ring larger than the scratch holds.
"""

import ctypes as C

import numpy as np
import pytest

import oracle
from persistent_fusion_amd import gpuos, runner, workloads

pytestmark = pytest.mark.gpu

HIP_HOST_MALLOC_MAPPED = 0x2
HIP_HOST_MALLOC_COHERENT = 0x40000000


def say(msg):
    print(msg, flush=True)


class PinnedWorkspace:
    """Pinned, device-mapped, coherent host memory from hipHostMalloc (the
    caller's allocation, made before the no-allocation entry point runs)."""

    def __init__(self, nbytes):
        self.hip = C.CDLL("libamdhip64.so")
        self.hip.hipHostMalloc.argtypes = [C.POINTER(C.c_void_p), C.c_size_t, C.c_uint]
        self.hip.hipHostFree.argtypes = [C.c_void_p]
        self.ptr = C.c_void_p()
        rc = self.hip.hipHostMalloc(C.byref(self.ptr), nbytes,
                                    HIP_HOST_MALLOC_MAPPED | HIP_HOST_MALLOC_COHERENT)
        assert rc == 0 and self.ptr.value, f"hipHostMalloc: {rc}"
        self.nbytes = nbytes

    def free(self):
        if self.ptr.value:
            self.hip.hipHostFree(self.ptr)
            self.ptr = C.c_void_p()


def _need_gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gpuos.lib()


def _run(wls, **ctx_kw):
    """Runs the workloads one after another on one context; returns their
    outputs."""
    outs = []
    ctx = gpuos.Context(0, **ctx_kw)
    try:
        for wl in wls:
            tensors = runner.to_device(wl, 0)
            runner.submit_workload(ctx, wl, runner.addr_fn(tensors, wl))
            ctx.sync(0, 60.0)
            outs.append(runner.download(tensors, wl, wl.outputs))
    finally:
        ctx.destroy()
    return outs


@pytest.mark.parametrize("call", [0, 1])
def test_static_context_matches_the_allocating_one(call):
    _need_gpu()
    slots, wls = [
        (4096, [workloads.gen_elementwise_queue(seed=10), workloads.gen_fused_chain(seed=10, n=1_000_003),
                workloads.gen_decode(seed=10, layers=2, tokens=2)]),
        (256, [workloads.gen_elementwise_queue(seed=11, n_ops=200), workloads.gen_fused_chain(seed=11, n=65_541)]),
    ][call]
    say(f"static context, call {call}: {slots} slots, {[wl.name for wl in wls]}")
    ws = PinnedWorkspace(gpuos.static_host_bytes(slots))
    try:
        got = _run(wls, host_ws=ws.ptr.value, host_ws_bytes=ws.nbytes, ring_slots=slots)
    finally:
        ws.free()
    want = _run(wls, ring_slots=slots)
    for wl, g, w in zip(wls, got, want):
        ref, scales = oracle.run(wl, scales=True)
        for name in wl.outputs:
            assert np.array_equal(g[name].view(np.uint8), w[name].view(np.uint8)), (wl.name, name)
            r = oracle.compare(g[name], ref[name], wl.dtypes[name], scales.get(name))
            assert r.ok, f"{wl.name}/{name}: {r}"


def test_static_context_limits():
    _need_gpu()
    say("static context limits")
    ws = PinnedWorkspace(gpuos.static_host_bytes(1024))
    try:
        big = gpuos.static_host_bytes(8192)
        with pytest.raises(gpuos.GpuosError, match="EINVAL"):
            gpuos.Context(0, host_ws=ws.ptr.value, host_ws_bytes=big, ring_slots=8192)
        with pytest.raises(gpuos.GpuosError, match="EINVAL"):  # workspace too small
            gpuos.Context(0, host_ws=ws.ptr.value, host_ws_bytes=ws.nbytes, ring_slots=2048)
        ctx = gpuos.Context(0, host_ws=ws.ptr.value, host_ws_bytes=ws.nbytes, ring_slots=1024)
        try:
            other = PinnedWorkspace(gpuos.static_host_bytes(1024))
            try:
                with pytest.raises(gpuos.GpuosError, match="ESTATE"):
                    gpuos.Context(0, host_ws=other.ptr.value, host_ws_bytes=other.nbytes, ring_slots=1024)
            finally:
                other.free()
        finally:
            ctx.destroy()
        # the device is free again
        ctx = gpuos.Context(0, host_ws=ws.ptr.value, host_ws_bytes=ws.nbytes, ring_slots=1024)
        ctx.destroy()
    finally:
        ws.free()
