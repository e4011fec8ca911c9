"""GPU: waits that time out, and destroying a context with work queued.

Every condition is forced from the host with the SPIN debug op, whose tile
waits a bounded time (at most 10 ms per tile) and then ends normally, so every
kernel in these tests exits on its own:

* gpuos_sync with a time limit shorter than the queued spins returns
  ETIMEDOUT, the last op stays pending, and a later wait completes them;
* gpuos_destroy with ops queued drains them first: their results are final
  and equal the oracle's;
* gpuos_destroy with a time limit shorter than the queue leaks the context
  (ETIMEDOUT) instead of freeing memory under the running kernel; the kernel
  drains the queue and leaves by itself, and the GPU stays usable.
"""

import time

import pytest

import oracle
from persistent_fusion_amd import gpuos, runner, workloads

pytestmark = pytest.mark.gpu

SPIN_NS = 10_000_000  # the longest spin one tile takes


def _need_gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gpuos.lib()


def say(msg):
    print(msg, flush=True)


def spins(k, chained=True):
    """k SPIN ops of 10 ms; chained, each waits for the one before."""
    return (gpuos.GpuosOp * k)(*[gpuos.make_op("spin", 0, dims=(SPIN_NS,), deps=([-1] if chained and i else []))
                                 for i in range(k)])


def test_sync_times_out_while_an_op_spins():
    _need_gpu()
    say("sync with a 1 ms limit on three chained 10 ms spins")
    with gpuos.Context(0) as c:
        ids = c.submit(spins(3))
        with pytest.raises(gpuos.GpuosError) as e:
            c.sync(0, 0.001)
        assert e.value.status == gpuos.ETIMEDOUT
        assert not c.query(ids[-1])  # the last spin cannot have ended yet
        c.sync(0, 10.0)
        assert all(c.query(i) for i in ids)


def test_destroy_drains_queued_ops():
    _need_gpu()
    say("destroy with a spin and a 200-op queue pending")
    wl = workloads.gen_elementwise_queue(seed=5, n_ops=200, n=4096)
    tensors = runner.to_device(wl, 0)
    addr = runner.addr_fn(tensors, wl)
    arr = gpuos.encode_ops(wl.ops, 0, len(wl.ops), addr, {})
    c = gpuos.Context(0)
    c.submit(spins(1))
    c.submit(arr, len(wl.ops))
    c.destroy(30.0)  # flushes, waits for every op, then stops the kernel
    got = runner.download(tensors, wl, wl.outputs)
    want = oracle.run(wl)
    for name in wl.outputs:
        r = oracle.compare(got[name], want[name], wl.dtypes[name])
        assert r.ok, f"{name}: {r}"


def test_destroy_timeout_leaks_and_the_kernel_leaves_by_itself():
    _need_gpu()
    say("destroy with a 1 ms limit on five chained 10 ms spins")
    c = gpuos.Context(0)
    c.submit(spins(5))
    with pytest.raises(gpuos.GpuosError) as e:
        c.destroy(0.001)
    assert e.value.status == gpuos.ETIMEDOUT and "leaked" in str(e.value)
    # the leaked kernel drains its 50 ms queue, sees the stop request and
    # leaves; a new context then gets the whole GPU and runs normally
    time.sleep(0.3)
    say("a new context after the leak")
    wl = workloads.gen_elementwise_queue(seed=6, n_ops=100, n=4096)
    got = runner.run_resident(wl, device=0)
    want = oracle.run(wl)
    for name in wl.outputs:
        r = oracle.compare(got[name], want[name], wl.dtypes[name])
        assert r.ok, f"{name}: {r}"
