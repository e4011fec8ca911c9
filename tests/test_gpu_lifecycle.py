"""GPU tests of the resident kernel's lifecycle: the kernel leaves after an
idle period and the runtime launches it again when work arrives, without
losing or repeating any op.  Results are checked bit for bit against the
oracle (the 1,000-op elementwise queue: ADD, MUL, RELU, SCALE)."""

import random
import time

import pytest

import oracle
from persistent_fusion_amd import gpuos, runner, workloads

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def _check_queue(wl, tensors):
    got = runner.download(tensors, wl, wl.outputs)
    want = oracle.run(wl)
    for name in wl.outputs:
        r = oracle.compare(got[name], want[name], "f32")
        assert r.ok, f"{name}: {r}"


def _submit_range(ctx, wl, addr, g0, g1, id_of):
    arr = gpuos.encode_ops(wl.ops, g0, g1, addr, id_of)
    ids = ctx.submit(arr, g1 - g0)
    for k, i in enumerate(range(g0, g1)):
        id_of[i] = ids[k]


def test_idle_exit_and_relaunch():
    say("lifecycle: idle exit between chunks")
    wl = workloads.gen_elementwise_queue(seed=3)
    t = runner.to_device(wl)
    addr = runner.addr_fn(t, wl)
    ctx = gpuos.Context(0, idle_exit_ms=2)
    try:
        id_of = {}
        n = len(wl.ops)
        for k in range(10):
            _submit_range(ctx, wl, addr, k * n // 10, (k + 1) * n // 10, id_of)
            ctx.flush()
            time.sleep(0.02)  # ten times the idle limit: the kernel leaves
        ctx.sync(0, 30.0)
        ctx.stop()
        st = ctx.stats()
    finally:
        ctx.destroy()
    say(f"launches {st['launches']} kernel_ns {st['kernel_ns']}")
    assert st["launches"] >= 5
    assert st["kernel_ns"] > 0
    _check_queue(wl, t)


def test_flushes_around_the_idle_limit():
    """Flushes land just before, at and after the moment the kernel decides
    to leave; every op must still run exactly once."""
    say("lifecycle: flushes around the idle limit")
    wl = workloads.gen_elementwise_queue(seed=4)
    t = runner.to_device(wl)
    addr = runner.addr_fn(t, wl)
    rng = random.Random(0)
    ctx = gpuos.Context(0, idle_exit_ms=1)
    try:
        id_of = {}
        for i in range(300):
            _submit_range(ctx, wl, addr, i, i + 1, id_of)
            ctx.flush()
            time.sleep(rng.uniform(0.0005, 0.0015))
        _submit_range(ctx, wl, addr, 300, len(wl.ops), id_of)
        ctx.sync(0, 30.0)
        st = ctx.stats()
    finally:
        ctx.destroy()
    say(f"launches {st['launches']}")
    assert st["launches"] >= 2
    _check_queue(wl, t)


def test_query_relaunches():
    """gpuos_query alone (no sync) brings an idled-out kernel back."""
    say("lifecycle: query after idle exit")
    wl = workloads.gen_elementwise_queue(seed=5)
    t = runner.to_device(wl)
    addr = runner.addr_fn(t, wl)
    ctx = gpuos.Context(0, idle_exit_ms=1)
    try:
        id_of = {}
        _submit_range(ctx, wl, addr, 0, 500, id_of)
        ctx.flush()
        time.sleep(0.02)
        _submit_range(ctx, wl, addr, 500, len(wl.ops), id_of)
        ctx.flush()
        last = id_of[len(wl.ops) - 1]
        t0 = time.time()
        while not ctx.query(last):
            assert time.time() - t0 < 30.0, "ops did not complete"
            time.sleep(0.0001)
        st = ctx.stats()
    finally:
        ctx.destroy()
    assert st["launches"] >= 2
    _check_queue(wl, t)


def test_never_idle_exit():
    say("lifecycle: idle exit off")
    wl = workloads.gen_elementwise_queue(seed=6)
    t = runner.to_device(wl)
    addr = runner.addr_fn(t, wl)
    ctx = gpuos.Context(0, idle_exit_ms=0xFFFFFFFF)
    try:
        id_of = {}
        _submit_range(ctx, wl, addr, 0, 500, id_of)
        ctx.flush()
        time.sleep(0.05)
        _submit_range(ctx, wl, addr, 500, len(wl.ops), id_of)
        ctx.sync(0, 30.0)
        st = ctx.stats()
    finally:
        ctx.destroy()
    assert st["launches"] == 1
    _check_queue(wl, t)


def test_yield_gives_the_gpu_back_and_the_next_flush_relaunches():
    """gpuos_yield: once the queue is done the kernel leaves at once (a
    PyTorch kernel launched next runs without waiting for the idle period),
    and the next flush relaunches it without losing or repeating an op."""
    import torch

    say("lifecycle: yield")
    wl = workloads.gen_elementwise_queue(seed=5)
    t = runner.to_device(wl)
    addr = runner.addr_fn(t, wl)
    x = torch.randn(1024, device="cuda")
    ctx = gpuos.Context(0, idle_exit_ms=60000)  # no idle exit: only yield ends a launch
    try:
        id_of = {}
        n = len(wl.ops)
        waits = []
        for k in range(4):
            _submit_range(ctx, wl, addr, k * n // 4, (k + 1) * n // 4, id_of)
            ctx.flush()
            ctx.yield_gpu()
            ctx.yield_gpu()  # parked: returns at once
            t0 = time.perf_counter()
            y = x * 2.0  # a torch kernel while the context is parked
            torch.cuda.synchronize()
            waits.append(time.perf_counter() - t0)
            assert torch.equal(y, x * 2.0)
        ctx.sync(0, 30.0)
        ctx.stop()
        st = ctx.stats()
    finally:
        ctx.destroy()
    say(f"launches {st['launches']}, torch waits {[round(w * 1e3, 2) for w in waits]} ms")
    assert st["launches"] == 4
    assert max(waits) < 1.0  # far below the 60 s idle period
    _check_queue(wl, t)
