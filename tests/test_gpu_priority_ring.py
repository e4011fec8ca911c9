"""GPU: the priority ring's direct claims.

The reserved waves take latency-critical descriptors straight from the host
ring and run all of a descriptor's tiles themselves.  Small streaming ops are
planned as one tile; these tests cover the other shapes ("LithOS", section
5.3, the priority scheduler; the priority ring of this library):

* latency-critical ops of several tiles (elementwise ops past 2^16 elements
  with a ragged tail, row sums and softmax over many rows, multi-row RMSNorm),
  chained through latency-critical dependencies and interleaved with
  best-effort ops: every output against the oracle, and every ticket of both
  rings run exactly once;
* compiled program bodies on the priority ring: the queue is handed to the
  compiled variant, whose reserved waves run the latency-critical programs.
"""

import numpy as np
import pytest

import oracle
from persistent_fusion_amd import gpuos, runner, workloads
from persistent_fusion_amd.workloads import Op, Program, Ref, Workload

pytestmark = pytest.mark.gpu


def _need_gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gpuos.lib()


def say(msg):
    print(msg, flush=True)


def check(wl, got):
    want, scales = oracle.run(wl, scales=True)
    for name in wl.outputs:
        r = oracle.compare(got[name], want[name], wl.dtypes[name], scales.get(name))
        assert r.ok, f"{wl.name}/{name}: {r}"


def _multi_tile_workload(seed):
    rng = np.random.default_rng(seed)
    bufs, dts, ops = {}, {}, []

    def buf(name, n, dt="f32", zero=False):
        v = np.zeros(n, np.float32) if zero else rng.uniform(-2, 2, n).astype(np.float32)
        bufs[name] = workloads.f32_to_bf16_trunc(v) if dt == "bf16" else v
        dts[name] = dt
        return Ref(name)

    n1, n2 = 200_003, 70_001
    a, b = buf("a", n1), buf("b", n1)
    hb, hc = buf("hb", n2, "bf16"), buf("hc", n2, "bf16")
    rows, L = 37, 1000
    s = buf("s", rows * L)
    xr = buf("xr", 64 * 896, "bf16")
    g = buf("g", 896, "bf16")
    big = buf("big", 1 << 20)
    # latency-critical chain: y1 = a + b, y2 = relu(y1) (reads y1), y3 = exp(y2 * 0.25)
    ops.append(Op("add", buf("y1", n1, zero=True), (a, b), n=n1, lc=True))
    ops.append(Op("mul", buf("bo0", 1 << 20, zero=True), (big, big), n=1 << 20))           # best effort
    ops.append(Op("relu", buf("y2", n1, zero=True), (Ref("y1"),), n=n1, lc=True))
    ops.append(Op("scale", buf("y3", n1, zero=True), (Ref("y2"),), n=n1, alpha=0.25, lc=True))
    ops.append(Op("exp", buf("y4", n1, zero=True), (Ref("y3"),), n=n1, lc=True))
    ops.append(Op("add", buf("h1", n2, "bf16", zero=True), (hb, hc), n=n2, dtype="bf16", lc=True))
    ops.append(Op("relu", buf("bo1", 1 << 20, zero=True), (big,), n=1 << 20))                # best effort
    ops.append(Op("row_sum", buf("rs", rows, zero=True), (s,), n=rows * L, rows=rows, row_len=L, lc=True))
    ops.append(Op("row_softmax", buf("sm", rows * L, zero=True), (s,), n=rows * L, rows=rows, row_len=L,
                  lc=True))
    ops.append(Op("rmsnorm", buf("rn", 64 * 896, "bf16", zero=True), (xr,), g, n=64 * 896, dtype="bf16",
                  rows=64, row_len=896, eps=float(np.float32(1e-6)), lc=True))
    outs = ["y1", "y2", "y3", "y4", "h1", "rs", "sm", "rn", "bo0", "bo1"]
    return Workload("lc_multi_tile", bufs, dts, ops, outputs=outs)


def test_multi_tile_latency_critical_ops():
    _need_gpu()
    say("multi-tile latency-critical ops")
    wl = _multi_tile_workload(seed=301)
    tensors = runner.to_device(wl, 0)
    addr = runner.addr_fn(tensors, wl)
    ctx = gpuos.Context(0, priority=1, tile_counts=1 << 16)
    try:
        runner.submit_workload(ctx, wl, addr)
        ctx.sync(0, 60.0)
        counts = {r: (ctx.tickets(r), np.array(ctx.tile_counts(r, ctx.tickets(r) + 64))) for r in (0, 1)}
    finally:
        ctx.destroy()
    n1 = counts[1][0]
    say(f"  ring 1: {n1} tickets")
    assert n1 > 8, "the latency-critical ops should span several tiles"
    for ring, (n, c) in counts.items():
        assert np.all(c[:n] == 1), f"ring {ring}: tickets run {sorted(set(c[:n].tolist()))} times"
        assert np.all(c[n:] == 0), f"ring {ring}: unpublished tickets ran"
    check(wl, runner.download(tensors, wl, wl.outputs))


def test_compiled_programs_on_the_priority_ring():
    _need_gpu()
    say("compiled programs on the priority ring")
    rng = np.random.default_rng(302)
    n = 8192
    bufs, ops = {}, []
    clamp = Program((("max", 3, 0, 8), ("min", 3, 3, 9), ("mul", 3, 3, 1)), 2, 3, consts=(-0.5, 0.5))
    for k in range(40):
        for nm in (f"a{k}", f"b{k}"):
            bufs[nm] = rng.uniform(-1, 1, n).astype(np.float32)
        bufs[f"y{k}"] = np.zeros(n, np.float32)
        if k % 4 == 0:
            ops.append(Op("program", Ref(f"y{k}"), (Ref(f"a{k}"), Ref(f"b{k}")), n=n, prog=clamp, lc=True))
        else:
            ops.append(Op("mul", Ref(f"y{k}"), (Ref(f"a{k}"), Ref(f"b{k}")), n=n))
    wl = Workload("lc-compiled", bufs, {k: "f32" for k in bufs}, ops, outputs=[f"y{k}" for k in range(40)])
    wl.groups = [(0, 40)]
    st = {}
    got = runner.run_resident(wl, priority=1, fusion=2, compile_programs=True, stats=st)
    say(f"  kernel switches {st['kernel_switches']}, compiled {st['programs_compiled']}")
    assert st["programs_compiled"] == 10
    assert st["kernel_switches"] == 1
    check(wl, got)
