"""GPU: ops at the largest extents the runtime accepts.  Kernels address an
operand with 32-bit byte offsets, so an operand may span at most 0xFFF00000
bytes (4 GiB - 1 MiB) and n is at most 2^30: these tests run an fp32 ADD and
the fused chain relu(a*x + b) one element short of the fp32 limit (so the
last vector is ragged) and a bf16 ADD at n = 2^30.  Inputs are seeded and
drawn on the device; outputs are checked against the oracle bit for bit on
samples (both ends of the range and random positions in between), which the
oracle computes one by one from the same input values."""

import numpy as np
import pytest

import oracle
from persistent_fusion_amd import gpuos
from persistent_fusion_amd.workloads import Op, Ref, Workload

pytestmark = pytest.mark.gpu

N_F32 = 0xFFF00000 // 4 - 1  # 1,073,479,679 fp32 elements: the largest extent, minus one
N_BF16 = 1 << 30


def _need_gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gpuos.lib()


def say(msg):
    print(msg, flush=True)


def _samples(n, seed):
    rng = np.random.default_rng(seed)
    idx = np.concatenate([np.arange(0, 8192), np.arange(n - 8192, n), rng.integers(0, n, 65536)])
    return np.unique(idx)


def _host(t, idx, bits=False):
    """Elements idx of device tensor t, as a numpy array (uint16 bits for bf16)."""
    import torch

    sel = t[torch.from_numpy(idx).to(t.device)]
    if t.dtype == torch.bfloat16:
        return sel.view(torch.int16).cpu().numpy().view(np.uint16)
    return sel.cpu().numpy()


def _rand(n, seed, dtype):
    import torch

    g = torch.Generator(device="cuda").manual_seed(seed)
    return (torch.rand(n, generator=g, device="cuda") * 4 - 2).to(dtype)


def test_largest_fp32_add_and_fused_chain():
    _need_gpu()
    import torch

    n = N_F32
    say(f"limits: fp32 n={n}")
    x, a, b = (_rand(n, s, torch.float32) for s in (70, 71, 72))
    y, s1, t1, t2 = (torch.empty(n, device="cuda") for _ in range(4))
    P = lambda t: t.data_ptr()
    ops = (gpuos.GpuosOp * 4)(
        gpuos.make_op("add", P(s1), [P(x), P(a)], n=n),
        gpuos.make_op("mul", P(t1), [P(a), P(x)], n=n, flags=gpuos.FLAG_TRANSIENT),
        gpuos.make_op("add", P(t2), [P(t1), P(b)], n=n, flags=gpuos.FLAG_TRANSIENT),
        gpuos.make_op("relu", P(y), [P(t2)], n=n),
    )
    ctx = gpuos.Context(0)
    try:
        ctx.submit(ops)
        ctx.sync(0, 60.0)
        st = ctx.stats()
    finally:
        ctx.destroy()
    assert st["ops_fused"] == 2  # the chain ran as one fused pass
    idx = _samples(n, 73)
    hx, ha, hb = (_host(t, idx) for t in (x, a, b))
    k = len(idx)
    bufs = {"x": hx, "a": ha, "b": hb, "s1": np.zeros(k, np.float32), "t1": np.zeros(k, np.float32),
            "t2": np.zeros(k, np.float32), "y": np.zeros(k, np.float32)}
    wl = Workload("limits", bufs, {key: "f32" for key in bufs}, [
        Op("add", Ref("s1"), (Ref("x"), Ref("a")), n=k),
        Op("mul", Ref("t1"), (Ref("a"), Ref("x")), n=k),
        Op("add", Ref("t2"), (Ref("t1"), Ref("b")), n=k),
        Op("relu", Ref("y"), (Ref("t2"),), n=k),
    ])
    want = oracle.run(wl)
    for name, t in (("s1", s1), ("y", y)):
        got = _host(t, idx)
        assert np.array_equal(got.view(np.uint32), want[name].view(np.uint32)), name


def test_largest_bf16_add():
    _need_gpu()
    import torch

    n = N_BF16
    say(f"limits: bf16 n={n}")
    x, a = (_rand(n, s, torch.bfloat16) for s in (74, 75))
    y = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    ops = (gpuos.GpuosOp * 1)(gpuos.make_op("add", y.data_ptr(), [x.data_ptr(), a.data_ptr()], n=n,
                                            dtype="bf16"))
    ctx = gpuos.Context(0)
    try:
        ctx.submit(ops)
        ctx.sync(0, 60.0)
    finally:
        ctx.destroy()
    idx = _samples(n, 76)
    k = len(idx)
    bufs = {"x": _host(x, idx), "a": _host(a, idx), "y": np.zeros(k, np.uint16)}
    wl = Workload("limits-bf16", bufs, {key: "bf16" for key in bufs},
                  [Op("add", Ref("y"), (Ref("x"), Ref("a")), n=k, dtype="bf16")])
    want = oracle.run(wl)["y"]
    assert np.array_equal(_host(y, idx), want)
