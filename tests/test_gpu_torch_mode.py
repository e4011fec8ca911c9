"""GPU: the PyTorch front end (eager elementwise ops queued into the resident
kernel).  Results are compared with the same program run by PyTorch itself:
bit for bit for ops with exactly rounded results (add, mul, scale, relu,
copy; torch rounds them the same way), within the exp tolerance otherwise."""

import numpy as np
import pytest

from persistent_fusion_amd import gpuos

pytestmark = pytest.mark.gpu


def _need_gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gpuos.lib()


def say(msg):
    print(msg, flush=True)


def _program(torch, x, b, s, dtype):
    """A small eager program: broadcasts, in-place ops, a transpose, a scalar."""
    y = x * b                # [R, C] * [C]
    y = y + x                # plain
    y.relu_()                # in place
    z = y.t() * s            # transposed [C, R] * [R]
    z = z * 0.5              # scalar -> SCALE
    w = z.clone()
    w.add_(z)
    if dtype != torch.int32:
        e = (w * 0.01).exp()
    else:
        e = w
    return y, z, w, e


@pytest.mark.parametrize("dtype_name", ["float32", "bfloat16", "float16", "int32"])
def test_mode_matches_eager(dtype_name):
    _need_gpu()
    import torch

    from persistent_fusion_amd.torch_mode import GpuosMode

    say(f"torch mode {dtype_name}")
    dtype = getattr(torch, dtype_name)
    g = torch.Generator(device="cpu").manual_seed(60)
    R, Cn = 37, 300

    def draw(*shape):
        if dtype == torch.int32:
            return torch.randint(-1000, 1000, shape, generator=g, dtype=torch.int32).cuda()
        return torch.randn(*shape, generator=g).to(dtype).cuda()

    x, b, s = draw(R, Cn), draw(Cn), draw(R)
    want = _program(torch, x, b, s if dtype != torch.int32 else s, dtype) if dtype != torch.int32 else None
    if dtype == torch.int32:
        # torch's int32 mul by 0.5 promotes to float; the program keeps ints
        def prog(x, b, s):
            y = x * b
            y = y + x
            y.relu_()
            z = y.t() * s
            w = z.clone()
            w.add_(z)
            return y, z, w
        want = prog(x, b, s)
    mode = GpuosMode(0)
    try:
        with mode:
            got = prog(x, b, s) if dtype == torch.int32 else _program(torch, x, b, s, dtype)
    finally:
        mode.close()
    # every op is queued (the transpose only makes a view): nothing waits
    assert mode.stats["queued"] >= 6 and mode.stats["passed_through"] == 0, mode.stats
    assert mode.stats["metadata"] >= 1, mode.stats
    for k, (gt, wt) in enumerate(zip(got, want)):
        if k == 3 and dtype != torch.int32:  # exp: within the tolerance class
            rt = {torch.float32: 1e-5, torch.bfloat16: 1e-2, torch.float16: 2e-3}[dtype]
            assert torch.allclose(gt.float(), wt.float(), rtol=rt, atol=0), k
        else:
            assert torch.equal(gt, wt), k


def test_mode_orders_around_torch_ops_and_keeps_memory():
    """PyTorch ops between queued ops see final values; temporaries freed by
    Python stay allocated until the queue has run."""
    _need_gpu()
    import torch

    from persistent_fusion_amd.torch_mode import GpuosMode

    say("torch mode with torch ops in between")
    torch.manual_seed(61)
    a = torch.randn(64, 64, device="cuda")
    want_t = a
    for _ in range(20):
        want_t = torch.relu(want_t * 0.9 + a)
        want_t = want_t @ a * 0.01  # a matmul: not intercepted
    mode = GpuosMode(0)
    try:
        with mode:
            t = a
            for _ in range(20):
                t = torch.relu(t * 0.9 + a)
                t = t @ a * 0.01
            got = t.clone()
    finally:
        mode.close()
    assert mode.stats["queued"] > 40 and mode.stats["syncs"] >= 20
    assert torch.equal(got, want_t)


@pytest.mark.parametrize("dtype_name", ["float32", "bfloat16", "float16"])
def test_ops_without_an_opcode_run_as_programs(dtype_name):
    """sub, div, neg, abs and number add/sub/rsub become programs defined at
    run time; their results are PyTorch's, bit for bit."""
    _need_gpu()
    import torch

    from persistent_fusion_amd.torch_mode import GpuosMode

    say(f"torch mode programs {dtype_name}")
    dtype = getattr(torch, dtype_name)
    g = torch.Generator(device="cpu").manual_seed(62)
    x = torch.randn(5000, generator=g).to(dtype).cuda()
    y = (torch.rand(5000, generator=g) + 0.5).to(dtype).cuda()

    def prog(x, y):
        a = x - y
        b = a / y
        c = -b
        d = c.abs()
        e = d + 1.25
        f = e - 3
        h = 1 - f
        h.sub_(x)
        h.div_(y)
        return a, b, c, d, e, f, h

    want = prog(x, y)
    mode = GpuosMode(0)
    try:
        with mode:
            got = prog(x, y)
            got2 = prog(x, y)  # the same bodies and constants again: no new programs
    finally:
        mode.close()
    assert mode.stats["programs"] == 18 and mode.stats["passed_through"] == 0, mode.stats
    assert len(mode._pids) == 7, mode._pids  # sub, div, neg, abs, +1.25, -3, 1-x
    for k, (gt, g2, wt) in enumerate(zip(got, got2, want)):
        assert torch.equal(gt, wt) and torch.equal(g2, wt), k


def test_host_ops_do_not_wait_and_kept_tensors_are_bounded():
    """CPU-only ops inside the mode neither wait for the queue nor make the
    resident kernel leave; a long run of queued ops waits for the queue
    whenever max_kept tensors are held, and the results stay PyTorch's."""
    _need_gpu()
    import torch

    from persistent_fusion_amd.torch_mode import GpuosMode

    say("torch mode host ops and kept bound")
    torch.manual_seed(63)
    x = torch.randn(4096, device="cuda")
    mode = GpuosMode(0, batch=16, max_kept=200)
    try:
        with mode:
            y = x * 0.5
            c = torch.arange(10) * 3          # host only
            d = c + 1
            t = y
            for _ in range(300):
                t = t * 0.999 + x
            launches_inside = mode.ctx.stats()["launches"]
        got_y, got_t = y.clone(), t.clone()
    finally:
        mode.close()
    want_t = x * 0.5
    for _ in range(300):
        want_t = want_t * 0.999 + x
    assert mode.stats["host_ops"] >= 2 and mode.stats["passed_through"] == 0, mode.stats
    assert launches_inside == 1  # no yield happened for the host ops
    assert mode.stats["syncs"] >= 3  # the kept-tensor bound forced waits
    assert torch.equal(d, torch.arange(10) * 3 + 1)
    assert torch.equal(got_y, x * 0.5) and torch.equal(got_t, want_t)


@pytest.mark.parametrize("dtype_name", ["float32", "bfloat16"])
def test_contiguous_transposes_are_queued(dtype_name):
    """x.t().contiguous() and a batched x.transpose(1, 2).contiguous() are
    queued as transposed COPYs (ragged blocks included) and equal PyTorch's
    results bit for bit; a default clone of a transpose keeps the
    transposed layout, as in PyTorch."""
    _need_gpu()
    import torch

    from persistent_fusion_amd.torch_mode import GpuosMode

    dtype = getattr(torch, dtype_name)
    say(f"torch mode: contiguous transposes {dtype_name}")
    g = torch.Generator(device="cuda").manual_seed(7)
    x = torch.randn(300, 257, generator=g, device="cuda").to(dtype)
    xb = torch.randn(3, 136, 72, generator=g, device="cuda").to(dtype)
    mode = GpuosMode(0)
    try:
        with mode:
            t2 = x.t().contiguous()
            t3 = xb.transpose(1, 2).contiguous()
            queued = mode.stats["queued"]
            kept = x.t().clone()
    finally:
        mode.close()
    assert queued == 2 and mode.stats["queued"] == 3 and mode.stats["passed_through"] == 0, mode.stats
    assert t2.is_contiguous() and torch.equal(t2, x.t().contiguous())
    assert t3.is_contiguous() and torch.equal(t3, xb.transpose(1, 2).contiguous())
    assert kept.stride() == x.t().stride() and torch.equal(kept, x.t())


@pytest.mark.parametrize("dtype_name", ["float32", "bfloat16", "float16"])
def test_mode_queue_matches_the_oracle(dtype_name):
    """Every op the mode queued, replayed by the oracle on the same initial
    storages, gives the device's final storages element by element (bit for
    bit for the exact-class ops, within the tolerance for exp)."""
    _need_gpu()
    import torch

    import oracle
    from torch_record import RecordingMode, final_storages, snapshot, to_workload

    say(f"torch mode against the oracle {dtype_name}")
    dtype = getattr(torch, dtype_name)
    g = torch.Generator(device="cpu").manual_seed(64)
    R, Cn = 45, 260
    x = torch.randn(R, Cn, generator=g).to(dtype).cuda()
    b = torch.randn(Cn, generator=g).to(dtype).cuda()
    s = torch.randn(R, generator=g).to(dtype).cuda()
    w = (torch.rand(R, Cn, generator=g) + 0.5).to(dtype).cuda()
    init = snapshot([x, b, s, w])
    mode = RecordingMode(0)
    try:
        with mode:
            y = x * b                 # broadcast along rows
            y = y + x
            y.relu_()
            z = y.t() * s             # transposed input, broadcast; keeps the layout
            z = z * 0.5
            c = z.clone()             # a dense transposed clone
            c.add_(z)
            d = x - w                 # programs defined at run time
            d = d / w
            d = -d
            e = (d * 0.05).exp()
            f = x.t().contiguous()    # transposed COPY
            h = f * 2.0 + 1.25
    finally:
        mode.close()
    assert mode.stats["passed_through"] == 0, mode.stats
    wl = to_workload(mode.record, init)
    say(f"  {len(wl.ops)} queued ops over {len(wl.buffers)} storages")
    assert len(wl.ops) == mode.stats["queued"]
    got = final_storages(wl)
    want, scales = oracle.run(wl, scales=True)
    for name in wl.buffers:
        r = oracle.compare(got[name], want[name], wl.dtypes[name], scales.get(name))
        assert r.ok, f"{name}: {r}"
    # the outputs have PyTorch's layouts
    assert z.stride() == (y.t() * s).stride() and c.stride() == z.stride()


def test_mode_outputs_keep_eager_layouts():
    """Out-of-place results have the strides eager PyTorch gives them, so a
    view taken of them afterwards works the same inside the mode."""
    _need_gpu()
    import torch

    from persistent_fusion_amd.torch_mode import GpuosMode

    say("torch mode output layouts")
    g = torch.Generator(device="cpu").manual_seed(65)
    x = torch.randn(33, 70, generator=g).cuda()
    m = torch.randn(70, 33, generator=g).cuda()
    v = torch.randn(33, generator=g).cuda()
    cube = torch.randn(4, 6, 9, generator=g).cuda()

    def prog():
        a = torch.relu(x.t())          # (70, 33) with strides (1, 70)
        flat = a.t().reshape(-1)       # a view only because a kept its layout
        b = x.t() + m                  # mixed layouts
        c = m * v                      # broadcast, contiguous
        d = x.t() * v                  # broadcast, transposed
        e = cube.permute(2, 0, 1).exp()
        return a, flat, b, c, d, e

    want = prog()
    mode = GpuosMode(0)
    try:
        with mode:
            got = prog()
    finally:
        mode.close()
    assert mode.stats["passed_through"] == 0, mode.stats
    for k, (gt, wt) in enumerate(zip(got, want)):
        assert gt.stride() == wt.stride(), (k, gt.stride(), wt.stride())
        if k == 5:
            assert torch.allclose(gt, wt, rtol=1e-5, atol=0), k
        else:
            assert torch.equal(gt, wt), k
