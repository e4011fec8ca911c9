"""GPU: degenerate and boundary cases of the queue, each against the oracle.

* an op with more dependencies than a descriptor carries (it waits for the
  in-order retire cursor instead);
* a latency-critical op reading a best-effort op's output (a hazard across
  the two rings, honoured by the host before publishing);
* empty submissions and syncs with nothing pending;
* a strictly dependent chain of 3,000 ops (every op reads the previous
  op's output), so every descriptor waits on its predecessor;
* a GATHER index out of range, which the kernel's own bound check turns
  into the device error word (no out-of-range access is made).
"""

import numpy as np
import pytest

import oracle
from persistent_fusion_amd import gpuos, runner
from persistent_fusion_amd.workloads import Op, Ref, Workload

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


def test_write_after_many_readers():
    """20 ops read x; then one op overwrites x: it depends on all 20 readers
    (more than a descriptor's 14 dependency slots)."""
    _need_gpu()
    say("edge: write after 20 readers")
    rng = np.random.default_rng(100)
    n = 50_000
    bufs = {"x": rng.uniform(-1, 1, n).astype(np.float32), "z": rng.uniform(-1, 1, n).astype(np.float32)}
    ops = []
    for k in range(20):
        bufs[f"r{k}"] = np.zeros(n, np.float32)
        ops.append(Op("scale", Ref(f"r{k}"), (Ref("x"),), n=n, alpha=0.5 + k))
    ops.append(Op("mul", Ref("x"), (Ref("z"), Ref("z")), n=n))
    ops.append(Op("add", Ref("z"), (Ref("x"), Ref("r19")), n=n))
    wl = Workload("many-readers", bufs, {k: "f32" for k in bufs}, ops,
                  outputs=["x", "z"] + [f"r{k}" for k in range(20)])
    for fusion in (1, 2):
        got = runner.run_resident(wl, fusion=fusion)
        check(wl, got)


def test_latency_critical_op_reads_a_best_effort_output():
    _need_gpu()
    say("edge: cross-ring hazard")
    rng = np.random.default_rng(101)
    n = 1 << 20
    bufs = {k: rng.uniform(-1, 1, n).astype(np.float32) for k in ("a", "b")}
    for k in ("t", "u", "v"):
        bufs[k] = np.zeros(n, np.float32)
    ops = [
        Op("mul", Ref("t"), (Ref("a"), Ref("b")), n=n),             # best effort
        Op("relu", Ref("u"), (Ref("t"),), n=n, lc=True),            # latency critical, reads t
        Op("add", Ref("v"), (Ref("u"), Ref("a")), n=n),             # best effort, reads u
    ]
    wl = Workload("cross-ring", bufs, {k: "f32" for k in bufs}, ops, outputs=["t", "u", "v"])
    got = runner.run_resident(wl, priority=1)
    check(wl, got)


def test_empty_submissions_and_syncs():
    _need_gpu()
    say("edge: empty submissions")
    import torch

    x = torch.rand(4096, device="cuda")
    y = torch.empty_like(x)
    ctx = gpuos.Context(0)
    try:
        ctx.sync(0, 5.0)                       # nothing submitted yet
        assert ctx.submit((gpuos.GpuosOp * 1)(), 0) == []
        ctx.flush()
        ctx.sync(0, 5.0)
        ids = ctx.submit(gpuos.make_op("relu", y.data_ptr(), [x.data_ptr()], n=4096))
        ctx.sync(0, 5.0)
        ctx.sync(ids[0], 5.0)                  # already complete
        ctx.flush()                            # nothing staged
        assert ctx.query(ids[0]) == 1
    finally:
        ctx.destroy()
    assert torch.equal(y, torch.relu(x))


def test_dependent_chain_of_3000_ops():
    _need_gpu()
    say("edge: 3,000-op dependent chain")
    rng = np.random.default_rng(102)
    n = 4096
    bufs = {"s": rng.uniform(-1, 1, n).astype(np.float32), "w": rng.uniform(0.5, 1.5, n).astype(np.float32),
            "p": np.zeros(n, np.float32), "q": np.zeros(n, np.float32)}
    ops = []
    kinds = ("mul", "add", "relu", "scale")
    src = Ref("s")
    for i in range(3000):
        dst = Ref("p" if i % 2 == 0 else "q")
        k = kinds[i % 4]
        if k in ("mul", "add"):
            ops.append(Op(k, dst, (src, Ref("w")), n=n))
        elif k == "scale":
            ops.append(Op(k, dst, (src,), n=n, alpha=0.75))
        else:
            ops.append(Op(k, dst, (src,), n=n))
        src = dst
    wl = Workload("chain", bufs, {k: "f32" for k in bufs}, ops, outputs=["p", "q"])
    for fusion in (1, 2):
        got = runner.run_resident(wl, fusion=fusion)
        check(wl, got)


def test_gather_index_out_of_range_poisons_the_context():
    """The kernel checks every GATHER index against src_len before reading:
    an index out of range sets the device error word (no access is made),
    the context reports EDEVICE and refuses work, the kernel still stops
    normally, and a new context on the same GPU runs correctly."""
    _need_gpu()
    import torch

    say("edge: gather index out of range")
    x = torch.arange(100, dtype=torch.float32, device="cuda")
    idx = torch.tensor([0, 5, 100, 7], dtype=torch.int32, device="cuda")  # 100 is past src_len
    y = torch.full((4,), -1.0, device="cuda")
    op = gpuos.make_op("gather", y.data_ptr(), [x.data_ptr()], idx.data_ptr(), n=4, src_len=(100, 0))
    ctx = gpuos.Context(0)
    with pytest.raises(gpuos.GpuosError) as e:
        ctx.submit(op)
        ctx.sync(0, 10.0)
    assert e.value.status == gpuos.EDEVICE
    assert ctx.stats()["device_error"] == 2  # the gather-range code
    with pytest.raises(gpuos.GpuosError):
        ctx.submit(op)
    with pytest.raises(gpuos.GpuosError) as e:
        ctx.destroy()
    assert e.value.status == gpuos.EDEVICE
    assert y.cpu().tolist() == [0.0, 5.0, -1.0, 7.0]  # in-range elements gathered, the bad one untouched
    rng = np.random.default_rng(103)
    bufs = {"a": rng.uniform(-1, 1, 5000).astype(np.float32), "b": np.zeros(5000, np.float32)}
    wl = Workload("after-error", bufs, {"a": "f32", "b": "f32"}, [Op("relu", Ref("b"), (Ref("a"),), n=5000)],
                  outputs=["b"])
    check(wl, runner.run_resident(wl))
