"""GPU: ops defined at run time (register programs interpreted by the resident
kernel) against the oracle.  Programs without EXP are bit-exact; with EXP the
tolerance class applies.  Also: a program updated while ops that use it are
queued, in-place programs, misaligned operands, and the fused chain computed
by one program at full size."""

import numpy as np
import pytest

import oracle
from persistent_fusion_amd import gpuos, runner, workloads
from persistent_fusion_amd.workloads import Op, Program, Ref, Workload
from program_cases import CHAINS, SINGLE, program_workload

pytestmark = pytest.mark.gpu


def _need_gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gpuos.lib()


def say(msg):
    print(msg, flush=True)


def check(wl, got, outputs=None):
    want, scales = oracle.run(wl, scales=True)
    for name in outputs or wl.outputs:
        r = oracle.compare(got[name], want[name], wl.dtypes[name], scales.get(name))
        assert r.ok, f"{wl.name}/{name}: {r}"


@pytest.mark.parametrize("fusion", [1, 2])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("n", [1, 5, 64 * 8 + 3, 20_011])
def test_every_instruction_and_chain(dtype, n, fusion):
    """fusion 2: every program interpreted; fusion 1: fp32 chains lowered to
    built-in descriptors (the rest interpreted)."""
    _need_gpu()
    say(f"programs dtype={dtype} n={n} fusion={fusion}")
    progs = [Program((ins,), len(ins) - 2, 3) for ins in SINGLE] + CHAINS
    wl = program_workload(progs, n, dtype, seed=80 + n)
    got = runner.run_resident(wl, fusion=fusion)
    check(wl, got)


@pytest.mark.parametrize("misalign,in_place", [(True, False), (False, True), (True, True)])
def test_misaligned_and_in_place(misalign, in_place):
    _need_gpu()
    say(f"programs misalign={misalign} in_place={in_place}")
    wl = program_workload(CHAINS, 100_003, "f32", seed=90, misalign=misalign, in_place=in_place)
    for fusion in (1, 2):
        got = runner.run_resident(wl, fusion=fusion)
        check(wl, got)


def test_update_while_queued():
    """Ops keep the body they were submitted with: a program redefined
    between two submissions gives the old result to the first ops and the
    new one to the later ops, with one flush for all of them."""
    _need_gpu()
    import torch

    say("program update while queued")
    rng = np.random.default_rng(91)
    n, per = 4096, 100
    v1 = Program((("mul", 3, 0, 1), ("add", 3, 3, 8)), 2, 3, consts=(0.5,))
    v2 = Program((("sub", 3, 0, 1), ("relu", 3, 3), ("mul", 3, 3, 8)), 2, 3, consts=(3.0,))
    x = rng.uniform(-1, 1, (2 * per, n)).astype(np.float32)
    w = rng.uniform(-1, 1, (2 * per, n)).astype(np.float32)
    tx, tw = torch.from_numpy(x).cuda(), torch.from_numpy(w).cuda()
    ty = torch.full((2 * per, n), float("nan"), device="cuda")
    ctx = gpuos.Context(0)
    try:
        pid = ctx.program_define(gpuos.program_of(v1))
        def ops(rows):
            arr = (gpuos.GpuosOp * len(rows))()
            for k, r in enumerate(rows):
                arr[k] = gpuos.make_op("program", ty[r].data_ptr(), [tx[r].data_ptr(), tw[r].data_ptr()],
                                       n=n, dims=(pid,))
            return arr
        ctx.submit(ops(range(per)))
        ctx.program_update(pid, gpuos.program_of(v2))
        ctx.submit(ops(range(per, 2 * per)))
        ctx.sync(0, 30.0)
    finally:
        ctx.destroy()
    got = ty.cpu().numpy()
    for rows, prog in ((range(per), v1), (range(per, 2 * per), v2)):
        bufs = {"x": x[list(rows)].reshape(-1), "w": w[list(rows)].reshape(-1),
                "y": np.zeros(len(rows) * n, np.float32)}
        wl = Workload("upd", bufs, {k: "f32" for k in bufs},
                      [Op("program", Ref("y"), (Ref("x"), Ref("w")), n=len(rows) * n, prog=prog)])
        want = oracle.run(wl)["y"]
        assert np.array_equal(got[list(rows)].reshape(-1).view(np.uint32), want.view(np.uint32))


def test_programs_in_a_queue_with_builtin_ops():
    """Program ops reading and feeding built-in ops: hazards order them."""
    _need_gpu()
    say("programs mixed with built-in ops")
    rng = np.random.default_rng(92)
    n = 30_000
    bufs = {k: rng.uniform(-2, 2, n).astype(np.float32) for k in ("a", "b", "c")}
    for k in ("t", "u", "v", "y"):
        bufs[k] = np.zeros(n, np.float32)
    sq = Program((("mul", 3, 0, 0), ("sub", 3, 3, 1)), 2, 3)        # a*a - b
    mx = Program((("max", 3, 0, 1), ("min", 3, 3, 2)), 3, 3)         # clamp(max(u, v), c)
    ops = [
        Op("relu", Ref("t"), (Ref("a"),), n=n),
        Op("program", Ref("u"), (Ref("t"), Ref("b")), n=n, prog=sq),
        Op("exp", Ref("v"), (Ref("c"),), n=n),
        Op("program", Ref("y"), (Ref("u"), Ref("v"), Ref("c")), n=n, prog=mx),
        Op("program", Ref("t"), (Ref("y"), Ref("a")), n=n, prog=sq),   # rewrites t after its readers
    ]
    wl = Workload("mixed", bufs, {k: "f32" for k in bufs}, ops, outputs=["t", "u", "v", "y"])
    got = runner.run_resident(wl)
    check(wl, got)


def test_program_chain_full_size_equals_the_fused_chain():
    """relu(a*x + b) at 16M elements as one program, interpreted (fusion
    off) and lowered to the fused micro-program (fusion on): bit-identical
    to the built-in fused chain and to the oracle."""
    _need_gpu()
    say("program chain 16M")
    wl = workloads.gen_program_chain(seed=0)
    ref = runner.run_resident(workloads.gen_fused_chain(seed=0), outputs=["y"])
    for fusion in (2, 1):
        got = runner.run_resident(wl, outputs=["y"], fusion=fusion)
        check(wl, got, ["y"])
        assert np.array_equal(got["y"].view(np.uint32), ref["y"].view(np.uint32)), fusion


def test_programs_in_the_priority_ring():
    """Latency-critical PROGRAM ops (claimed from the priority ring) between
    best-effort built-in ops: every output matches the oracle."""
    _need_gpu()
    say("programs in the priority ring")
    rng = np.random.default_rng(93)
    n = 8192
    bufs = {}
    ops = []
    clamp = Program((("max", 3, 0, 8), ("min", 3, 3, 9), ("mul", 3, 3, 1)), 2, 3, consts=(-0.5, 0.5))
    for k in range(40):
        for nm in (f"a{k}", f"b{k}"):
            bufs[nm] = rng.uniform(-1, 1, n).astype(np.float32)
        bufs[f"y{k}"] = np.zeros(n, np.float32)
        if k % 4 == 0:
            ops.append(Op("program", Ref(f"y{k}"), (Ref(f"a{k}"), Ref(f"b{k}")), n=n, prog=clamp, lc=True))
        else:
            ops.append(Op("mul", Ref(f"y{k}"), (Ref(f"a{k}"), Ref(f"b{k}")), n=n))
    wl = Workload("lc-programs", bufs, {k: "f32" for k in bufs}, ops,
                  outputs=[f"y{k}" for k in range(40)])
    got = runner.run_resident(wl, priority=1)
    check(wl, got)
