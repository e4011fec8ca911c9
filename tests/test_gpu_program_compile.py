"""GPU: program bodies compiled at run time (gpuos_program_compile).

The pages' runtime compiles operators while the persistent kernel runs and
installs them with two slots, so an operator can be replaced safely ("GPUOS:
A GPU Operating System Primitive for Transparent Operation Fusion", section
"The Paper").  Here hipRTC builds a variant of the resident kernel whose op
table holds the programs' bodies as straight-line code, and the queue is
handed between the built-in kernel and the variant where it has drained.

* Every instruction alone and the chains, in fp32, bf16 and fp16, at sizes
  from 1 element to several tiles with a ragged tail: compiled results match
  the oracle and are bit-identical to the interpreter's.
* A queue that mixes compiled programs with ops only the built-in kernel
  runs: the queue changes kernels at the drain points and every output
  matches the oracle.
* Two slots: a program recompiled with a new body while ops of the old body
  are queued; each op runs the body it was submitted with.
* Speed: a 16M-element program op runs at the built-in elementwise op's
  bandwidth (same bytes moved), and no slower than the interpreter.
"""

import time

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


PROGS = [Program((ins,), len(ins) - 2, 3) for ins in SINGLE] + CHAINS


def _run_in(ctx, wl, prog_ids):
    """Submits wl's ops on an open context (programs already defined)."""
    tensors = runner.to_device(wl, 0)
    addr = runner.addr_fn(tensors, wl)
    arr = gpuos.encode_ops(wl.ops, 0, len(wl.ops), addr, {}, prog_ids)
    ctx.submit(arr, len(wl.ops))
    ctx.flush()
    ctx.sync(0, 60.0)
    return runner.download(tensors, wl, wl.outputs)


def test_compiled_bodies_match_the_oracle_and_the_interpreter():
    _need_gpu()
    ctx = gpuos.Context(0, fusion=2)  # no lowering: every program op is a PROGRAM descriptor
    try:
        prog_ids = {p: ctx.program_define(gpuos.program_of(p)) for p in PROGS}
        t0 = time.perf_counter()
        log = ctx.program_compile()
        say(f"compiled {len(PROGS)} bodies for 3 dtypes in {time.perf_counter() - t0:.1f} s"
            + (f" (log: {log[:200]})" if log else ""))
        src = ctx.rtc_source()
        assert src.count("struct RtcBody") == len(PROGS)
        for dtype in ("f32", "bf16", "f16"):
            for n in (1, 5, 64 * 8 + 3, 20_011):
                say(f"compiled programs dtype={dtype} n={n}")
                wl = program_workload(PROGS, n, dtype, seed=180 + n)
                before = ctx.stats()["programs_compiled"]
                got = _run_in(ctx, wl, prog_ids)
                assert ctx.stats()["programs_compiled"] - before == len(PROGS)
                check(wl, got)
                interp = runner.run_resident(wl, fusion=2)
                for name in wl.outputs:
                    assert np.array_equal(got[name].view(np.uint8), interp[name].view(np.uint8)), \
                        f"{dtype} n={n} {name}: compiled and interpreted results differ"
        st = ctx.stats()
        assert st["kernel_switches"] >= 1
    finally:
        ctx.destroy()


def test_misaligned_and_in_place_compiled():
    _need_gpu()
    for misalign, in_place in ((True, False), (False, True)):
        say(f"compiled programs misalign={misalign} in_place={in_place}")
        wl = program_workload(CHAINS, 100_003, "f32", seed=190, misalign=misalign, in_place=in_place)
        st = {}
        got = runner.run_resident(wl, fusion=2, compile_programs=True, stats=st)
        assert st["programs_compiled"] == len(CHAINS)
        check(wl, got)


def test_queue_changes_kernels_at_drain_points():
    """Compiled programs between ops the variant does not run (bf16 ops,
    row softmax): the queue moves between kernels and every result holds."""
    _need_gpu()
    say("mixed queue over both kernels")
    rng = np.random.default_rng(193)
    n, rows, L = 50_000, 64, 512
    bufs = {k: rng.uniform(-2, 2, n).astype(np.float32) for k in ("a", "b", "c")}
    for k in ("t", "u", "v", "y"):
        bufs[k] = np.zeros(n, np.float32)
    bufs["hb"] = oracle.f32_to_bf16(rng.uniform(-1, 1, n).astype(np.float32))
    bufs["hy"] = np.zeros(n, np.uint16)
    bufs["s"] = rng.uniform(-3, 3, rows * L).astype(np.float32)
    bufs["sm"] = np.zeros(rows * L, np.float32)
    dts = {k: "f32" for k in bufs}
    dts["hb"] = dts["hy"] = "bf16"
    clamp = Program((("max", 3, 0, 8), ("min", 3, 3, 9), ("mul", 3, 3, 1)), 2, 3, consts=(-0.5, 0.5))
    sq = Program((("mul", 3, 0, 0), ("sub", 3, 3, 1), ("div", 3, 3, 8)), 2, 3, consts=(3.0,))
    ops = [
        Op("program", Ref("t"), (Ref("a"), Ref("b")), n=n, prog=clamp),
        Op("add", Ref("u"), (Ref("t"), Ref("c")), n=n),                      # runs in either kernel
        Op("program", Ref("v"), (Ref("u"), Ref("a")), n=n, prog=sq),
        Op("relu", Ref("hy"), (Ref("hb"),), n=n, dtype="bf16"),              # built-in kernel only
        Op("program", Ref("y"), (Ref("v"), Ref("t")), n=n, prog=clamp),
        Op("row_softmax", Ref("sm"), (Ref("s"),), n=rows * L, rows=rows, row_len=L),  # built-in only
        Op("program", Ref("t"), (Ref("y"), Ref("c")), n=n, prog=sq),         # rewrites t after its readers
    ]
    wl = Workload("mixed_kernels", bufs, dts, ops, outputs=["t", "u", "v", "y", "hy", "sm"])
    wl.groups = [(0, 3), (3, 5), (5, 7)]
    st = {}
    got = runner.run_resident(wl, fusion=2, compile_programs=True, stats=st)
    say(f"  kernel switches {st['kernel_switches']}, launches {st['launches']}")
    # flush 1: to the variant before the first program; flush 2: back to the
    # built-in kernel for the bf16 relu, then to the variant for the program;
    # flush 3: the same around the softmax
    assert st["kernel_switches"] == 5
    assert st["programs_compiled"] == 4
    check(wl, got)


def test_recompile_while_queued_keeps_each_ops_body():
    """Two slots: ops of body v1 are queued on the compiled variant, the
    program is updated to v2 and compiled again, and ops of v2 follow in the
    same flush sequence; each op computes the body it was submitted with."""
    _need_gpu()
    import torch

    say("recompile while queued")
    rng = np.random.default_rng(194)
    n, per = 1 << 16, 40
    v1 = Program((("max", 3, 0, 8), ("mul", 3, 3, 1)), 2, 3, consts=(0.25,))
    v2 = Program((("sub", 3, 0, 1), ("abs", 3, 3), ("min", 3, 3, 8)), 2, 3, consts=(0.75,))
    x = rng.uniform(-1, 1, (2 * per, n)).astype(np.float32)
    w = rng.uniform(-1, 1, (2 * per, n)).astype(np.float32)
    tx, tw = torch.from_numpy(x).cuda(), torch.from_numpy(w).cuda()
    ty = torch.full((2 * per, n), float("nan"), device="cuda")
    ctx = gpuos.Context(0, fusion=2)
    try:
        pid = ctx.program_define(gpuos.program_of(v1))
        ctx.program_compile()

        def ops(rows):
            arr = (gpuos.GpuosOp * len(rows))()
            for k, r in enumerate(rows):
                arr[k] = gpuos.make_op("program", ty[r].data_ptr(), [tx[r].data_ptr(), tw[r].data_ptr()],
                                       n=n, dims=(pid,))
            return arr

        ctx.submit(ops(range(per)))
        ctx.flush()                      # v1 ops queued on the first variant
        ctx.program_update(pid, gpuos.program_of(v2))
        ctx.program_compile()            # second slot, while v1 ops may still run
        ctx.submit(ops(range(per, 2 * per)))
        ctx.flush()                      # hand-over to the second variant after the drain
        ctx.sync(0, 60.0)
        st = ctx.stats()
    finally:
        ctx.destroy()
    assert st["programs_compiled"] == 2 * per
    assert st["kernel_switches"] == 2
    got = ty.cpu().numpy()
    for rows, prog in ((range(per), v1), (range(per, 2 * per), v2)):
        bufs = {"x": x[list(rows)].reshape(-1), "w": w[list(rows)].reshape(-1),
                "y": np.zeros(len(rows) * n, np.float32)}
        wl = Workload("recompile", bufs, {k: "f32" for k in bufs},
                      [Op("program", Ref("y"), (Ref("x"), Ref("w")), n=len(rows) * n, prog=prog)])
        want = oracle.run(wl)["y"]
        assert np.array_equal(got[list(rows)].reshape(-1).view(np.uint32), want.view(np.uint32))


def _time_queue(ctx, arr, n_ops, reps=5):
    best = float("inf")
    for _ in range(reps):
        t0 = time.perf_counter()
        ctx.submit(arr, n_ops)
        ctx.flush()
        ctx.sync(0, 60.0)
        best = min(best, time.perf_counter() - t0)
    return best


CLAMP_SCALE = Program((("max", 3, 0, 8), ("min", 3, 3, 9), ("mul", 3, 3, 1)), 2, 3, consts=(-0.5, 0.5))
CLAMP_SCALE_DIV = Program((("max", 3, 0, 8), ("min", 3, 3, 9), ("mul", 3, 3, 1), ("div", 3, 3, 10)), 2, 3,
                          consts=(-0.5, 0.5, 3.0))


@pytest.mark.parametrize("prog,floor", [(CLAMP_SCALE, 0.9), (CLAMP_SCALE_DIV, 0.0)],
                         ids=["clamp_scale", "clamp_scale_div"])
def test_compiled_program_runs_at_builtin_speed(prog, floor):
    """A 2-input program (clamp then scale) over 16M fp32 elements moves the
    bytes of a built-in MUL; compiled, it runs at the MUL's bandwidth.  With a
    correctly rounded division appended (about 15 vector instructions per
    element) the rate is reported and checked against the interpreter only."""
    _need_gpu()
    import torch

    say(f"compiled program speed, 16M elements, {len(prog.insns)} instructions")
    n, k = 1 << 24, 12
    g = torch.Generator(device="cuda").manual_seed(5)
    xs = [torch.rand(n, device="cuda", generator=g) * 2 - 1 for _ in range(4)]
    ws = [torch.rand(n, device="cuda", generator=g) * 2 - 1 for _ in range(4)]
    ys = [torch.empty(n, device="cuda") for _ in range(4)]
    gbs = {}
    for mode in ("builtin_mul", "interpreted", "compiled"):
        ctx = gpuos.Context(0, fusion=2)
        try:
            pid = ctx.program_define(gpuos.program_of(prog))
            if mode == "compiled":
                ctx.program_compile()
            arr = (gpuos.GpuosOp * k)()
            for i in range(k):
                j = i % 4
                if mode == "builtin_mul":
                    arr[i] = gpuos.make_op("mul", ys[j].data_ptr(), [xs[j].data_ptr(), ws[j].data_ptr()], n=n)
                else:
                    arr[i] = gpuos.make_op("program", ys[j].data_ptr(), [xs[j].data_ptr(), ws[j].data_ptr()],
                                           n=n, dims=(pid,))
            _time_queue(ctx, arr, k, reps=2)  # warm (and the hand-over to the variant)
            t = _time_queue(ctx, arr, k)
            gbs[mode] = k * 3 * 4 * n / t / 1e9
        finally:
            ctx.destroy()
    say(f"  GB/s: {gbs}")
    assert gbs["compiled"] >= floor * gbs["builtin_mul"], gbs
    assert gbs["compiled"] >= gbs["interpreted"] * 0.98, gbs
    # the last queue's result (compiled) against the oracle on a sample
    idx = np.random.default_rng(6).choice(n, 4096, replace=False)
    j = (k - 1) % 4
    bufs = {"x": xs[j].cpu().numpy()[idx], "w": ws[j].cpu().numpy()[idx], "y": np.zeros(idx.size, np.float32)}
    wl = Workload("speed_sample", bufs, {q: "f32" for q in bufs},
                  [Op("program", Ref("y"), (Ref("x"), Ref("w")), n=idx.size, prog=prog)])
    want = oracle.run(wl)["y"]
    assert np.array_equal(ys[j].cpu().numpy()[idx].view(np.uint32), want.view(np.uint32))
