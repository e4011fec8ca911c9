"""GPU parity: the resident kernel (and the per-op comparator) against the oracle.

Every test runs seeded workloads through libgpuos.so on cuda:0 and compares
the outputs with the CPU oracle element by element: bit-exact for COPY,
GATHER, ADD, MUL, SCALE, RELU and ROPE, within 1e-5 (fp32) / 1e-2 (bf16)
relative to the oracle's error scale for reductions and transcendentals.
"""

import math

import numpy as np
import pytest

import oracle
from persistent_fusion_amd import gpuos, runner, workloads
from persistent_fusion_amd.workloads import Op, Ref, Workload

pytestmark = pytest.mark.gpu


def _need_gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gpuos.lib()  # fails loudly when the native library is missing


def say(msg):
    print(msg, flush=True)


def check(wl, got, outputs=None, upto=None):
    want, scales = oracle.run(wl, upto=upto, scales=True)
    for name in outputs or wl.outputs:
        r = oracle.compare(got[name], want[name], wl.dtypes[name], scales.get(name))
        assert r.ok, f"{wl.name}/{name}: {r}"


# ----------------------------------------------------------------------------
# the fused chain y = relu(a*x + b)


@pytest.mark.parametrize("n", [1, 63, 1000, 4097, 1_000_003])
@pytest.mark.parametrize("fusion", [1, 2])
def test_fused_chain_resident(n, fusion):
    _need_gpu()
    say(f"fused chain n={n} fusion={fusion}")
    wl = workloads.gen_fused_chain(seed=1, n=n)
    got = runner.run_resident(wl, outputs=["y"], fusion=fusion)
    check(wl, got, ["y"])


@pytest.mark.parametrize("fuse", [False, True])
def test_fused_chain_per_op_launches(fuse):
    _need_gpu()
    say(f"fused chain per-op fuse={fuse}")
    wl = workloads.gen_fused_chain(seed=2, n=1_000_003)
    got = runner.run_per_op(wl, outputs=["y"], fuse=fuse)
    check(wl, got, ["y"])


def test_fused_chain_full_size():
    _need_gpu()
    say("fused chain n=16777216")
    wl = workloads.gen_fused_chain(seed=0)
    got = runner.run_resident(wl, outputs=["y"])
    check(wl, got, ["y"])


# ----------------------------------------------------------------------------
# queue of 1,000 elementwise ops on 4,096-element vectors


@pytest.mark.parametrize("fusion", [1, 2])
def test_elementwise_queue_full(fusion):
    _need_gpu()
    say(f"elementwise queue 1000x4096 fusion={fusion}")
    wl = workloads.gen_elementwise_queue(seed=0)
    got = runner.run_resident(wl, fusion=fusion)
    check(wl, got)


@pytest.mark.parametrize("auto_deps", [1, 2])
def test_elementwise_queue_explicit_or_auto_deps(auto_deps):
    _need_gpu()
    say(f"elementwise queue auto_deps={auto_deps}")
    wl = workloads.gen_elementwise_queue(seed=3, n_ops=600, n=4097)
    got = runner.run_resident(wl, auto_deps=auto_deps)
    check(wl, got)


def test_elementwise_queue_per_op():
    _need_gpu()
    say("elementwise queue per-op")
    wl = workloads.gen_elementwise_queue(seed=0)
    got = runner.run_per_op(wl)
    check(wl, got)


def test_elementwise_queue_small_ring_wraps():
    _need_gpu()
    say("elementwise queue ring_slots=64")
    wl = workloads.gen_elementwise_queue(seed=4, n_ops=1000, n=1024)
    got = runner.run_resident(wl, ring_slots=64)
    check(wl, got)


# ----------------------------------------------------------------------------
# fp16, int32 and strided / broadcast views


def _f16(rng, n, scale=1.0):
    return (rng.standard_normal(n) * scale).astype(np.float32).astype(np.float16)


@pytest.mark.parametrize("kind", ["copy", "add", "mul", "scale", "relu", "exp", "silu_mul"])
def test_f16_elementwise(kind):
    _need_gpu()
    rng = np.random.default_rng(50)
    for n, src in ((1, (0, 0)), (63, (0, 0)), (1000, (0, 0)), (4097, (0, 0)), (100_003, (0, 0)),
                   (999, (37, 0))):
        say(f"f16 {kind} n={n} src_len={src}")
        a, b = _f16(rng, n), _f16(rng, n)
        a[:5] = np.array([0.0, -0.0, 6e-8, -65504.0, np.inf], np.float16)[: min(5, n)]
        bufs = {"a": a, "b": b, "y": np.zeros(n, np.float16)}
        ins = (Ref("a"), Ref("b")) if kind in ("add", "mul", "silu_mul") else (Ref("a"),)
        wl = Workload("f16", bufs, {"a": "f16", "b": "f16", "y": "f16"},
                      [Op(kind, Ref("y"), ins, n=n, dtype="f16", alpha=0.75, src_len=src)],
                      outputs=["y"])
        check(wl, runner.run_resident(wl))


@pytest.mark.parametrize("kind", ["row_sum", "row_softmax", "rmsnorm", "rope"])
def test_f16_rows_and_rope(kind):
    _need_gpu()
    rng = np.random.default_rng(51)
    for rows, L in ((3, 64), (5, 1000), (2, 4096), (7, 33)):
        if kind == "rope" and L % 2:
            continue
        say(f"f16 {kind} rows={rows} L={L}")
        n = rows * L
        bufs = {"x": _f16(rng, n), "g": _f16(rng, L, 0.5), "tab": workloads.rope_table([11], L).reshape(-1),
                "y": np.zeros(rows if kind == "row_sum" else n, np.float16)}
        dts = {"x": "f16", "g": "f16", "tab": "f32", "y": "f16"}
        aux = Ref("g") if kind == "rmsnorm" else Ref("tab") if kind == "rope" else None
        op = Op(kind, Ref("y"), (Ref("x"),), aux, n=n, dtype="f16", rows=rows, row_len=L,
                eps=float(np.float32(1e-6)), dims=(rows, L) if kind == "rope" else ())
        wl = Workload("f16rows", bufs, dts, [op], outputs=["y"])
        check(wl, runner.run_resident(wl))


@pytest.mark.parametrize("kind", ["add", "mul", "relu", "copy"])
def test_i32_elementwise_wraps(kind):
    _need_gpu()
    rng = np.random.default_rng(52)
    for n in (1, 7, 4096, 65_537):
        say(f"i32 {kind} n={n}")
        a = rng.integers(-2 ** 31, 2 ** 31, n).astype(np.int32)
        b = rng.integers(-2 ** 31, 2 ** 31, n).astype(np.int32)
        a[:4] = np.array([2 ** 31 - 1, -2 ** 31, -1, 0], np.int32)[: min(4, n)]
        bufs = {"a": a, "b": b, "y": np.zeros(n, np.int32)}
        ins = (Ref("a"), Ref("b")) if kind in ("add", "mul") else (Ref("a"),)
        wl = Workload("i32", bufs, {"a": "i32", "b": "i32", "y": "i32"},
                      [Op(kind, Ref("y"), ins, n=n, dtype="i32")], outputs=["y"])
        check(wl, runner.run_resident(wl))


_VIEW_CASES = {
    # name: (shape, out strides, in0 strides, in1 strides, in0 len, in1 len, out len)
    "bias_add": ((37, 300), (300, 1), (300, 1), (0, 1), 37 * 300, 300, 37 * 300),
    "row_scale": ((41, 129), (129, 1), (129, 1), (1, 0), 41 * 129, 41, 41 * 129),
    "transpose": ((33, 70), (1, 33), (70, 1), (0, 0), 33 * 70, 0, 33 * 70),
    # COPY of these two takes the transposed-block path: ragged row and column
    # blocks, a padded even output row stride (16-bit pairs stored as words, the
    # odd last column alone), input columns 16-byte aligned
    "transpose_read": ((328, 257), (260, 1), (1, 328), (0, 0), 328 * 257, 0, 328 * 260),
    # batched: x.transpose(1, 2) of a contiguous [3, 136, 72] input, copied out
    "transpose_read_batched": ((3, 72, 136), (72 * 136, 136, 1), (72 * 136, 1, 72), (0, 0, 0),
                               3 * 72 * 136, 0, 3 * 72 * 136),
    # batched with ragged batch strides (one element past the batch's size, in
    # and out): the first batch's input columns are 16-byte aligned and the
    # others' are not, and the output's 16-bit pairs shift between batches, so
    # the batches of one descriptor take different paths
    "transpose_read_batched_ragged": ((3, 72, 136), (72 * 136 + 1, 136, 1), (72 * 136 + 1, 1, 72),
                                      (0, 0, 0), 2 * (72 * 136 + 1) + 72 * 136, 0,
                                      2 * (72 * 136 + 1) + 72 * 136),
    # odd strides: misaligned input columns and output pairs, element by element
    "transpose_read_odd": ((70, 33), (33, 1), (1, 70), (0, 0), 70 * 33, 0, 70 * 33),
    "outer": ((50, 64), (64, 1), (1, 0), (0, 1), 50, 64, 50 * 64),
    "strided_out": ((8, 100), (400, 2), (100, 1), (100, 1), 800, 800, 3200),
    "scalar": ((5000,), (1,), (1,), (0,), 5000, 1, 5000),
    "4d": ((3, 4, 5, 6), (120, 30, 6, 1), (1, 3, 12, 60), (0, 6, 0, 1), 360, 30, 360),
    "long_rows": ((3, 5000), (5000, 1), (5000, 1), (0, 1), 15000, 5000, 15000),
}


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16", "i32"])
@pytest.mark.parametrize("case", sorted(_VIEW_CASES))
def test_views(case, dtype):
    _need_gpu()
    shape, so, s0, s1, la, lb, lo = _VIEW_CASES[case]
    rng = np.random.default_rng(53)
    n = int(np.prod(shape))
    kinds = ["add", "mul", "relu", "copy"] if dtype == "i32" else ["add", "mul", "scale", "relu",
                                                                     "exp", "silu_mul", "copy"]
    for kind in kinds:
        binary = kind in ("add", "mul", "silu_mul")
        if binary and lb == 0:
            continue
        say(f"view {case} {dtype} {kind}")

        def draw(m):
            if dtype == "i32":
                return rng.integers(-2 ** 31, 2 ** 31, m).astype(np.int32)
            v = rng.standard_normal(m).astype(np.float32)
            return {"f32": v, "bf16": workloads.f32_to_bf16_trunc(v), "f16": v.astype(np.float16)}[dtype]

        npdt = workloads.NP_DTYPE[dtype]
        bufs = {"a": draw(la), "b": draw(max(lb, 1)), "y": np.zeros(lo, npdt)}
        ins = (Ref("a"), Ref("b")) if binary else (Ref("a"),)
        wl = Workload("view", bufs, {"a": dtype, "b": dtype, "y": dtype},
                      [Op(kind, Ref("y"), ins, n=n, dtype=dtype, alpha=-1.25,
                          view=(shape, so, s0, s1))], outputs=["y"])
        check(wl, runner.run_resident(wl))


def test_view_in_place_and_queue_with_hazards():
    """A queue mixing viewed and plain ops over shared buffers: the hazards
    derived from view ranges order it as submitted."""
    _need_gpu()
    say("views in a queue")
    rng = np.random.default_rng(54)
    R, Cn = 64, 96
    bufs = {"x": rng.standard_normal(R * Cn).astype(np.float32),
            "b": rng.standard_normal(Cn).astype(np.float32),
            "s": rng.standard_normal(R).astype(np.float32),
            "t": np.zeros(R * Cn, np.float32), "u": np.zeros(R * Cn, np.float32)}
    ops = [Op("add", Ref("t"), (Ref("x"), Ref("b")), n=R * Cn, view=((R, Cn), (Cn, 1), (Cn, 1), (0, 1))),
           Op("relu", Ref("t"), (Ref("t"),), n=R * Cn, view=((R, Cn), (Cn, 1), (Cn, 1), (0, 0))),
           Op("copy", Ref("b"), (Ref("x", 5),), n=Cn),  # overwrites the broadcast row afterwards
           Op("mul", Ref("u"), (Ref("t"), Ref("s")), n=R * Cn, view=((Cn, R), (1, Cn), (1, Cn), (0, 1))),
           Op("add", Ref("x"), (Ref("x"), Ref("u")), n=R * Cn)]
    wl = Workload("viewq", bufs, {k: "f32" for k in bufs}, ops, outputs=["x", "b", "t", "u"])
    check(wl, runner.run_resident(wl))


# ----------------------------------------------------------------------------
# every opcode on ragged sizes


def _ew_workload(kind, dtype, n, seed, src_len=(0, 0)):
    rng = np.random.default_rng(seed)
    conv = (lambda a: workloads.f32_to_bf16_trunc(a)) if dtype == "bf16" else (lambda a: a)
    npdt = np.uint16 if dtype == "bf16" else np.float32
    la = src_len[0] or n
    lb = src_len[1] or n
    bufs = {"a": conv((rng.standard_normal(la) * 3).astype(np.float32)),
            "b": conv((rng.standard_normal(lb) * 3).astype(np.float32)),
            "y": np.zeros(n, npdt)}
    dts = {k: dtype for k in bufs}
    ar = 2 if kind in ("add", "mul", "silu_mul") else 1
    ins = (Ref("a"), Ref("b"))[:ar]
    op = Op(kind, Ref("y"), ins, n=n, dtype=dtype, alpha=-0.6875, src_len=src_len[:2])
    return Workload(f"{kind}-{dtype}-{n}", bufs, dts, [op], outputs=["y"])


@pytest.mark.parametrize("kind", ["add", "mul", "scale", "relu", "exp", "copy", "silu_mul"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_elementwise_ops_ragged(kind, dtype):
    _need_gpu()
    for n in (1, 63, 64, 65, 4095, 4096, 4097, (1 << 20) + 3):
        say(f"{kind} {dtype} n={n}")
        wl = _ew_workload(kind, dtype, n, seed=n)
        got = runner.run_resident(wl)
        check(wl, got)


@pytest.mark.parametrize("kind", ["add", "mul", "scale", "relu", "exp", "copy", "silu_mul"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_elementwise_ops_streamed(kind, dtype):
    """The non-temporal (streamed) variants of the elementwise bodies."""
    _need_gpu()
    for n in (1, 4097, (1 << 20) + 3):
        say(f"streamed {kind} {dtype} n={n}")
        wl = _ew_workload(kind, dtype, n, seed=n + 1)
        got = runner.run_resident(wl, stream_min_kib=1)
        check(wl, got)


@pytest.mark.parametrize("n", [63, 1_000_003])
def test_fused_chain_streamed(n):
    _need_gpu()
    say(f"streamed fused chain n={n}")
    wl = workloads.gen_fused_chain(seed=3, n=n)
    got = runner.run_resident(wl, outputs=["y"], stream_min_kib=1)
    check(wl, got, ["y"])


@pytest.mark.parametrize("kind", ["add", "relu", "copy"])
def test_cyclic_sources(kind):
    _need_gpu()
    say(f"cyclic {kind}")
    wl = _ew_workload(kind, "f32", 10_000, seed=5, src_len=(777, 4096))
    got = runner.run_resident(wl)
    check(wl, got)
    got = runner.run_per_op(wl)
    check(wl, got)


def test_special_values_bit_exact():
    _need_gpu()
    say("special values")
    vals = np.array([0.0, -0.0, np.nan, np.inf, -np.inf, 1e-45, -1e-45, 2.0 ** -140, 3.4e38,
                     -3.4e38, 1.0, -1.0], np.float32)
    n = vals.size * 100
    a = np.tile(vals, 100)
    b = np.roll(a, 7)
    bufs = {"a": a, "b": b}
    ops = []
    for i, kind in enumerate(("add", "mul", "relu", "scale")):
        bufs[f"y{i}"] = np.zeros(n, np.float32)
        ins = (Ref("a"), Ref("b")) if kind in ("add", "mul") else (Ref("a"),)
        ops.append(Op(kind, Ref(f"y{i}"), ins, n=n, alpha=3.0))
    wl = Workload("special", bufs, {k: "f32" for k in bufs}, ops, outputs=[f"y{i}" for i in range(4)])
    got = runner.run_resident(wl)
    check(wl, got)


@pytest.mark.parametrize("kind", ["row_sum", "row_softmax", "rmsnorm"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_row_ops(kind, dtype):
    _need_gpu()
    rng = np.random.default_rng(7)
    conv = (lambda a: workloads.f32_to_bf16_trunc(a)) if dtype == "bf16" else (lambda a: a)
    npdt = np.uint16 if dtype == "bf16" else np.float32
    for rows, L in ((1, 1), (3, 63), (14, 512), (5, 896), (2, 4096), (300, 129), (1, 4095)):
        say(f"{kind} {dtype} rows={rows} L={L}")
        n = rows * L
        bufs = {"x": conv((rng.standard_normal(n) * 2).astype(np.float32)),
                "g": conv(rng.standard_normal(L).astype(np.float32)),
                "y": np.zeros(rows if kind == "row_sum" else n, npdt)}
        op = Op(kind, Ref("y"), (Ref("x"),), Ref("g") if kind == "rmsnorm" else None, n=n,
                dtype=dtype, rows=rows, row_len=L, eps=float(np.float32(1e-6)))
        wl = Workload(kind, bufs, {k: dtype for k in bufs}, [op], outputs=["y"])
        check(wl, runner.run_resident(wl))


@pytest.mark.parametrize("L", [63, 64, 512, 4096])
def test_softmax_special_rows(L):
    """NaN, +inf, all -inf, a single -inf and a constant row, on the
    per-element path (63), the in-register path (64, 512) and the long-row
    path (4096)."""
    _need_gpu()
    say(f"softmax special rows L={L}")
    x = np.random.default_rng(8).standard_normal(6 * L).astype(np.float32)
    x[3] = np.nan
    x[L + 5] = np.inf
    x[2 * L:3 * L] = -np.inf
    x[3 * L + 1] = -np.inf
    x[4 * L:5 * L] = 88.0
    x[5 * L + L // 2] = 1e4  # one element far above the rest: every other is exp(-inf-ish) = 0
    bufs = {"x": x, "y": np.zeros(6 * L, np.float32)}
    wl = Workload("softmax-special", bufs, {"x": "f32", "y": "f32"},
                  [Op("row_softmax", Ref("y"), (Ref("x"),), n=6 * L, rows=6, row_len=L)], outputs=["y"])
    check(wl, runner.run_resident(wl))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rope(dtype):
    _need_gpu()
    rng = np.random.default_rng(9)
    for heads, hd in ((14, 64), (3, 10), (1, 128)):
        say(f"rope {dtype} heads={heads} hd={hd}")
        n = heads * hd
        conv = (lambda a: workloads.f32_to_bf16_trunc(a)) if dtype == "bf16" else (lambda a: a)
        bufs = {"x": conv(rng.standard_normal(n).astype(np.float32)),
                "t": workloads.rope_table([537], hd)[0],
                "y": np.zeros(n, np.uint16 if dtype == "bf16" else np.float32)}
        ops = [Op("rope", Ref("y"), (Ref("x"),), Ref("t"), n=n, dtype=dtype, rows=heads, row_len=hd,
                  dims=(heads, hd)),
               Op("rope", Ref("x"), (Ref("x"),), Ref("t"), n=n, dtype=dtype, rows=heads, row_len=hd,
                  dims=(heads, hd))]  # in place
        wl = Workload("rope", bufs, {"x": dtype, "t": "f32", "y": dtype}, ops, outputs=["y", "x"])
        check(wl, runner.run_resident(wl))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gemv(dtype):
    _need_gpu()
    rng = np.random.default_rng(10)
    for M, K in ((1, 8), (5, 7), (2688, 896), (896, 4864), (9728, 896), (33, 100)):
        say(f"gemv {dtype} M={M} K={K}")
        conv = (lambda a: workloads.f32_to_bf16_trunc(a)) if dtype == "bf16" else (lambda a: a)
        bufs = {"W": workloads.f32_to_bf16_trunc((rng.standard_normal(M * K) * 0.05).astype(np.float32)),
                "x": conv(rng.standard_normal(K).astype(np.float32)),
                "y": np.zeros(M, np.uint16 if dtype == "bf16" else np.float32)}
        wl = Workload("gemv", bufs, {"W": "bf16", "x": dtype, "y": dtype},
                      [Op("gemv", Ref("y"), (Ref("x"),), Ref("W"), n=M, dtype=dtype, dims=(M, K))],
                      outputs=["y"])
        check(wl, runner.run_resident(wl))


def _gemv_add_workload(dtype, M, K, res_first, in_place, seed):
    rng = np.random.default_rng(seed)
    conv = (lambda a: workloads.f32_to_bf16_trunc(a)) if dtype == "bf16" else (lambda a: a)
    npdt = np.uint16 if dtype == "bf16" else np.float32
    bufs = {"W": workloads.f32_to_bf16_trunc((rng.standard_normal(M * K) * 0.05).astype(np.float32)),
            "x": conv(rng.standard_normal(K).astype(np.float32)),
            "r": conv(rng.standard_normal(M).astype(np.float32)),
            "y": np.zeros(M, npdt), "z": np.zeros(M, npdt)}
    z = "r" if in_place else "z"
    ins = (Ref("r"), Ref("y")) if res_first else (Ref("y"), Ref("r"))
    ops = [Op("gemv", Ref("y"), (Ref("x"),), Ref("W"), n=M, dtype=dtype, dims=(M, K)),
           Op("add", Ref(z), ins, n=M, dtype=dtype)]
    dts = {"W": "bf16", "x": dtype, "r": dtype, "y": dtype, "z": dtype}
    return Workload("gemv_add", bufs, dts, ops, outputs=["y", z])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gemv_add_fused(dtype):
    """GEMV followed by a residual ADD runs as one descriptor; each op is
    checked on the GPU's own inputs, and the fused run stores exactly what
    the two separate ops store (also when the ADD writes the residual in
    place)."""
    _need_gpu()
    for M, K, res_first in ((896, 896, True), (896, 4864, False), (1000, 6000, True),
                            (33, 100, False), (1, 8, True)):
        say(f"gemv+add {dtype} M={M} K={K} res_first={res_first}")
        wl = _gemv_add_workload(dtype, M, K, res_first, False, 20 + M)
        got = runner.run_resident(wl)
        bad = oracle.local_check(wl, got, oracle.compare)
        assert not bad, [(i, n, str(r)) for i, n, r in bad]
        for in_place in (False, True):
            wl = _gemv_add_workload(dtype, M, K, res_first, in_place, 20 + M)
            fused = runner.run_resident(wl, fusion=1)
            plain = runner.run_resident(wl, fusion=2)
            for name in wl.outputs:
                assert np.array_equal(fused[name].view(np.uint8), plain[name].view(np.uint8)), name


@pytest.mark.parametrize("H,D,S", [(14, 64, 512), (2, 8, 5), (3, 10, 70), (4, 128, 64),
                                   (2, 16, 100), (1, 8, 4)])
def test_attention(H, D, S):
    _need_gpu()
    say(f"attention H={H} D={D} S={S}")
    rng = np.random.default_rng(11)
    bf = workloads.f32_to_bf16_trunc
    bufs = {"q": bf(rng.standard_normal(H * D).astype(np.float32)),
            "K": bf(rng.standard_normal(S * H * D).astype(np.float32)),
            "V": bf(rng.standard_normal(S * H * D).astype(np.float32)),
            "s": np.zeros(H * S, np.float32), "p": np.zeros(H * S, np.float32),
            "o": np.zeros(H * D, np.uint16)}
    ops = [Op("attn_score", Ref("s"), (Ref("q"),), Ref("K"), n=H * S, dtype="bf16",
              alpha=1 / math.sqrt(D), dims=(H, D, S)),
           Op("row_softmax", Ref("p"), (Ref("s"),), n=H * S, rows=H, row_len=S),
           Op("attn_av", Ref("o"), (Ref("p"),), Ref("V"), n=H * D, dtype="bf16", dims=(H, D, S))]
    wl = Workload("attn", bufs, {"q": "bf16", "K": "bf16", "V": "bf16", "s": "f32", "p": "f32",
                                 "o": "bf16"}, ops, outputs=["s", "p", "o"])
    got = runner.run_resident(wl)
    # local check: each op against the oracle run on the GPU's own inputs
    want, sc = oracle.run(wl, upto=1, scales=True)
    assert oracle.compare(got["s"], want["s"], "f32", sc["s"]).ok
    b2 = dict(wl.buffers, s=got["s"])
    want, sc = oracle.run(Workload("attn", b2, wl.dtypes, ops[1:2]), scales=True)
    assert oracle.compare(got["p"], want["p"], "f32", sc["p"]).ok
    b3 = dict(wl.buffers, p=got["p"])
    want, sc = oracle.run(Workload("attn", b3, wl.dtypes, ops[2:3]), scales=True)
    r = oracle.compare(got["o"], want["o"], "bf16", sc["o"])
    assert r.ok, str(r)
    # softmax and AV fused into one descriptor (when the shape allows) store
    # exactly what the separate ops store
    plain = runner.run_resident(wl, fusion=2)
    for name in ("s", "p", "o"):
        assert np.array_equal(got[name].view(np.uint8), plain[name].view(np.uint8)), name


def test_gather():
    _need_gpu()
    say("gather")
    rng = np.random.default_rng(12)
    x = rng.standard_normal(1000).astype(np.float32)
    idx = rng.integers(0, 1000, 5000).astype(np.int32)
    bufs = {"x": x, "i": idx, "y": np.zeros(5000, np.float32)}
    wl = Workload("gather", bufs, {"x": "f32", "i": "i32", "y": "f32"},
                  [Op("gather", Ref("y"), (Ref("x"),), Ref("i"), n=5000, src_len=(1000, 0))],
                  outputs=["y"])
    check(wl, runner.run_resident(wl))


def test_small_decode_local_check():
    _need_gpu()
    say("decode 2 layers x 3 tokens, verification form")
    wl = workloads.gen_decode(seed=0, layers=2, tokens=3, distinct=True)
    got = runner.run_resident(wl)
    bad = oracle.local_check(wl, got, oracle.compare)
    assert not bad, [(i, wl.ops[i].kind, n, str(r)) for i, n, r in bad[:5]]


@pytest.mark.parametrize("H,hd", [(14, 64), (3, 16), (2, 128), (5, 8)])
def test_norm_gemv_rotary_fused(H, hd):
    """RMSNORM -> GEMV(q|k|v) -> ROPE q, ROPE k (into a cache slot), COPY v
    (into a cache slot) as one descriptor: each op checked on the GPU's own
    inputs, and the fused run stores exactly what the five separate ops
    store."""
    _need_gpu()
    say(f"norm-gemv rotary H={H} hd={hd}")
    D, S, slot = H * hd, 4, 2
    rng = np.random.default_rng(30 + H)
    bf = workloads.f32_to_bf16_trunc
    tab = workloads.rope_table([17], hd).reshape(-1)
    bufs = {"x": bf(rng.standard_normal(D).astype(np.float32)),
            "g": bf((rng.standard_normal(D) * 0.5).astype(np.float32)),
            "W": bf((rng.standard_normal(3 * D * D) * 0.05).astype(np.float32)),
            "tab": tab.astype(np.float32),
            "h": np.zeros(D, np.uint16), "qkv": np.zeros(3 * D, np.uint16), "q": np.zeros(D, np.uint16),
            "K": bf(rng.standard_normal(S * D).astype(np.float32)),
            "V": bf(rng.standard_normal(S * D).astype(np.float32))}
    dts = {k: "bf16" for k in bufs}
    dts["tab"] = "f32"
    ops = [Op("rmsnorm", Ref("h"), (Ref("x"),), Ref("g"), n=D, dtype="bf16", rows=1, row_len=D,
              eps=float(np.float32(1e-6))),
           Op("gemv", Ref("qkv"), (Ref("h"),), Ref("W"), n=3 * D, dtype="bf16", dims=(3 * D, D)),
           Op("rope", Ref("q"), (Ref("qkv", 0),), Ref("tab"), n=D, dtype="bf16", rows=H, row_len=hd,
              dims=(H, hd)),
           Op("rope", Ref("K", slot * D), (Ref("qkv", D),), Ref("tab"), n=D, dtype="bf16", rows=H,
              row_len=hd, dims=(H, hd)),
           Op("copy", Ref("V", slot * D), (Ref("qkv", 2 * D),), n=D, dtype="bf16")]
    wl = Workload("norm_gemv_rope", bufs, dts, ops, outputs=["h", "qkv", "q", "K", "V"])
    got = runner.run_resident(wl)
    bad = oracle.local_check(wl, got, oracle.compare)
    assert not bad, [(i, n, str(r)) for i, n, r in bad]
    plain = runner.run_resident(wl, fusion=2)
    for name in wl.outputs:
        assert np.array_equal(got[name], plain[name]), name


def test_decode_fusion_is_bit_identical():
    """The decode's fused descriptors (RMSNORM -> GEMV -> SILU_MUL, RMSNORM ->
    GEMV -> ROPE q, ROPE k, COPY v, GEMV -> residual ADD, ROW_SOFTMAX ->
    ATTN_AV) store exactly the values the separate ops store (same sums in
    the same order, same bf16 roundings)."""
    _need_gpu()
    say("decode 3 layers x 3 tokens, fusion on vs off")
    outs = {}
    for fusion in (1, 2):
        wl = workloads.gen_decode(seed=4, layers=3, tokens=3)
        names = (["x", "h", "qkv", "q", "scores", "probs", "attn", "o", "gu", "act", "down"] +
                 [f"K{l}" for l in range(3)] + [f"V{l}" for l in range(3)])
        outs[fusion] = runner.run_resident(wl, outputs=names, fusion=fusion)
    for name, v in outs[1].items():
        assert np.array_equal(v, outs[2][name]), name
