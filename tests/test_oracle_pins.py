"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test checks one op definition against a worked example printed on a page,
a closed form, an invariant, exact rational arithmetic on tiny inputs, or an
independent library routine.  They run on the CPU (``-m "not gpu"``).
"""

import itertools
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import bf16_to_f32, compare, f32_to_bf16
from oracle.interpreter import apply_op, out_len
from persistent_fusion_amd import traffic
from persistent_fusion_amd.workloads import (Op, Ref, Workload, gen_decode, gen_dynamic_dag,
                                             gen_elementwise_queue, gen_fused_chain,
                                             gen_priority_mix, rope_table)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32(v: float) -> float:
    """Python double rounded to the nearest fp32 (C cast semantics)."""
    try:
        return struct.unpack("<f", struct.pack("<f", v))[0]
    except OverflowError:
        return math.copysign(math.inf, v)


def bits32(v) -> int:
    return int(np.float32(v).view(np.uint32))


def wl_of(bufs, ops, dtypes=None):
    dts = dtypes or {k: ("bf16" if v.dtype == np.uint16 else "i32" if v.dtype == np.int32
                         else "f16" if v.dtype == np.float16 else "f32")
                     for k, v in bufs.items()}
    return Workload("t", {k: np.asarray(v) for k, v in bufs.items()}, dts, ops)


# ----------------------------------------------------------------------------
# worked example from the pages


def _read_golden():
    rows, consts, nbytes = [], None, {}
    with open(os.path.join(GOLDEN, "relu_axb_constants.txt")) as f:
        for line in f:
            t = line.split()
            if not t or t[0].startswith("#"):
                continue
            if t[0] == "const":
                consts = (float(t[1]), float(t[2]))
            elif t[0] == "row":
                rows.append((int(t[1]), float(t[2]), float(t[3])))
            else:
                nbytes[t[0]] = int(t[1])
    return consts, rows, nbytes


def test_golden_relu_axb_page_constants():
    (a, b), rows, _ = _read_golden()
    n = 200
    x = (np.arange(n) % 100 - 50).astype(np.float32)
    bufs = {"x": x, "bv": np.full(n, b, np.float32), "av": np.full(n, a, np.float32),
            "t1": np.zeros(n, np.float32), "t2": np.zeros(n, np.float32),
            "y": np.zeros(n, np.float32), "y2": np.zeros(n, np.float32)}
    ops = [
        # scalar a as SCALE's alpha, scalar b as a constant vector
        Op("scale", Ref("t1"), (Ref("x"),), n=n, alpha=a),
        Op("add", Ref("t2"), (Ref("t1"), Ref("bv")), n=n),
        Op("relu", Ref("y"), (Ref("t2"),), n=n),
        # the same chain with a as a vector operand
        Op("mul", Ref("t1"), (Ref("av"), Ref("x")), n=n),
        Op("add", Ref("t2"), (Ref("t1"), Ref("bv")), n=n),
        Op("relu", Ref("y2"), (Ref("t2"),), n=n),
    ]
    out = oracle.run(wl_of(bufs, ops))
    for i, xi, yi in rows:
        assert out["x"][i] == xi
        assert out["y"][i] == np.float32(yi), (i, out["y"][i], yi)
        assert out["y2"][i] == np.float32(yi)
        assert bits32(out["y"][i]) == bits32(yi)  # +0, never -0


def test_golden_traffic_model_page_bytes():
    _, _, nbytes = _read_golden()
    n = 1000
    chain = [Op("mul", Ref("t1"), (Ref("a"), Ref("x")), n=n, transient=True),
             Op("add", Ref("t2"), (Ref("t1"), Ref("b")), n=n, transient=True),
             Op("relu", Ref("y"), (Ref("t2"),), n=n)]
    scal = {"a", "b"}
    assert traffic.unfused_bytes(chain, scal) == nbytes["bytes_unfused"] * n
    assert traffic.fused_chain_bytes(chain, scal) == nbytes["bytes_fused"] * n
    # vector a, b (the 16M-element workload): 32 vs 16 bytes per element
    assert traffic.unfused_bytes(chain) == 32 * n
    assert traffic.fused_chain_bytes(chain) == 16 * n
    wl = gen_fused_chain(n=4096)
    assert traffic.fused_chain_bytes(wl.ops) == wl.meta["fused_bytes"] // wl.meta["n"] * 4096


def test_golden_launch_model_page_figures():
    """The launch-cost model reproduces the figures the page prints for its
    decode step, at the page's rounding."""
    vals = {}
    with open(os.path.join(GOLDEN, "launch_model.txt")) as f:
        for line in f:
            t = line.split()
            if t and not t[0].startswith("#"):
                vals[t[0]] = [float(v) for v in t[1:]]
    launches, per_us, compute_ms = vals["inputs"]
    m = traffic.launch_model(int(launches), per_us * 1e-6, compute_ms * 1e-3)
    ov_ms, tot_ms, pct = vals["printed"]
    assert f"{m['overhead_s'] * 1e3:.1f}" == f"{ov_ms:.1f}"
    assert f"{m['total_s'] * 1e3:.1f}" == f"{tot_ms:.1f}"
    assert f"{100 * m['share']:.0f}" == f"{pct:.0f}"
    # invariants: no launches cost nothing; doubling the work per launch (a
    # larger batch under the same launches) lowers the share
    assert traffic.launch_model(0, 1e-5, 1e-3)["share"] == 0.0
    a = traffic.launch_model(400, 1e-5, 2e-3)["share"]
    b = traffic.launch_model(400, 1e-5, 4e-3)["share"]
    assert b < a
    with pytest.raises(ValueError):
        traffic.launch_model(-1, 1e-5, 1e-3)


# ----------------------------------------------------------------------------
# closed forms on constants


@pytest.mark.parametrize("a,x,b,want", [(2.0, 3.0, -7.0, 0.0), (0.5, 3.0, 0.25, 1.75),
                                        (1.5, -50.0, 0.5, 0.0), (1.5, 49.0, 0.5, 74.0)])
def test_relu_axb_closed_form(a, x, b, want):
    n = 5
    bufs = {"a": np.full(n, a, np.float32), "x": np.full(n, x, np.float32),
            "b": np.full(n, b, np.float32), "t": np.zeros(n, np.float32),
            "u": np.zeros(n, np.float32), "y": np.zeros(n, np.float32)}
    ops = [Op("mul", Ref("t"), (Ref("a"), Ref("x")), n=n),
           Op("add", Ref("u"), (Ref("t"), Ref("b")), n=n),
           Op("relu", Ref("y"), (Ref("u"),), n=n)]
    out = oracle.run(wl_of(bufs, ops))
    assert np.all(out["y"] == np.float32(want))
    assert np.all(out["y"].view(np.uint32) == bits32(want))


def test_relu_signed_zero_nan_and_denormals():
    vals = np.array([-0.0, 0.0, np.nan, -np.nan, np.inf, -np.inf, 1e-45, -1e-45, 3.0, -3.0],
                    np.float32)
    n = vals.size
    bufs = {"x": vals, "y": np.zeros(n, np.float32)}
    out = oracle.run(wl_of(bufs, [Op("relu", Ref("y"), (Ref("x"),), n=n)]))
    want = [0.0, 0.0, 0.0, 0.0, math.inf, 0.0, 1e-45, 0.0, 3.0, 0.0]
    for g, w in zip(out["y"], want):
        assert bits32(g) == bits32(w)


def test_denormals_are_preserved():
    d = np.float32(2.0 ** -140)  # subnormal in fp32
    n = 4
    bufs = {"a": np.full(n, d, np.float32), "b": np.full(n, d, np.float32),
            "h": np.full(n, 2.0 ** -10, np.float32),
            "s": np.zeros(n, np.float32), "p": np.zeros(n, np.float32)}
    ops = [Op("add", Ref("s"), (Ref("a"), Ref("b")), n=n),
           Op("mul", Ref("p"), (Ref("a"), Ref("h")), n=n)]
    out = oracle.run(wl_of(bufs, ops))
    assert np.all(out["s"] == np.float32(2.0 ** -139))
    # 2^-150 is exactly half the smallest subnormal: ties-to-even rounds it to +0
    assert np.all(out["p"].view(np.uint32) == 0)
    bufs["h"] = np.full(n, 2.0 ** -3, np.float32)
    out = oracle.run(wl_of(bufs, ops))
    assert np.all(out["p"] == np.float32(2.0 ** -143))


# ----------------------------------------------------------------------------
# brute force on tiny queues: an independent per-element evaluator


def _eval_queue_elementwise(wl: Workload):
    """Recursive per-element evaluation of a fp32 elementwise queue.

    The value of buffer b at element k just before op p runs is the output of
    the last earlier op that wrote that element, evaluated element-wise in
    Python doubles and rounded to fp32 after each operation (double rounding
    is innocuous for one fp32 add or multiply), or the initial contents.
    """
    memo = {}

    def value(buf, k, pos):
        key = (buf, k, pos)
        if key in memo:
            return memo[key]
        v = None
        for j in range(pos - 1, -1, -1):
            op = wl.ops[j]
            if op.out.buf == buf and op.out.off <= k < op.out.off + op.n:
                v = op_elem(j, k - op.out.off)
                break
        if v is None:
            v = float(wl.buffers[buf][k])
        memo[key] = v
        return v

    def op_elem(j, e):
        op = wl.ops[j]
        srcs = []
        for i, r in enumerate(op.ins):
            L = op.src_len[i] or op.n
            srcs.append(value(r.buf, r.off + (e % L), j))
        if op.kind == "add":
            return f32(srcs[0] + srcs[1])
        if op.kind == "mul":
            return f32(srcs[0] * srcs[1])
        if op.kind == "scale":
            return f32(float(np.float32(op.alpha)) * srcs[0])
        if op.kind == "relu":
            return srcs[0] if srcs[0] > 0 else 0.0
        if op.kind == "copy":
            return srcs[0]
        raise AssertionError(op.kind)

    final = {}
    for name, arr in wl.buffers.items():
        final[name] = np.array([value(name, k, len(wl.ops)) for k in range(arr.shape[0])],
                               np.float32)
    return final


def _same_bits(a, b):
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    both_nan = np.isnan(a) & np.isnan(b)
    return bool(np.all((a.view(np.uint32) == b.view(np.uint32)) | both_nan))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_elementwise_queue_matches_per_element_evaluation(seed):
    wl = gen_elementwise_queue(seed=seed, n_ops=60, n=16)
    got = oracle.run(wl)
    want = _eval_queue_elementwise(wl)
    for name in wl.buffers:
        assert _same_bits(got[name], want[name]), name


def test_reuse_and_cyclic_queue_matches_per_element_evaluation():
    rng = np.random.default_rng(5)
    bufs = {"A": rng.standard_normal(12).astype(np.float32),
            "B": rng.standard_normal(5).astype(np.float32),
            "C": np.zeros(12, np.float32)}
    ops = [
        Op("mul", Ref("C"), (Ref("A"), Ref("B")), n=12, src_len=(12, 5)),      # cyclic B
        Op("add", Ref("A", 2), (Ref("C", 1), Ref("A")), n=9, src_len=(0, 3)),  # overlap + cyclic
        Op("relu", Ref("C"), (Ref("C"),), n=12),                               # in place
        Op("scale", Ref("B"), (Ref("C", 3),), n=5, alpha=-0.75),
        Op("copy", Ref("A"), (Ref("B"),), n=7, src_len=(5, 0)),
        Op("add", Ref("C", 4), (Ref("A", 1), Ref("C")), n=8),
    ]
    wl = wl_of(bufs, ops)
    got = oracle.run(wl)
    want = _eval_queue_elementwise(wl)
    for name in bufs:
        assert _same_bits(got[name], want[name]), name


def _hazard(a: Op, b: Op) -> bool:
    def rng_(r, cnt):
        return (r.buf, r.off, r.off + cnt)

    def ov(x, y):
        return x[0] == y[0] and x[1] < y[2] and y[1] < x[2]

    wa = rng_(a.out, out_len(a))
    wb = rng_(b.out, out_len(b))
    ra = [rng_(r, a.src_len[i] or a.n) for i, r in enumerate(a.ins)]
    rb = [rng_(r, b.src_len[i] or b.n) for i, r in enumerate(b.ins)]
    return ov(wa, wb) or any(ov(wa, r) for r in rb) or any(ov(wb, r) for r in ra)


def test_every_topological_order_gives_identical_buffers():
    rng = np.random.default_rng(11)
    n = 6
    bufs = {k: rng.standard_normal(n).astype(np.float32) for k in "ABCD"}
    ops = [Op("mul", Ref("C"), (Ref("A"), Ref("B")), n=n),
           Op("add", Ref("D"), (Ref("A"), Ref("A")), n=n),
           Op("relu", Ref("A"), (Ref("C"),), n=n),
           Op("scale", Ref("B"), (Ref("D"),), n=n, alpha=1.25),
           Op("add", Ref("D"), (Ref("B"), Ref("C")), n=n),
           Op("exp", Ref("C"), (Ref("D"),), n=n)]
    base = oracle.run(wl_of(bufs, ops))
    orders = 0
    for perm in itertools.permutations(range(len(ops))):
        pos = {p: i for i, p in enumerate(perm)}
        if any(pos[i] > pos[j] for i in range(len(ops)) for j in range(i + 1, len(ops))
               if _hazard(ops[i], ops[j])):
            continue
        orders += 1
        out = oracle.run(wl_of(bufs, [ops[p] for p in perm]))
        for k in bufs:
            assert _same_bits(out[k], base[k])
    assert orders > 1


# ----------------------------------------------------------------------------
# bf16 conversion


def test_bf16_rounding_edge_cases():
    cases = [
        (1.0, 0x3F80),
        (1.0 + 2.0 ** -8, 0x3F80),            # exact tie: rounds to even (down)
        (1.0 + 3 * 2.0 ** -8, 0x3F82),        # tie between 0x3F81 and 0x3F82: to even (up)
        (1.0 + 2.0 ** -8 + 2.0 ** -20, 0x3F81),  # just above the tie: up
        (-2.5, 0xC020),
        (0.0, 0x0000), (-0.0, 0x8000),
        (math.inf, 0x7F80), (-math.inf, 0xFF80),
        (3.3895313892515355e38, 0x7F7F),     # largest finite bf16
        (3.4e38, 0x7F80),                     # rounds up past the largest finite: inf
        (2.0 ** -133, 0x0001),                # smallest bf16 subnormal
    ]
    x = np.array([c[0] for c in cases], np.float32)
    got = f32_to_bf16(x)
    for (v, want), g in zip(cases, got):
        assert int(g) == want, (v, hex(int(g)), hex(want))
    nan = f32_to_bf16(np.array([np.nan, -np.nan], np.float32))
    assert np.all(np.isnan(bf16_to_f32(nan)))
    assert np.all((nan & 0x7FC0) == 0x7FC0)


def test_bf16_matches_torch_rne():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 1e3,
                        (rng.integers(0, 2 ** 32, 20000, dtype=np.uint64)).astype(np.uint32).view(np.float32)])
    x = x[~np.isnan(x)]
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16(x), want)
    back = bf16_to_f32(want)
    assert np.array_equal(back, torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_bf16_elementwise_is_fp32_then_rne():
    rng = np.random.default_rng(4)
    n = 64
    a = f32_to_bf16(rng.standard_normal(n).astype(np.float32))
    b = f32_to_bf16(rng.standard_normal(n).astype(np.float32))
    bufs = {"a": a, "b": b, "y": np.zeros(n, np.uint16)}
    out = oracle.run(wl_of(bufs, [Op("add", Ref("y"), (Ref("a"), Ref("b")), n=n, dtype="bf16")]))
    torch = pytest.importorskip("torch")
    ta = torch.from_numpy(bf16_to_f32(a))
    tb = torch.from_numpy(bf16_to_f32(b))
    want = (ta + tb).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out["y"], want)


# ----------------------------------------------------------------------------
# EXP


def test_exp_special_values_and_library():
    x = np.array([0.0, -0.0, 1.0, -1.0, 10.5, -20.25, 88.7, 88.8, -100.0, -np.inf, np.inf, np.nan],
                 np.float32)
    n = x.size
    out = oracle.run(wl_of({"x": x, "y": np.zeros(n, np.float32)},
                           [Op("exp", Ref("y"), (Ref("x"),), n=n)]))["y"]
    assert out[0] == 1.0 and out[1] == 1.0
    for xi, yi in zip(x[2:8], out[2:8]):
        assert bits32(yi) == bits32(f32(math.exp(float(xi))))
    assert out[7] == np.inf           # exp(88.8) overflows fp32
    assert out[8] > 0 and out[8] < 2.0 ** -126  # subnormal result is kept
    assert out[9] == 0.0 and out[10] == np.inf and np.isnan(out[11])


# ----------------------------------------------------------------------------
# row reductions


def test_row_sum_exact_cases_and_rational_sum():
    L = 256
    bufs = {"x": np.full(4 * L, 2.0 ** -3, np.float32), "y": np.zeros(4, np.float32)}
    bufs["x"][L:2 * L] = 2.0 ** 5
    bufs["x"][2 * L:3 * L] = -(2.0 ** -20)
    bufs["x"][3 * L:] = np.arange(L, dtype=np.float32)
    out = oracle.run(wl_of(bufs, [Op("row_sum", Ref("y"), (Ref("x"),), n=4 * L, rows=4, row_len=L)]))
    assert list(out["y"]) == [L * 2.0 ** -3, L * 2.0 ** 5, -L * 2.0 ** -20, L * (L - 1) / 2]
    rng = np.random.default_rng(7)
    R, L = 20, 333
    x = (rng.standard_normal(R * L) * np.exp(rng.uniform(-8, 8, R * L))).astype(np.float32)
    bufs = {"x": x, "y": np.zeros(R, np.float32)}
    wl = wl_of(bufs, [Op("row_sum", Ref("y"), (Ref("x"),), n=R * L, rows=R, row_len=L)])
    out, sc = oracle.run(wl, scales=True)
    for r in range(R):
        exact = sum(Fraction(float(v)) for v in x[r * L:(r + 1) * L])
        want = f32(float(exact))
        assert abs(float(out["y"][r]) - want) <= abs(want) * 2.0 ** -23 + 1e-300
        assert sc["y"][r] == pytest.approx(float(np.abs(x[r * L:(r + 1) * L].astype(np.float64)).sum()))


def test_row_sum_permutation_invariant():
    rng = np.random.default_rng(8)
    L = 1000
    x = rng.standard_normal(L).astype(np.float32)
    xp = rng.permutation(x)
    bufs = {"x": np.concatenate([x, xp]), "y": np.zeros(2, np.float32)}
    out, sc = oracle.run(wl_of(bufs, [Op("row_sum", Ref("y"), (Ref("x"),), n=2 * L, rows=2, row_len=L)]),
                         scales=True)
    assert abs(out["y"][0] - out["y"][1]) <= 1e-7 * sc["y"][0]


def _softmax(x, R, L):
    bufs = {"x": np.asarray(x, np.float32), "y": np.zeros(R * L, np.float32)}
    return oracle.run(wl_of(bufs, [Op("row_softmax", Ref("y"), (Ref("x"),), n=R * L, rows=R,
                                      row_len=L)]))["y"].reshape(R, L)


def test_softmax_invariants():
    rng = np.random.default_rng(9)
    R, L = 16, 512
    x = (rng.standard_normal(R * L) * 4).astype(np.float32)
    y = _softmax(x, R, L)
    s = y.astype(np.float64).sum(axis=1)
    assert np.all(np.abs(s - 1.0) <= L * 2.0 ** -24)
    assert np.all(np.argmax(y, axis=1) == np.argmax(x.reshape(R, L), axis=1))
    # shifting a row by a constant leaves it unchanged (within rounding of the shift)
    y2 = _softmax(x + np.float32(3.0), R, L)
    assert np.allclose(y2, y, rtol=1e-5, atol=0)
    # constant rows of power-of-two length give exactly 1/L
    for L2 in (128, 1024, 4096):
        yc = _softmax(np.full(L2, -7.25, np.float32), 1, L2)
        assert np.all(yc == np.float32(1.0 / L2))


def test_softmax_brute_force_and_special_rows():
    rng = np.random.default_rng(10)
    L = 7
    x = rng.standard_normal(3 * L).astype(np.float32)
    y = _softmax(x, 3, L)
    for r in range(3):
        row = [float(v) for v in x[r * L:(r + 1) * L]]
        m = max(row)
        e = [math.exp(v - m) for v in row]
        tot = math.fsum(e)
        for j in range(L):
            assert abs(float(y[r, j]) - e[j] / tot) <= 2.0 ** -23 * (e[j] / tot)
    special = np.array([0, 1, np.nan, 2, 3, np.inf, -np.inf, -np.inf, -np.inf], np.float32)
    ys = _softmax(special, 3, 3)
    assert np.all(np.isnan(ys))


def test_rmsnorm_invariants_and_brute_force():
    rng = np.random.default_rng(12)
    R, L = 6, 896
    x = rng.standard_normal(R * L).astype(np.float32) * 3
    g = (rng.standard_normal(L) * 0.5 + 1).astype(np.float32)
    eps = float(np.float32(1e-6))
    bufs = {"x": x, "g": g, "y": np.zeros(R * L, np.float32)}
    y = oracle.run(wl_of(bufs, [Op("rmsnorm", Ref("y"), (Ref("x"),), Ref("g"), n=R * L, rows=R,
                                   row_len=L, eps=eps)]))["y"].reshape(R, L)
    z = y.astype(np.float64) / g.astype(np.float64)
    rms = np.sqrt((z * z).mean(axis=1))
    assert np.all(np.abs(rms - 1.0) <= 1e-5)
    for r in range(R):
        row = x[r * L:(r + 1) * L]
        ss = sum(Fraction(float(v)) ** 2 for v in row)
        inv = 1.0 / math.sqrt(float(ss / L) + eps)
        for j in (0, 1, 17, L - 1):
            want = float(row[j]) * inv * float(g[j])
            assert abs(float(y[r, j]) - want) <= 2.0 ** -22 * abs(want)
    # rows whose mean square is comparable to eps: catches eps outside the root
    xs = (rng.standard_normal(L) * 1e-3).astype(np.float32)
    bufs = {"x": xs, "g": g, "y": np.zeros(L, np.float32)}
    y = oracle.run(wl_of(bufs, [Op("rmsnorm", Ref("y"), (Ref("x"),), Ref("g"), n=L, rows=1,
                                   row_len=L, eps=eps)]))["y"]
    ss = sum(Fraction(float(v)) ** 2 for v in xs)
    inv = 1.0 / math.sqrt(float(ss / L) + eps)
    for j in (0, 5, L - 1):
        want = float(xs[j]) * inv * float(g[j])
        assert abs(float(y[j]) - want) <= 2.0 ** -22 * abs(want)
    # constant row c: y = sign(c) * g up to the eps term
    bufs = {"x": np.full(L, -2.0, np.float32), "g": g, "y": np.zeros(L, np.float32)}
    y = oracle.run(wl_of(bufs, [Op("rmsnorm", Ref("y"), (Ref("x"),), Ref("g"), n=L, rows=1,
                                   row_len=L, eps=eps)]))["y"]
    assert np.allclose(y, -g, rtol=1e-6)


# ----------------------------------------------------------------------------
# rotary


def _rope(x, tab, heads, hd, dtype="f32"):
    bufs = {"x": x, "t": np.asarray(tab, np.float32),
            "y": np.zeros(heads * hd, np.uint16 if dtype == "bf16" else np.float32)}
    return oracle.run(wl_of(bufs, [Op("rope", Ref("y"), (Ref("x"),), Ref("t"), n=heads * hd,
                                      dtype=dtype, rows=heads, row_len=hd, dims=(heads, hd))]))["y"]


def test_rope_position_zero_is_identity_and_quarter_turn_swaps():
    rng = np.random.default_rng(13)
    H, hd = 3, 8
    x = rng.standard_normal(H * hd).astype(np.float32)
    tab0 = rope_table([0], hd)[0]
    assert np.all(tab0[:hd // 2] == 1) and np.all(tab0[hd // 2:] == 0)
    assert _same_bits(_rope(x, tab0, H, hd), x)
    quarter = np.concatenate([np.zeros(hd // 2), np.ones(hd // 2)]).astype(np.float32)
    y = _rope(x, quarter, H, hd).reshape(H, hd)
    xr = x.reshape(H, hd)
    assert np.array_equal(y[:, :hd // 2], -xr[:, hd // 2:])
    assert np.array_equal(y[:, hd // 2:], xr[:, :hd // 2])


def test_rope_brute_force_and_norm():
    rng = np.random.default_rng(14)
    H, hd = 4, 64
    x = rng.standard_normal(H * hd).astype(np.float32)
    tab = rope_table([531], hd)[0]
    y = _rope(x, tab, H, hd)
    half = hd // 2
    for h in range(H):
        for i in range(half):
            a, b = float(x[h * hd + i]), float(x[h * hd + half + i])
            c, s = float(tab[i]), float(tab[half + i])
            assert bits32(y[h * hd + i]) == bits32(f32(f32(a * c) - f32(b * s)))
            assert bits32(y[h * hd + half + i]) == bits32(f32(f32(b * c) + f32(a * s)))
            n0 = math.hypot(a, b)
            n1 = math.hypot(float(y[h * hd + i]), float(y[h * hd + half + i]))
            assert abs(n1 - n0) <= 4 * 2.0 ** -24 * n0
    # bf16 output is the fp32 rotation rounded with RNE
    yb = _rope(f32_to_bf16(x), tab, H, hd, "bf16")
    yf = _rope(bf16_to_f32(f32_to_bf16(x)), tab, H, hd)
    assert np.array_equal(yb, f32_to_bf16(yf))


# ----------------------------------------------------------------------------
# GEMV and attention


def _exact_dot(a, b):
    return float(sum(Fraction(float(p)) * Fraction(float(q)) for p, q in zip(a, b)))


def test_gemv_identity_onehot_and_rational_dot():
    rng = np.random.default_rng(15)
    K = 8
    x = f32_to_bf16(rng.standard_normal(K).astype(np.float32))
    eye = f32_to_bf16(np.eye(K, dtype=np.float32).reshape(-1))
    bufs = {"W": eye, "x": x, "y": np.zeros(K, np.uint16)}
    y = oracle.run(wl_of(bufs, [Op("gemv", Ref("y"), (Ref("x"),), Ref("W"), n=K, dtype="bf16",
                                   dims=(K, K))]))["y"]
    assert np.array_equal(y, x)
    # one-hot rows act as a gather
    M = 5
    idx = [3, 0, 7, 7, 2]
    W = np.zeros((M, K), np.float32)
    W[np.arange(M), idx] = 1.0
    bufs = {"W": f32_to_bf16(W.reshape(-1)), "x": x, "y": np.zeros(M, np.uint16)}
    y = oracle.run(wl_of(bufs, [Op("gemv", Ref("y"), (Ref("x"),), Ref("W"), n=M, dtype="bf16",
                                   dims=(M, K))]))["y"]
    assert np.array_equal(y, x[idx])
    # non-square, fp32 output, against an exact rational dot product
    M, K = 5, 7
    W = f32_to_bf16(rng.standard_normal(M * K).astype(np.float32))
    xf = rng.standard_normal(K).astype(np.float32)
    bufs = {"W": W, "x": xf, "y": np.zeros(M, np.float32)}
    y = oracle.run(wl_of(bufs, [Op("gemv", Ref("y"), (Ref("x"),), Ref("W"), n=M, dims=(M, K))]))["y"]
    Wf = bf16_to_f32(W).reshape(M, K)
    for i in range(M):
        assert bits32(y[i]) == bits32(f32(_exact_dot(Wf[i], xf)))


def test_attention_brute_force():
    rng = np.random.default_rng(16)
    H, D, S = 3, 4, 5
    q = f32_to_bf16(rng.standard_normal(H * D).astype(np.float32))
    Kc = f32_to_bf16(rng.standard_normal(S * H * D).astype(np.float32))
    Vc = f32_to_bf16(rng.standard_normal(S * H * D).astype(np.float32))
    p = rng.uniform(0, 1, H * S).astype(np.float32)
    bufs = {"q": q, "K": Kc, "V": Vc, "p": p, "s": np.zeros(H * S, np.float32),
            "o": np.zeros(H * D, np.float32)}
    ops = [Op("attn_score", Ref("s"), (Ref("q"),), Ref("K"), n=H * S, dtype="bf16", alpha=0.5,
              dims=(H, D, S)),
           Op("attn_av", Ref("o"), (Ref("p"),), Ref("V"), n=H * D, dtype="f32", dims=(H, D, S))]
    wl = wl_of(bufs, ops)
    wl.dtypes["o"] = "f32"
    out = oracle.run(wl)
    qf, Kf, Vf = bf16_to_f32(q), bf16_to_f32(Kc), bf16_to_f32(Vc)
    for h in range(H):
        for j in range(S):
            ex = 0.5 * _exact_dot(qf[h * D:(h + 1) * D], Kf[j * H * D + h * D: j * H * D + (h + 1) * D])
            assert bits32(out["s"][h * S + j]) == bits32(f32(ex))
        for d in range(D):
            ex = _exact_dot(p[h * S:(h + 1) * S], [Vf[j * H * D + h * D + d] for j in range(S)])
            assert bits32(out["o"][h * D + d]) == bits32(f32(ex))


def test_attention_zero_query_gives_column_mean():
    rng = np.random.default_rng(17)
    H, D, S = 2, 8, 512
    Kc = f32_to_bf16(rng.standard_normal(S * H * D).astype(np.float32))
    Vc = f32_to_bf16(rng.standard_normal(S * H * D).astype(np.float32))
    bufs = {"q": np.zeros(H * D, np.uint16), "K": Kc, "V": Vc, "s": np.zeros(H * S, np.float32),
            "p": np.zeros(H * S, np.float32), "o": np.zeros(H * D, np.float32)}
    ops = [Op("attn_score", Ref("s"), (Ref("q"),), Ref("K"), n=H * S, dtype="bf16", alpha=0.125,
              dims=(H, D, S)),
           Op("row_softmax", Ref("p"), (Ref("s"),), n=H * S, rows=H, row_len=S),
           Op("attn_av", Ref("o"), (Ref("p"),), Ref("V"), n=H * D, dtype="f32", dims=(H, D, S))]
    out = oracle.run(wl_of(bufs, ops))
    assert np.all(out["s"] == 0)
    assert np.all(out["p"] == np.float32(1.0 / S))
    Vf = bf16_to_f32(Vc).reshape(S, H * D)
    for c in range(H * D):
        want = f32(float(sum(Fraction(float(v)) for v in Vf[:, c]) / S))
        assert bits32(out["o"][c]) == bits32(want)


def test_silu_mul_limits():
    g = np.array([0.0, 30.0, -30.0, 1.0, -1.0, 200.0, -200.0], np.float32)
    u = np.array([5.0, 2.0, 2.0, 3.0, 3.0, 1.0, 1.0], np.float32)
    n = g.size
    bufs = {"g": g, "u": u, "y": np.zeros(n, np.float32)}
    y = oracle.run(wl_of(bufs, [Op("silu_mul", Ref("y"), (Ref("g"), Ref("u")), n=n)]))["y"]
    assert y[0] == 0.0
    assert y[1] == np.float32(60.0)
    assert 0 > float(y[2]) > -1e-11
    assert bits32(y[3]) == bits32(f32(1.0 / (1.0 + math.exp(-1.0)) * 3.0))
    assert bits32(y[4]) == bits32(f32(-1.0 / (1.0 + math.exp(1.0)) * 3.0))
    assert y[5] == 200.0 and float(y[6]) <= 0 and float(y[6]) > -1e-80


def test_gather_and_copy():
    x = np.arange(10, dtype=np.float32) * 1.5
    idx = np.array([9, 0, 3, 3, 7], np.int32)
    bufs = {"x": x, "i": idx, "y": np.zeros(5, np.float32), "z": np.zeros(23, np.float32)}
    out = oracle.run(wl_of(bufs, [Op("gather", Ref("y"), (Ref("x"),), Ref("i"), n=5, src_len=(10, 0)),
                                  Op("copy", Ref("z"), (Ref("x", 2),), n=23, src_len=(4, 0))]))
    assert list(out["y"]) == [x[9], x[0], x[3], x[3], x[7]]
    assert list(out["z"]) == [x[2 + (k % 4)] for k in range(23)]
    bufs["i"] = np.array([0, 10, 1, 1, 1], np.int32)
    with pytest.raises(oracle.OracleError):
        oracle.run(wl_of(bufs, [Op("gather", Ref("y"), (Ref("x"),), Ref("i"), n=5, src_len=(10, 0))]))


# ----------------------------------------------------------------------------
# fp16, int32 and views (the generic tensor abstraction of "GPUOS: A GPU
# Operating System Primitive for Transparent Operation Fusion", section "The
# Paper": arbitrary shapes, strides, dtypes, broadcasting)


def _f16_neighbours_and_midpoints():
    """Every finite positive fp16 value, and the exact midpoint between each
    pair of neighbours (12 significant bits: exact in fp32)."""
    bits = np.arange(0, 0x7C00, dtype=np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2.0
    return bits, vals, mids


def test_f16_rounding_is_round_to_nearest_even():
    bits, vals, mids = _f16_neighbours_and_midpoints()
    # exact values survive widening and narrowing
    rt = oracle.run(wl_of({"x": bits.view(np.float16), "o": np.zeros(bits.size, np.float16)},
                          [Op("relu", Ref("o"), (Ref("x"),), n=bits.size, dtype="f16")]))
    assert np.array_equal(rt["o"].view(np.uint16), bits)  # relu of a non-negative value is the value
    # ties go to the neighbour with an even last bit, others to the nearest
    from oracle.interpreter import _store_from_f32
    got = _store_from_f32(mids.astype(np.float32), "f16").view(np.uint16)
    lo, hi = bits[:-1], bits[1:]
    want = np.where(lo % 2 == 0, lo, hi)
    assert np.array_equal(got, want)
    quarter = (3 * vals[:-1] + vals[1:]) / 4.0  # closer to the lower neighbour
    assert np.array_equal(_store_from_f32(quarter.astype(np.float32), "f16").view(np.uint16), lo)
    # overflow: the largest finite fp16 is 65504; halfway to 2^16 and beyond is inf
    big = _store_from_f32(np.array([65504.0, 65519.0, 65520.0, 1e6, -1e6], np.float32), "f16")
    assert list(big[:2]) == [65504.0, 65504.0] and np.isinf(big[2:]).all()


def test_f16_matches_torch_half():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(40)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 100,
                        rng.standard_normal(2000).astype(np.float32) * 1e-6])
    from oracle.interpreter import _store_from_f32
    want = torch.from_numpy(x).half().numpy()
    assert np.array_equal(_store_from_f32(x, "f16").view(np.uint16), want.view(np.uint16))


def test_f16_elementwise_is_fp32_then_rne():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(41)
    n = 257
    a = rng.standard_normal(n).astype(np.float16)
    b = rng.standard_normal(n).astype(np.float16)
    bufs = {"a": a, "b": b, "y": np.zeros(n, np.float16), "z": np.zeros(n, np.float16)}
    out = oracle.run(wl_of(bufs, [Op("mul", Ref("y"), (Ref("a"), Ref("b")), n=n, dtype="f16"),
                                  Op("scale", Ref("z"), (Ref("a"),), n=n, dtype="f16", alpha=0.3)]))
    ta, tb = torch.from_numpy(a).float(), torch.from_numpy(b).float()
    assert np.array_equal(out["y"].view(np.uint16), (ta * tb).half().numpy().view(np.uint16))
    sc = (torch.tensor(np.float32(0.3)) * ta).half().numpy()
    assert np.array_equal(out["z"].view(np.uint16), sc.view(np.uint16))


def test_int32_add_mul_wrap_and_relu():
    rng = np.random.default_rng(42)
    edge = [0, 1, -1, 2 ** 31 - 1, -2 ** 31, 2 ** 16, -2 ** 16, 46341, -46341]
    a = np.array(edge + list(rng.integers(-2 ** 31, 2 ** 31, 200)), np.int64)
    b = np.array(list(reversed(edge)) + list(rng.integers(-2 ** 31, 2 ** 31, 200)), np.int64)
    n = a.size
    bufs = {"a": a.astype(np.int32), "b": b.astype(np.int32), "s": np.zeros(n, np.int32),
            "p": np.zeros(n, np.int32), "r": np.zeros(n, np.int32)}
    out = oracle.run(wl_of(bufs, [Op("add", Ref("s"), (Ref("a"), Ref("b")), n=n, dtype="i32"),
                                  Op("mul", Ref("p"), (Ref("a"), Ref("b")), n=n, dtype="i32"),
                                  Op("relu", Ref("r"), (Ref("a"),), n=n, dtype="i32")]))

    def wrap(v):  # Python integers are exact: reduce mod 2^32 into [-2^31, 2^31)
        v %= 2 ** 32
        return v - 2 ** 32 if v >= 2 ** 31 else v

    for i in range(n):
        x, y = int(a[i]), int(b[i])
        assert int(out["s"][i]) == wrap(x + y)
        assert int(out["p"][i]) == wrap(x * y)
        assert int(out["r"][i]) == (x if x > 0 else 0)


def test_view_broadcasts_match_numpy_broadcasting():
    rng = np.random.default_rng(43)
    R, Cn = 5, 7
    x = rng.standard_normal(R * Cn).astype(np.float32)
    row = rng.standard_normal(Cn).astype(np.float32)
    col = rng.standard_normal(R).astype(np.float32)
    bufs = {"x": x, "row": row, "col": col, "y1": np.zeros(R * Cn, np.float32),
            "y2": np.zeros(R * Cn, np.float32), "y3": np.zeros(R * Cn, np.float32),
            "y4": np.zeros(R * Cn, np.float32)}
    ops = [
        # bias add: [R, C] + [C]
        Op("add", Ref("y1"), (Ref("x"), Ref("row")), n=R * Cn,
           view=((R, Cn), (Cn, 1), (Cn, 1), (0, 1))),
        # per-row scale: [R, C] * [R, 1]
        Op("mul", Ref("y2"), (Ref("x"), Ref("col")), n=R * Cn,
           view=((R, Cn), (Cn, 1), (Cn, 1), (1, 0))),
        # transpose: out[j, i] = x[i, j]
        Op("copy", Ref("y3"), (Ref("x"),), n=R * Cn, view=((R, Cn), (1, R), (Cn, 1), (0, 0))),
        # outer product of two vectors
        Op("mul", Ref("y4"), (Ref("col"), Ref("row")), n=R * Cn,
           view=((R, Cn), (Cn, 1), (1, 0), (0, 1))),
    ]
    out = oracle.run(wl_of(bufs, ops))
    X = x.reshape(R, Cn)
    assert np.array_equal(out["y1"].reshape(R, Cn), X + row[None, :])
    assert np.array_equal(out["y2"].reshape(R, Cn), X * col[:, None])
    assert np.array_equal(out["y3"].reshape(Cn, R), X.T)
    assert np.array_equal(out["y4"].reshape(R, Cn), col[:, None] * row[None, :])


def test_view_strided_output_and_in_place():
    x = np.arange(24, dtype=np.float32)
    bufs = {"x": x.copy(), "y": np.full(48, -1.0, np.float32)}
    ops = [Op("scale", Ref("y"), (Ref("x"),), n=24, alpha=2.0, view=((4, 6), (12, 2), (6, 1), (0, 0))),
           Op("relu", Ref("x", 1), (Ref("x", 1),), n=4, view=((2, 2), (12, 1), (12, 1), (0, 0)))]
    out = oracle.run(wl_of(bufs, ops))
    y = out["y"].reshape(4, 12)
    assert np.array_equal(y[:, 0::2], 2.0 * x.reshape(4, 6)) and np.all(y[:, 1::2] == -1.0)
    assert np.array_equal(out["x"], x)  # relu of non-negative values in place leaves them
    # an output addressing an element twice is rejected
    with pytest.raises(oracle.OracleError):
        oracle.run(wl_of({"x": x.copy(), "y": np.zeros(24, np.float32)},
                         [Op("copy", Ref("y"), (Ref("x"),), n=24, view=((4, 6), (0, 1), (6, 1), (0, 0)))]))


# ----------------------------------------------------------------------------
# the comparison rule


def test_compare_flags_one_ulp_in_exact_class_and_accepts_within_tolerance():
    rng = np.random.default_rng(18)
    want = rng.standard_normal(1000).astype(np.float32)
    got = want.copy()
    assert compare(got, want, "f32").ok
    got.view(np.uint32)[123] += 1
    r = compare(got, want, "f32")
    assert r.count == 1 and r.first_index == 123
    scale = np.abs(want).astype(np.float64)
    assert compare(got, want, "f32", scale).ok  # 1 ulp is inside 1e-5 relative
    got[5] = want[5] * (1 + 3e-5)
    assert not compare(got, want, "f32", scale).ok
    # NaN matches NaN in both classes; inf must match by class
    w = np.array([np.nan, np.inf, 1.0], np.float32)
    assert compare(np.array([np.nan, np.inf, 1.0], np.float32), w, "f32").ok
    assert not compare(np.array([np.nan, 3e38, 1.0], np.float32), w, "f32", np.ones(3)).ok
    # -0 differs from +0 in the exact class
    assert not compare(np.array([-0.0], np.float32), np.array([0.0], np.float32), "f32").ok


def test_compare_uses_the_subnormal_spacing_below_the_normal_range():
    # fp32 subnormals are multiples of 2**-149: a relative bound means nothing
    # there, so the tolerance class accepts two steps of that spacing
    want = np.array([3.377129299022809e-43, 2.0 ** -149, 1e-40, 1.0], np.float32)
    scale = np.abs(want).astype(np.float64)
    for steps, ok in ((1, True), (2, True), (3, False)):
        got = want.copy()
        got.view(np.uint32)[0] += steps
        assert compare(got, want, "f32", scale).ok is ok, steps
    got = want.copy()
    got[1] = 0.0  # one step below the smallest subnormal
    assert compare(got, want, "f32", scale).ok
    got = want.copy()
    got[2] = 0.0  # a subnormal of 1e-40 flushed to zero is far more than two steps
    assert not compare(got, want, "f32", scale).ok
    got = want.copy()
    got.view(np.uint32)[3] += 3  # normal range: the relative bound is unchanged
    assert compare(got, want, "f32", scale).ok
    got[3] = np.float32(1.0 + 3e-5)
    assert not compare(got, want, "f32", scale).ok
    # the exact class still needs equal bits
    got = want.copy()
    got.view(np.uint32)[0] += 1
    assert not compare(got, want, "f32").ok
    # bf16 subnormals are multiples of 2**-133
    wb = np.array([0x0005, 0x3F80], np.uint16)
    sb = np.abs(bf16_to_f32(wb)).astype(np.float64)
    assert compare(np.array([0x0007, 0x3F80], np.uint16), wb, "bf16", sb).ok
    assert not compare(np.array([0x0008, 0x3F80], np.uint16), wb, "bf16", sb).ok


# ----------------------------------------------------------------------------
# generators


def test_generators_are_deterministic_and_shaped():
    a = gen_elementwise_queue(seed=0, n_ops=100, n=64)
    b = gen_elementwise_queue(seed=0, n_ops=100, n=64)
    assert [o.kind for o in a.ops] == [o.kind for o in b.ops]
    assert all(np.array_equal(a.buffers[k], b.buffers[k]) for k in a.buffers)
    assert {o.kind for o in a.ops} == {"add", "mul", "relu", "scale"}
    assert np.all(np.abs(a.buffers["S0"]) <= 1)
    dec = gen_decode(layers=2, tokens=3, kv_len=16)
    assert len(dec.ops) == 2 * 3 * 15 and len(dec.groups) == 3
    dag = gen_dynamic_dag(n_ops=500, n_max=1 << 14, pool_len=1 << 14)
    for i, op in enumerate(dag.ops):
        assert all(i - 8 <= d < i for d in op.deps)
        if op.kind in ("row_sum", "row_softmax"):
            # rows = max(1, n // L): a draw shorter than its row becomes one row
            assert op.n == op.rows * op.row_len and 128 <= op.row_len <= 4096
            assert 128 <= op.n <= 1 << 14
        else:
            assert 256 <= op.n <= 1 << 14
    mix = gen_priority_mix(rounds=3, be_n=1024, lc_n=256)
    assert sum(o.lc for o in mix.ops) == 30 and len(mix.ops) == 33


def test_small_decode_runs_and_feeds_back():
    wl = gen_decode(layers=2, tokens=2, kv_len=32)
    out = oracle.run(wl)
    assert not np.array_equal(out["x"], wl.buffers["x"])
    # token t wrote its cache slot t
    assert not np.array_equal(out["K0"][:896], wl.buffers["K0"][:896])
    assert np.array_equal(out["K0"][2 * 896:], wl.buffers["K0"][2 * 896:])


# ----------------------------------------------------------------------------
# PROGRAM ops (operators defined at run time)

from persistent_fusion_amd.workloads import Program  # noqa: E402

NAN = float("nan")
INF = float("inf")


def _run_prog(prog, ins, dt="f32"):
    """Runs one PROGRAM op over the given input columns; returns (out, scale)."""
    npdt = {"f32": np.float32, "f16": np.float16}[dt]
    n = len(ins[0])
    bufs = {f"i{j}": np.asarray(c, npdt) for j, c in enumerate(ins)}
    bufs["y"] = np.zeros(n, npdt)
    op = Op("program", Ref("y"), tuple(Ref(f"i{j}") for j in range(len(ins))), n=n, dtype=dt, prog=prog)
    wl = wl_of(bufs, [op])
    out, scales = oracle.run(wl, scales=True)
    return out["y"], scales.get("y")


def _exact(scale) -> bool:
    """Every element in the exact class (no error scale)."""
    return scale is None or bool(np.all(np.isnan(scale)))


def _one(name, *srcs_vals):
    """A one-instruction program name(r0, r1, r2) over single values."""
    k = len(srcs_vals)
    prog = Program(((name, 3) + tuple(range(k)),), n_inputs=k, result=3)
    y, _ = _run_prog(prog, [[v] for v in srcs_vals])
    return float(y[0])


@pytest.mark.parametrize("name,args,want", [
    ("add", (1.5, 2.25), 3.75),
    ("sub", (5.0, 3.0), 2.0),                 # operand order: a - b
    ("sub", (3.0, 5.0), -2.0),
    ("mul", (3.0, -0.5), -1.5),
    ("div", (1.0, 3.0), struct.unpack("<f", bytes.fromhex("abaaaa3e"))[0]),  # 0x3EAAAAAB
    ("div", (7.0, 2.0), 3.5),
    ("div", (1.0, 0.0), INF),
    ("div", (-1.0, 0.0), -INF),
    ("div", (0.0, 0.0), NAN),
    ("min", (2.0, 3.0), 2.0),
    ("min", (3.0, 2.0), 2.0),
    ("max", (2.0, 3.0), 3.0),
    ("min", (1.0, NAN), NAN),
    ("min", (NAN, 1.0), NAN),
    ("max", (NAN, 1.0), NAN),
    ("min", (-INF, 1.0), -INF),
    ("relu", (-2.0,), 0.0),
    ("relu", (2.0,), 2.0),
    ("relu", (NAN,), 0.0),
    ("exp", (0.0,), 1.0),
    ("exp", (1.0,), f32(math.e)),
    ("exp", (-INF,), 0.0),
    ("exp", (100.0,), INF),
    ("lt", (1.0, 2.0), 1.0),
    ("lt", (2.0, 1.0), 0.0),
    ("lt", (1.0, 1.0), 0.0),
    ("lt", (NAN, 1.0), 0.0),
    ("sel", (0.0, 5.0, 7.0), 7.0),
    ("sel", (2.0, 5.0, 7.0), 5.0),
    ("sel", (NAN, 5.0, 7.0), 5.0),             # NaN != 0
    ("mov", (-3.25,), -3.25),
    ("abs", (-INF,), INF),
    ("neg", (2.5,), -2.5),
])
def test_program_instruction_values(name, args, want):
    got = _one(name, *args)
    if math.isnan(want):
        assert math.isnan(got)
    else:
        assert bits32(got) == bits32(want), (name, args, got, want)


def test_program_signed_zero_rules():
    pz, nz = 0.0, -0.0
    assert bits32(_one("min", pz, nz)) == 0x80000000 and bits32(_one("min", nz, pz)) == 0x80000000
    assert bits32(_one("max", pz, nz)) == 0 and bits32(_one("max", nz, pz)) == 0
    assert bits32(_one("neg", pz)) == 0x80000000
    assert bits32(_one("abs", nz)) == 0
    assert bits32(_one("relu", nz)) == 0
    assert bits32(_one("sel", nz, 5.0, 7.0)) == bits32(7.0)   # -0 == 0
    nan_neg = _one("neg", NAN)
    assert math.isnan(nan_neg) and bits32(nan_neg) >> 31 == 1  # the sign of a NaN flips too


def test_program_arithmetic_is_correctly_rounded_fp32():
    # Python's double result rounded to fp32 is the correctly rounded fp32
    # result of +, -, *, / on fp32 operands (53 >= 2 * 24 + 2: the double
    # rounding is innocuous), an evaluation independent of numpy's float32 ops
    rng = np.random.default_rng(70)
    a = (rng.standard_normal(3000) * np.exp2(rng.integers(-30, 30, 3000))).astype(np.float32)
    b = (rng.standard_normal(3000) * np.exp2(rng.integers(-30, 30, 3000))).astype(np.float32)
    for name, fn in (("add", lambda x, y: x + y), ("sub", lambda x, y: x - y),
                     ("mul", lambda x, y: x * y), ("div", lambda x, y: x / y)):
        prog = Program(((name, 3, 0, 1),), n_inputs=2, result=3)
        y, scale = _run_prog(prog, [a, b])
        assert _exact(scale)
        want = np.array([f32(fn(float(x), float(z))) for x, z in zip(a, b)], np.float32)
        assert np.array_equal(y.view(np.uint32), want.view(np.uint32)), name


def test_program_registers_start_at_plus_zero_and_constants():
    # r5 is never written: it reads +0, so -0 + r5 = +0
    prog = Program((("add", 3, 0, 5),), n_inputs=1, result=3)
    y, _ = _run_prog(prog, [[-0.0, 2.0, NAN]])
    assert bits32(y[0]) == 0 and y[1] == 2.0 and math.isnan(y[2])
    # constants sit in r8..r15; the result may be any register
    prog = Program((("mul", 3, 0, 9), ("add", 4, 3, 15)), n_inputs=1, result=4,
                   consts=(0, 2.5, 0, 0, 0, 0, 0, -1.0))
    y, _ = _run_prog(prog, [[2.0, -4.0]])
    assert list(y) == [4.0, -11.0]
    prog = Program((("mov", 1, 0),), n_inputs=1, result=10, consts=(0, 0, 7.5))
    y, _ = _run_prog(prog, [[1.0, 2.0]])
    assert list(y) == [7.5, 7.5]
    # a later instruction sees an earlier one's result; inputs can be overwritten
    prog = Program((("mul", 0, 0, 0), ("mul", 0, 0, 0), ("sub", 2, 0, 1)), n_inputs=2, result=2)
    y, _ = _run_prog(prog, [[3.0], [1.0]])
    assert y[0] == 80.0  # 3^4 - 1


def test_program_output_is_rounded_once_to_the_dtype():
    # fp16: 1 + 2^-11 is a tie that rounds to 1.0, but the program keeps fp32
    # registers: (1 + 2^-11) + 2^-11 = 1 + 2^-10 is then stored exactly
    prog = Program((("add", 3, 0, 1), ("add", 3, 3, 1)), n_inputs=2, result=3)
    y, _ = _run_prog(prog, [[1.0], [2.0 ** -11]], dt="f16")
    assert y.dtype == np.float16 and float(y[0]) == 1.0 + 2.0 ** -10
    prog = Program((("add", 3, 0, 1),), n_inputs=2, result=3)
    y, _ = _run_prog(prog, [[1.0], [2.0 ** -11]], dt="f16")
    assert float(y[0]) == 1.0  # a single add: the tie goes to even


def test_program_matches_the_builtin_ops():
    rng = np.random.default_rng(71)
    n = 777
    a, x, b = (rng.uniform(-2, 2, n).astype(np.float32) for _ in range(3))
    # relu(a*x + b) as three built-in ops vs one program
    bufs = {"a": a, "x": x, "b": b, "t": np.zeros(n, np.float32), "y": np.zeros(n, np.float32)}
    ops = [Op("mul", Ref("t"), (Ref("a"), Ref("x")), n=n), Op("add", Ref("t"), (Ref("t"), Ref("b")), n=n),
           Op("relu", Ref("y"), (Ref("t"),), n=n)]
    want = oracle.run(wl_of(bufs, ops))["y"]
    prog = Program((("mul", 3, 0, 1), ("add", 3, 3, 2), ("relu", 3, 3)), n_inputs=3, result=3)
    got, scale = _run_prog(prog, [a, x, b])
    assert _exact(scale) and np.array_equal(got.view(np.uint32), want.view(np.uint32))
    # scaling by a constant register is SCALE
    prog = Program((("mul", 3, 8, 0),), n_inputs=1, result=3, consts=(0.3,))
    got, _ = _run_prog(prog, [x])
    bufs = {"x": x, "y": np.zeros(n, np.float32)}
    want = oracle.run(wl_of(bufs, [Op("scale", Ref("y"), (Ref("x"),), n=n, alpha=0.3)]))["y"]
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    # g / (1 + exp(-g)) * u, step by step in fp32, is SILU_MUL within its tolerance
    prog = Program((("neg", 3, 0), ("exp", 3, 3), ("add", 3, 3, 8), ("div", 3, 0, 3), ("mul", 3, 3, 1)),
                   n_inputs=2, result=3, consts=(1.0,))
    got, scale = _run_prog(prog, [a, x])
    assert not _exact(scale)
    bufs = {"g": a, "u": x, "y": np.zeros(n, np.float32)}
    want = oracle.run(wl_of(bufs, [Op("silu_mul", Ref("y"), (Ref("g"), Ref("u")), n=n)]))["y"]
    assert compare(got, want, "f32", np.abs(want.astype(np.float64))).ok


def test_program_ops_write_only_their_output_and_read_every_input():
    rng = np.random.default_rng(72)
    n = 50
    p, q, r = (rng.uniform(-1, 1, n).astype(np.float32) for _ in range(3))
    prog = Program((("sel", 3, 0, 1, 2),), n_inputs=3, result=3)
    bufs = {"p": np.where(p > 0, p, 0).astype(np.float32), "q": q, "r": r,
            "y": np.full(n + 3, 9.0, np.float32)}
    op = Op("program", Ref("y", 1), (Ref("p"), Ref("q"), Ref("r")), n=n, prog=prog)
    out = oracle.run(wl_of(bufs, [op]))
    y = out["y"]
    assert y[0] == 9.0 and y[-1] == 9.0 and y[-2] == 9.0
    assert np.array_equal(y[1:n + 1], np.where(bufs["p"] != 0, q, r))
    assert traffic.op_bytes(op) == 4 * n * 4
