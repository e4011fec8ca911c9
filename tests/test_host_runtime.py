"""Host half of the runtime, exercised without a GPU.

A context created on GPUOS_DEVICE_NONE keeps its rings in ordinary memory and
launches nothing; these tests inspect the descriptors it publishes (fusion
pass, hazard dependencies, ticket ranges, ring wraparound and back-pressure)
and the validation errors.  Device pointers here are opaque addresses that are
never dereferenced.
"""

import os
import re

import pytest

from persistent_fusion_amd import gpuos
from persistent_fusion_amd.gpuos import Context, DEVICE_NONE, GpuosError, decode_desc, make_op

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BASE = 0x7F0000000000
MB = 1 << 26


def buf(i):
    """Opaque device address number i (64 MiB apart)."""
    return BASE + i * MB


def ctx(**kw):
    kw.setdefault("ring_slots", 1024)
    return Context(DEVICE_NONE, **kw)


def desc(c, seq, ring=0):
    return decode_desc(c.read_desc(ring, seq))


def test_library_exports_every_declared_symbol():
    declared = set()
    for h in ("gpuos.h", "gpuos_debug.h"):
        text = open(os.path.join(ROOT, "include", h)).read()
        declared |= set(re.findall(r"^(?:int|void|uint64_t|size_t|const char\*)\s+(gpuos_[a-z_]+)\(",
                                   text, re.M))
    lib = gpuos.lib()
    missing = [s for s in sorted(declared) if not hasattr(lib, s)]
    assert not missing, missing
    assert set(gpuos.EXPORTS) == declared
    assert lib.gpuos_abi_version() == 9 == gpuos.ABI_VERSION


def test_fused_chain_becomes_one_descriptor():
    n = 1 << 20
    a, x, b, t1, t2, y = (buf(i) for i in range(6))
    ops = (gpuos.GpuosOp * 3)(
        make_op("mul", t1, [a, x], n=n, flags=gpuos.FLAG_TRANSIENT),
        make_op("add", t2, [t1, b], n=n, flags=gpuos.FLAG_TRANSIENT, deps=[-1]),
        make_op("relu", y, [t2], n=n, deps=[-1]),
    )
    with ctx() as c:
        ids = c.submit(ops)
        assert ids == [1, 2, 3]
        c.flush()
        assert c.published(0) == 1
        d = desc(c, 1)
        assert d["opcode"] == 32 and d["nsteps"] == 3 and d["user_ops"] == 3
        assert d["ptr"][0] == a  # chain input
        assert d["step_op"][:3] == [2, 1, 4]  # MUL, ADD, RELU
        # operands: x as fused input 1, b as fused input 2; only y is stored
        assert d["ptr"][1] == x and d["ptr"][2] == b
        assert [(f >> 4) & 3 for f in d["step_fl"][:3]] == [1, 2, 0]
        assert [bool(f & 4) for f in d["step_fl"][:3]] == [False, False, True]
        assert d["fused_out"][:3] == [0, 0, y]
        assert d["deps"] == [0] * 14
        assert d["ntiles"] * d["tile"] >= n and d["tstart"] == 0
        assert all(c.seq_of(i) == (0, 1) for i in ids)
        assert c.stats()["ops_fused"] == 2


def test_fusion_off_and_transient_output_read_later_is_kept():
    n = 4096
    a, x, b, t1, t2, y, z = (buf(i) for i in range(7))
    ops = (gpuos.GpuosOp * 4)(
        make_op("mul", t1, [a, x], n=n, flags=gpuos.FLAG_TRANSIENT),
        make_op("add", t2, [t1, b], n=n, flags=gpuos.FLAG_TRANSIENT),
        make_op("relu", y, [t2], n=n),
        make_op("copy", z, [t1], n=n),  # reads the transient t1 after the chain
    )
    with ctx(fusion=2) as c:
        c.submit(ops)
        c.flush()
        assert c.published(0) == 4
        assert [desc(c, s)["opcode"] for s in (1, 2, 3, 4)] == [4, 3, 6, 1]
        # auto deps: add waits for mul, relu for add, copy for mul
        assert desc(c, 2)["deps"][0] == 1 and desc(c, 3)["deps"][0] == 2
        assert desc(c, 4)["deps"][0] == 1
    with ctx() as c:
        c.submit(ops)
        c.flush()
        assert c.published(0) == 2  # chain of 3, then the copy
        d = desc(c, 1)
        assert d["fused_out"][:3] == [t1, 0, y]
        assert desc(c, 2)["deps"][0] == 1


def test_fusion_rejects_unsafe_chains():
    n = 4096
    p = [buf(i) for i in range(8)]
    with ctx() as c:
        # second op's other operand is the first op's own output at another
        # offset: the chain must not be fused
        ops = (gpuos.GpuosOp * 2)(
            make_op("add", p[2], [p[0], p[1]], n=n),
            make_op("mul", p[3], [p[2], p[2] + 64], n=n),
        )
        c.submit(ops)
        c.flush()
        assert c.published(0) == 2
    with ctx() as c:
        # different n: not fused
        ops = (gpuos.GpuosOp * 2)(
            make_op("add", p[2], [p[0], p[1]], n=n),
            make_op("relu", p[3], [p[2]], n=n // 2),
        )
        c.submit(ops)
        c.flush()
        assert c.published(0) == 2
    with ctx() as c:
        # in place chain x = relu(x * x) fuses (same base, loads before stores)
        ops = (gpuos.GpuosOp * 2)(
            make_op("mul", p[0], [p[0], p[0]], n=n),
            make_op("relu", p[0], [p[0]], n=n),
        )
        c.submit(ops)
        c.flush()
        assert c.published(0) == 1
        d = desc(c, 1)
        assert d["step_fl"][0] & 2  # FSF_SELF
        assert d["fused_out"][:2] == [p[0], p[0]]


def test_hazard_dependencies_raw_war_waw():
    n = 1024
    A, B, C_, D = (buf(i) for i in range(4))
    ops = (gpuos.GpuosOp * 4)(
        make_op("relu", B, [A], n=n),          # 1: reads A, writes B
        make_op("exp", C_, [A], n=n),          # 2: reads A, writes C
        make_op("scale", A, [D], n=n, alpha=2.0),  # 3: writes A (WAR on 1, 2)
        make_op("exp", B, [C_], n=n),          # 4: RAW on 2, WAW on 1
    )
    with ctx(fusion=2) as c:
        c.submit(ops)
        c.flush()
        deps = [sorted(x for x in desc(c, s)["deps"] if x) for s in (1, 2, 3, 4)]
        assert deps == [[], [], [1, 2], [1, 2]]
    with ctx(fusion=2, auto_deps=2) as c:
        c.submit(ops)
        c.flush()
        assert all(desc(c, s)["deps"] == [0] * 14 for s in (1, 2, 3, 4))


def test_partial_overlap_is_a_hazard_and_disjoint_is_not():
    A = buf(0)
    ops = (gpuos.GpuosOp * 3)(
        make_op("relu", A, [buf(1)], n=1000),            # writes A[0:1000]
        make_op("relu", A + 4000, [buf(2)], n=1000),     # writes A[1000:2000], disjoint
        make_op("exp", buf(3), [A + 3996], n=2),          # reads A[999:1001]: both
    )
    with ctx(fusion=2) as c:
        c.submit(ops)
        c.flush()
        assert desc(c, 2)["deps"] == [0] * 14
        assert sorted(x for x in desc(c, 3)["deps"] if x) == [1, 2]


def test_many_dependencies_fall_back_to_retire_order():
    # 14 readers fit in the descriptor; 15 fall back to the retire cursor
    n = 256
    for readers, fallback in ((14, False), (15, True)):
        ops = (gpuos.GpuosOp * (readers + 1))(
            *[make_op("relu", buf(10 + i), [buf(0)], n=n) for i in range(readers)],
            make_op("scale", buf(0), [buf(1)], n=n, alpha=1.0))
        with ctx(fusion=2) as c:
            c.submit(ops)
            c.flush()
            d = desc(c, readers + 1)
            if fallback:
                assert d["deps"] == [0] * 14 and d["wait_retired"] == readers
            else:
                assert sorted(x for x in d["deps"] if x) == list(range(1, readers + 1))
                assert d["wait_retired"] == 0


def test_ticket_ranges_are_contiguous_and_tiles_cover_ops():
    ops = (gpuos.GpuosOp * 5)(
        make_op("add", buf(0), [buf(1), buf(2)], n=10_000),
        make_op("row_softmax", buf(3), [buf(4)], n=14 * 512, rows=14, row_len=512),
        make_op("gemv", buf(5), [buf(6)], aux=buf(7), n=2688, dtype="bf16", dims=(2688, 896)),
        make_op("attn_av", buf(8), [buf(9)], aux=buf(10), n=896, dtype="bf16", dims=(14, 64, 512)),
        make_op("rope", buf(11), [buf(12)], aux=buf(13), n=896, dtype="bf16", rows=14, row_len=64),
    )
    with ctx(fusion=2) as c:
        c.submit(ops)
        c.flush()
        ds = [desc(c, s) for s in range(1, 6)]
        start = 0
        for d in ds:
            assert d["tstart"] == start
            start += d["ntiles"]
        assert ds[0]["ntiles"] * ds[0]["tile"] >= 10_000 and ds[0]["tile"] % 64 == 0
        assert ds[1]["ntiles"] * ds[1]["tile"] >= 14
        assert ds[2]["ntiles"] * ds[2]["tile"] >= 2688
        assert ds[3]["ntiles"] == 896 // 8
        assert ds[4]["ntiles"] == 1


def test_ring_wraparound_and_back_pressure():
    n = 256
    with ctx(fusion=2, auto_deps=2, ring_slots=64) as c:
        ops = (gpuos.GpuosOp * 150)(*[make_op("relu", buf(i % 7), [buf(100)], n=n) for i in range(150)])
        ids = c.submit(ops)
        with pytest.raises(GpuosError) as e:
            c.flush()
        assert e.value.status == gpuos.EAGAIN
        assert c.published(0) == 64
        with pytest.raises(GpuosError):
            c.read_desc(0, 65)
        c.retire(0, 40)
        with pytest.raises(GpuosError):
            c.flush()
        assert c.published(0) == 104
        # slot of seq 1 now holds seq 65
        with pytest.raises(GpuosError):
            c.read_desc(0, 1)
        d = desc(c, 65)
        assert d["seq"] == 65 and d["check"] == (65 ^ 0x9E3779B9)
        c.retire(0, 104)
        c.flush()
        assert c.published(0) == 150
        assert c.seq_of(ids[-1]) == (0, 150)
        c.retire(0, 150)
        assert c.query(ids[-1])


def test_priority_ring_and_cross_ring_rules():
    n = 4096
    with ctx(fusion=2) as c:
        ops = (gpuos.GpuosOp * 3)(
            make_op("add", buf(0), [buf(1), buf(2)], n=n),
            make_op("relu", buf(3), [buf(4)], n=n, dtype="bf16", flags=gpuos.FLAG_LC),
            make_op("scale", buf(5), [buf(3)], n=n, dtype="bf16", flags=gpuos.FLAG_LC, alpha=0.5),
        )
        ids = c.submit(ops)
        c.flush()
        assert c.published(0) == 1 and c.published(1) == 2
        assert c.seq_of(ids[1]) == (1, 1) and c.seq_of(ids[2]) == (1, 2)
        assert desc(c, 2, ring=1)["deps"][0] == 1
        bad = (gpuos.GpuosOp * 2)(
            make_op("add", buf(0), [buf(1), buf(2)], n=n),
            make_op("relu", buf(6), [buf(7)], n=n, flags=gpuos.FLAG_LC, deps=[-1]),
        )
        with pytest.raises(GpuosError) as e:
            c.submit(bad)
        assert e.value.status == gpuos.EINVAL


@pytest.mark.parametrize("op,msg", [
    (lambda: make_op("add", buf(0), [buf(1), 0], n=10), "in[1]"),
    (lambda: make_op("add", buf(0) + 2, [buf(1), buf(2)], n=10), "aligned"),
    (lambda: make_op("relu", buf(0), [buf(1)], n=0), "n must be"),
    (lambda: make_op("row_sum", buf(0), [buf(1)], n=100, rows=3, row_len=33), "rows"),
    (lambda: make_op("row_softmax", buf(0), [buf(1)], n=8192, rows=1, row_len=8192), "4096"),
    (lambda: make_op("gemv", buf(0), [buf(1)], aux=buf(2), n=10, dims=(11, 4)), "GEMV"),
    (lambda: make_op("rope", buf(0), [buf(1)], aux=buf(2), n=21, rows=3, row_len=7), "ROPE"),
    (lambda: make_op("gather", buf(0), [buf(1)], aux=buf(2), n=10), "src_len"),
    (lambda: make_op("exp", buf(0), [buf(1)], n=10, dtype="i32"), "int32"),
    (lambda: make_op("scale", buf(0), [buf(1)], n=10, dtype="i32", alpha=2.0), "int32"),
    (lambda: make_op("gemv", buf(0), [buf(1)], aux=buf(2), n=4, dtype="f16", dims=(4, 8)), "fp16"),
    # in place over a shifted copy of itself, cyclically, or where tiles read
    # beyond the elements they write
    (lambda: make_op("add", buf(0), [buf(0) + 4, buf(1)], n=10), "overlaps"),
    (lambda: make_op("relu", buf(0), [buf(0)], n=10, src_len=(4, 0)), "overlaps"),
    (lambda: make_op("row_sum", buf(0), [buf(0)], n=64, rows=2, row_len=32), "overlaps"),
    (lambda: make_op("gemv", buf(0), [buf(0)], aux=buf(2), n=4, dims=(4, 4)), "overlaps"),
    (lambda: make_op("rmsnorm", buf(0), [buf(1)], aux=buf(0), n=64, rows=2, row_len=32), "overlaps"),
])
def test_validation_errors_stage_nothing(op, msg):
    with ctx() as c:
        good = make_op("relu", buf(5), [buf(6)], n=16)
        arr = (gpuos.GpuosOp * 2)(good, op())
        with pytest.raises(GpuosError) as e:
            c.submit(arr)
        assert e.value.status == gpuos.EINVAL and msg in str(e.value)
        c.flush()
        assert c.published(0) == 0


def test_dependency_on_future_or_outside_ids_is_rejected():
    with ctx() as c:
        arr = (gpuos.GpuosOp * 1)(make_op("relu", buf(0), [buf(1)], n=16, deps=[5]))
        with pytest.raises(GpuosError):
            c.submit(arr)
        arr = (gpuos.GpuosOp * 1)(make_op("relu", buf(0), [buf(1)], n=16, deps=[-1]))
        with pytest.raises(GpuosError):
            c.submit(arr)
        ok = c.submit((gpuos.GpuosOp * 1)(make_op("relu", buf(0), [buf(1)], n=16)))
        arr = (gpuos.GpuosOp * 1)(make_op("exp", buf(2), [buf(3)], n=16, deps=[ok[0]]))
        c.submit(arr)
        c.flush()
        assert desc(c, 2)["deps"][0] == 1


def test_host_only_sync_reports_timeout_and_config_errors():
    with ctx() as c:
        c.submit((gpuos.GpuosOp * 1)(make_op("relu", buf(0), [buf(1)], n=16)))
        with pytest.raises(GpuosError) as e:
            c.sync(0, 0.01)
        assert e.value.status == gpuos.ETIMEDOUT
    for bad in ({"ring_slots": 100}, {"waves_per_cu": 6}, {"tile_elems": 100}, {"max_fuse": 9},
                {"lc_waves": 65}):
        with pytest.raises(GpuosError):
            Context(DEVICE_NONE, **bad)


def test_elementwise_queue_encoding_matches_workload():
    from persistent_fusion_amd.workloads import gen_elementwise_queue

    wl = gen_elementwise_queue(n_ops=50, n=4096)
    names = sorted(wl.buffers)
    base = {k: buf(i) for i, k in enumerate(names)}
    addr = lambda ref, dt: base[ref.buf] + ref.off * 4
    arr = gpuos.encode_ops(wl.ops, 0, 50, addr, {})
    with ctx(fusion=2) as c:
        c.submit(arr)
        c.flush()
        assert c.published(0) == 50
        got = []
        for i, op in enumerate(wl.ops):
            d = desc(c, i + 1)
            assert d["ptr"][0] == base[op.out.buf]
            got.append({x - 1 for x in d["deps"] if x})
    # a published dependency implied by another is dropped: each op keeps a
    # subset of its dependencies with the same transitive closure
    want = [set(op.deps) for op in wl.ops]
    assert all(g <= w for g, w in zip(got, want))
    assert _closure(got) == _closure(want)


def _closure(preds):
    reach = []
    for p in preds:
        r = set(p)
        for j in p:
            r |= reach[j]
        reach.append(r)
    return reach


def test_implied_dependencies_are_dropped():
    # a chain 1 <- 2 <- 3 where 3 also reads 1's output: 3 waits for 2 only;
    # 4 reads 1's and 3's outputs: 3 covers 1
    A, B, C_, D = (buf(i) for i in range(4))
    ops = (gpuos.GpuosOp * 4)(
        make_op("relu", B, [A], n=1024),            # 1
        make_op("exp", C_, [B], n=1024),            # 2: RAW on 1
        make_op("add", D, [C_, B], n=1024),         # 3: RAW on 2 and 1
        make_op("add", A + 8192, [B, D], n=1024),   # 4: RAW on 1 and 3
    )
    with ctx(fusion=2) as c:
        c.submit(ops)
        c.flush()
        deps = [sorted(x for x in desc(c, s)["deps"] if x) for s in (1, 2, 3, 4)]
    assert deps == [[], [1], [2], [3]]
    ops[1].deps[0] = -1                       # explicit: 2 after 1
    ops[2].deps[0], ops[2].deps[1] = -1, -2   # 3 after 2 and after 1
    with ctx(fusion=2, auto_deps=2) as c:     # explicit dependencies are pruned too
        c.submit(ops)
        c.flush()
        deps = [sorted(x for x in desc(c, s)["deps"] if x) for s in (1, 2, 3, 4)]
    assert deps == [[], [1], [2], []]


# ----------------------------------------------------------------------------
# RMSNORM -> GEMV (-> SILU_MUL) fusion


def _norm_gemv_ops(K=896, F=4864, with_gate=True, h_is_x=False, transient_h=False):
    x, g, h, W, gu, act = (buf(i) for i in range(6))
    h = x if h_is_x else h
    M = 2 * F
    ops = [make_op("rmsnorm", h, [x], aux=g, n=K, dtype="bf16", rows=1, row_len=K, eps=1e-6,
                   flags=gpuos.FLAG_TRANSIENT if transient_h else 0),
           make_op("gemv", gu, [h], aux=W, n=M, dtype="bf16", dims=(M, K))]
    if with_gate:
        ops.append(make_op("silu_mul", act, [gu, gu + 2 * F], n=F, dtype="bf16"))
    return (gpuos.GpuosOp * len(ops))(*ops), (x, g, h, W, gu, act)


def test_norm_gemv_gate_fuses_into_one_descriptor():
    ops, (x, g, h, W, gu, act) = _norm_gemv_ops()
    with ctx() as c:
        c.submit(ops)
        c.flush()
        assert c.published(0) == 1
        d = desc(c, 1)
        assert d["opcode"] == 33 and d["user_ops"] == 3
        ng = d["ng"]
        assert (ng["x"], ng["g"], ng["h"], ng["W"], ng["out"], ng["act"]) == (x, g, h, W, gu, act)
        assert (ng["M"], ng["K"], ng["F"]) == (2 * 4864, 896, 4864)
        assert abs(ng["eps"] - 1e-6) < 1e-12
        assert d["n"] == 4864 and d["ntiles"] * d["tile"] >= 4864
        # the weights have no queued writer: the kernel may stream them early
        assert d["flags"] & 0x80


def test_norm_gemv_without_gate_and_refusals():
    ops, _ = _norm_gemv_ops(with_gate=False)
    with ctx() as c:
        c.submit(ops)
        c.flush()
        assert c.published(0) == 1 and desc(c, 1)["user_ops"] == 2
    # a norm written over its own input would race with the other tiles
    ops, _ = _norm_gemv_ops(h_is_x=True)
    with ctx() as c:
        c.submit(ops)
        c.flush()
        assert c.published(0) == 3
    # fusion off: three descriptors
    ops, _ = _norm_gemv_ops()
    with ctx(fusion=2) as c:
        c.submit(ops)
        c.flush()
        assert c.published(0) == 3


def _norm_gemv_rope_ops(H=14, hd=64, copy_off=None, k_out_overlaps_qkv=False):
    D = H * hd
    x, g, h, W, qkv, q, kc, vc, tab = (buf(i) for i in range(9))
    kc = qkv + 2 * D if k_out_overlaps_qkv else kc
    voff = 2 * D if copy_off is None else copy_off
    ops = [make_op("rmsnorm", h, [x], aux=g, n=D, dtype="bf16", rows=1, row_len=D, eps=1e-6),
           make_op("gemv", qkv, [h], aux=W, n=3 * D, dtype="bf16", dims=(3 * D, D)),
           make_op("rope", q, [qkv], aux=tab, n=D, dtype="bf16", rows=H, row_len=hd),
           make_op("rope", kc, [qkv + 2 * D], aux=tab, n=D, dtype="bf16", rows=H, row_len=hd),
           make_op("copy", vc, [qkv + 2 * voff], n=D, dtype="bf16")]
    return (gpuos.GpuosOp * 5)(*ops), (x, g, h, W, qkv, q, kc, vc, tab)


def test_norm_gemv_rotary_fuses_five_ops():
    ops, (x, g, h, W, qkv, q, kc, vc, tab) = _norm_gemv_rope_ops()
    with ctx() as c:
        c.submit(ops)
        c.flush()
        assert c.published(0) == 1
        d = desc(c, 1)
        assert d["opcode"] == 33 and d["user_ops"] == 5
        ng = d["ng"]
        assert (ng["q"], ng["k"], ng["v"], ng["tabq"], ng["tabk"], ng["hd"]) == (q, kc, vc, tab, tab, 64)
        assert (ng["out"], ng["act"], ng["M"], ng["K"]) == (qkv, 0, 3 * 896, 896)
        assert d["n"] == 3 * 896 and d["ntiles"] * d["tile"] >= 3 * 896 // 2


def test_norm_gemv_rotary_refusals():
    # a COPY of the wrong third, or a rotated k written over the GEMV output,
    # leaves the rotary ops unfused (the norm and the GEMV still fuse)
    for kw in (dict(copy_off=0), dict(k_out_overlaps_qkv=True)):
        ops, _ = _norm_gemv_rope_ops(**kw)
        with ctx() as c:
            c.submit(ops)
            c.flush()
            assert c.published(0) == 4, kw
            assert desc(c, 1)["user_ops"] == 2


def test_norm_gemv_drops_unread_transient_norm_output():
    ops, _ = _norm_gemv_ops(transient_h=True)
    with ctx() as c:
        c.submit(ops)
        c.flush()
        assert desc(c, 1)["ng"]["h"] == 0


# ----------------------------------------------------------------------------
# GEMV -> residual ADD fusion


def _gemv_add_ops(M=896, K=4864, res_first=True, z_is=None, src_len=0, dtype="bf16"):
    x, W, y, r, z = (buf(i) for i in range(5))
    z = {None: z, "r": r, "x": x, "y": y}[z_is]
    ins = [r, y] if res_first else [y, r]
    ops = [make_op("gemv", y, [x], aux=W, n=M, dtype=dtype, dims=(M, K)),
           make_op("add", z, ins, n=M, dtype=dtype, src_len=(src_len, 0))]
    return (gpuos.GpuosOp * 2)(*ops), (x, W, y, r, z)


def test_gemv_add_fuses_into_one_descriptor():
    for res_first in (True, False):
        for z_is in (None, "r"):
            ops, (x, W, y, r, z) = _gemv_add_ops(res_first=res_first, z_is=z_is)
            with ctx() as c:
                c.submit(ops)
                c.flush()
                assert c.published(0) == 1
                d = desc(c, 1)
                assert d["opcode"] == 34 and d["user_ops"] == 2 and d["n"] == 896
                ga = d["ga"]
                assert (ga["out"], ga["x"], ga["res"], ga["W"], ga["sum"]) == (y, x, r, W, z)
                assert (ga["M"], ga["K"], ga["res_first"]) == (896, 4864, int(res_first))
                assert d["ntiles"] * d["tile"] >= 896 and d["flags"] & 0x80
    # fp32 works the same way
    ops, _ = _gemv_add_ops(dtype="f32")
    with ctx() as c:
        c.submit(ops)
        c.flush()
        assert c.published(0) == 1 and desc(c, 1)["opcode"] == 34


def test_gemv_add_refusals():
    # the sum written over the GEMV input or output would race with other rows
    for z_is in ("x", "y"):
        ops, _ = _gemv_add_ops(z_is=z_is)
        with ctx() as c:
            c.submit(ops)
            c.flush()
            assert c.published(0) == 2
    # a residual read cyclically stays unfused
    ops, _ = _gemv_add_ops(src_len=448)
    with ctx() as c:
        c.submit(ops)
        c.flush()
        assert c.published(0) == 2
    # fusion off
    ops, _ = _gemv_add_ops()
    with ctx(fusion=2) as c:
        c.submit(ops)
        c.flush()
        assert c.published(0) == 2


# ----------------------------------------------------------------------------
# ROW_SOFTMAX -> ATTN_AV fusion


def _softmax_av_ops(H=14, D=64, S=512, p_is=None, transient=False, out_dtype="bf16"):
    x, p, V, o = (buf(i) for i in range(4))
    p = {None: p, "x": x, "V": V}[p_is]
    ops = [make_op("row_softmax", p, [x], n=H * S, rows=H, row_len=S,
                   flags=gpuos.FLAG_TRANSIENT if transient else 0),
           make_op("attn_av", o, [p], aux=V, n=H * D, dtype=out_dtype, dims=(H, D, S))]
    return (gpuos.GpuosOp * 2)(*ops), (x, p, V, o)


def test_softmax_av_fuses_into_one_descriptor():
    for transient in (False, True):
        ops, (x, p, V, o) = _softmax_av_ops(transient=transient)
        with ctx() as c:
            c.submit(ops)
            c.flush()
            assert c.published(0) == 1
            d = desc(c, 1)
            assert d["opcode"] == 35 and d["user_ops"] == 2
            assert d["ptr"] == [o, 0 if transient else p, x, V]
            assert d["ntiles"] == 14 * 64 // 8 and d["tile"] == 1 and d["n"] == 14 * 64


def test_softmax_av_refusals():
    for kw in (dict(S=516), dict(S=70), dict(D=12), dict(p_is="x")):
        ops, _ = _softmax_av_ops(**kw)
        with ctx() as c:
            c.submit(ops)
            c.flush()
            assert c.published(0) == 2, kw
    ops, _ = _softmax_av_ops()
    with ctx(fusion=2) as c:
        c.submit(ops)
        c.flush()
        assert c.published(0) == 2


# ----------------------------------------------------------------------------
# views (strided and broadcast operands) and the fp16 / int32 dtypes


def _submit_views(c, ops, views):
    arr = (gpuos.GpuosOp * len(ops))(*ops)
    va = (gpuos.GpuosView * len(ops))(*views)
    return c.submit(arr, len(ops), views=va)


def test_views_are_normalised_into_the_descriptor():
    R, Cn = 6, 40
    x, b, y = buf(0), buf(1), buf(2)
    add = make_op("add", y, [x, b], n=R * Cn)
    with ctx() as c:
        # contiguous indexing written as a view is the plain op
        _submit_views(c, [add], [gpuos.make_view((R, Cn), [(Cn, 1), (Cn, 1), (Cn, 1)])])
        # bias add: b broadcast over the rows
        _submit_views(c, [add], [gpuos.make_view((R, Cn), [(Cn, 1), (Cn, 1), (0, 1)])])
        # 3-D with the two inner dimensions contiguous for every operand: merged
        _submit_views(c, [add], [gpuos.make_view((2, 3, Cn * 3 // 3 * R // 6), [(3 * Cn, Cn, 1), (3 * Cn, Cn, 1), (0, Cn, 1)])])
        c.flush()
        assert c.published(0) == 3
        d1, d2, d3 = desc(c, 1), desc(c, 2), desc(c, 3)
        assert not d1["flags"] & 0x40
        assert d2["flags"] & 0x40
        assert d2["view"]["shape"] == [1, 1, R, Cn]
        assert d2["view"]["stride"] == [[0, 0, Cn, 1], [0, 0, Cn, 1], [0, 0, 0, 1]]
        assert d2["ntiles"] * d2["tile"] >= R
        assert d3["view"]["shape"] == [1, 1, 2, 3 * Cn]
        assert d3["view"]["stride"] == [[0, 0, 3 * Cn, 1], [0, 0, 3 * Cn, 1], [0, 0, 0, 1]]


def test_transposed_copies_are_tiled_in_blocks():
    """A COPY whose (batched) 2-D view reads the input down the output's
    columns is flagged 0x20 and tiled per batch into blocks of one 128-byte
    line per input column (32 fp32 or 64 16-bit rows) by 128 columns; other
    ops over the same view, and views whose input rows are not contiguous,
    keep the row tiling."""
    x, y = buf(0), buf(1)
    R, L = 300, 257
    T = [(L, 1), (1, R), (0, 0)]
    with ctx() as c:
        _submit_views(c, [make_op("copy", y, [x], n=R * L)], [gpuos.make_view((R, L), T)])
        _submit_views(c, [make_op("copy", y, [x], n=R * L, dtype="bf16")], [gpuos.make_view((R, L), T)])
        _submit_views(c, [make_op("copy", y, [x], n=3 * R * L)],
                      [gpuos.make_view((3, R, L), [(R * L, L, 1), (R * L, 1, R), (0, 0, 0)])])
        _submit_views(c, [make_op("relu", y, [x], n=R * L)], [gpuos.make_view((R, L), T)])
        _submit_views(c, [make_op("copy", y, [x], n=R * L)], [gpuos.make_view((R, L), [(L, 1), (2, 2 * R), (0, 0)])])
        c.flush()
        assert c.published(0) == 5
        f32, bf16, batched, relu, strided = (desc(c, k) for k in range(1, 6))
        for d, rows_per_block, batches in ((f32, 32, 1), (bf16, 64, 1), (batched, 32, 3)):
            assert d["flags"] & 0x40 and d["flags"] & 0x20
            assert d["tile"] == rows_per_block
            assert d["ntiles"] == batches * -(-R // rows_per_block) * -(-L // 128)
        assert batched["view"]["shape"] == [1, 3, R, L]
        for d in (relu, strided):
            assert d["flags"] & 0x40 and not d["flags"] & 0x20


@pytest.mark.parametrize("view,msg", [
    (((4, 6), [(0, 1), (6, 1), (6, 1)]), "twice"),
    (((4, 6), [(6, 1), (-6, 1), (6, 1)]), "stride"),
    (((4, 5), [(5, 1), (5, 1), (5, 1)]), "multiply"),
    (((4, 6), [(6, 1), (1, 4), (6, 1)]), None),  # a transposed read is fine
])
def test_view_validation(view, msg):
    with ctx() as c:
        op = make_op("add", buf(2), [buf(0), buf(1)], n=24)
        if msg is None:
            _submit_views(c, [op], [gpuos.make_view(*view)])
            return
        with pytest.raises(GpuosError) as e:
            _submit_views(c, [op], [gpuos.make_view(*view)])
        assert e.value.status == gpuos.EINVAL and msg in str(e.value)


def test_view_rejections_for_ops_and_overlaps():
    with ctx() as c:
        # only elementwise ops take views
        g = make_op("gemv", buf(0), [buf(1)], aux=buf(2), n=4, dims=(4, 8))
        with pytest.raises(GpuosError):
            _submit_views(c, [g], [gpuos.make_view((4,), [(1,), (1,), (0,)])])
        # an output overlapping its input under another view would race
        x = buf(0)
        t = make_op("copy", x + 4, [x], n=24)
        with pytest.raises(GpuosError) as e:
            _submit_views(c, [t], [gpuos.make_view((4, 6), [(1, 4), (6, 1), (0, 0)])])
        assert "overlaps" in str(e.value)
        # ... but exactly in place is fine
        r = make_op("relu", x, [x], n=24)
        _submit_views(c, [r], [gpuos.make_view((4, 6), [(12, 2), (12, 2), (0, 0)])])
        # src_len and a view do not mix
        s = make_op("relu", buf(3), [buf(4)], n=24, src_len=(6, 0))
        with pytest.raises(GpuosError):
            _submit_views(c, [s], [gpuos.make_view((4, 6), [(6, 1), (0, 1), (0, 0)])])


def test_view_ranges_drive_hazards_and_views_are_not_fused():
    with ctx() as c:
        x, b, y, z = buf(0), buf(1), buf(2), buf(3)
        # y = x + b (b: 40 elements broadcast over 6 rows), then b is overwritten
        add = make_op("add", y, [x, b], n=240)
        wr = make_op("copy", b, [z], n=40)
        far = make_op("copy", b + 4 * 40, [z], n=40)  # past the broadcast row: no hazard
        arr = (gpuos.GpuosOp * 3)(add, wr, far)
        va = (gpuos.GpuosView * 3)(gpuos.make_view((6, 40), [(40, 1), (40, 1), (0, 1)]),
                                   gpuos.GpuosView(), gpuos.GpuosView())
        c.submit(arr, 3, views=va)
        c.flush()
        assert c.published(0) == 3
        assert desc(c, 2)["deps"][0] == 1
        assert desc(c, 3)["deps"][0] == 0
    # a viewed op next to a fusable fp32 op stays its own descriptor
    with ctx() as c:
        a, b, t, y = buf(0), buf(1), buf(2), buf(3)
        ops = [make_op("mul", t, [a, b], n=64), make_op("relu", y, [t], n=64)]
        views = [gpuos.GpuosView(), gpuos.make_view((8, 8), [(8, 1), (1, 8), (0, 0)])]
        _submit_views(c, ops, views)
        c.flush()
        assert c.published(0) == 2


def test_f16_and_i32_ops_are_accepted_and_not_fused():
    with ctx() as c:
        a, b, t, y = buf(0), buf(1), buf(2), buf(3)
        ops = [make_op("add", t, [a, b], n=64, dtype="f16"), make_op("relu", y, [t], n=64, dtype="f16"),
               make_op("mul", t, [a, b], n=64, dtype="i32"), make_op("relu", y, [t], n=64, dtype="i32"),
               make_op("rmsnorm", y, [a], aux=b, n=64, dtype="f16", rows=1, row_len=64, eps=1e-6)]
        c.submit((gpuos.GpuosOp * 5)(*ops))
        c.flush()
        assert c.published(0) == 5
        assert [desc(c, s)["dtype"] for s in range(1, 6)] == [3, 3, 2, 2, 3]


def test_graph_replay_poisons_only_buffers_written_whole_first():
    """Between graph replays the tests fill outputs with NaN; only buffers
    whose first use is a whole write may be poisoned (a KV cache written at
    one slot and a fed-back hidden state keep their contents)."""
    from persistent_fusion_amd import runner, workloads

    wl = workloads.gen_decode(seed=7, layers=2, tokens=3, distinct=True)
    p = set(runner.poisonable(wl, wl.outputs))
    assert {"K0", "K1", "V0", "V1"}.isdisjoint(p)
    assert {"qkv.0.0", "scores.1.1", "probs.2.0", "act.0.1", "xb.2.1"} <= p
    wl = workloads.gen_decode(seed=7, layers=2, tokens=3)
    assert runner.poisonable(wl, wl.outputs) == []
    wl = workloads.gen_fused_chain(seed=5, n=1000)
    assert runner.poisonable(wl, ["y"]) == ["y"]


def test_exact_in_place_ops_are_accepted():
    with ctx() as c:
        arr = (gpuos.GpuosOp * 4)(
            make_op("add", buf(0), [buf(0), buf(1)], n=10),
            make_op("relu", buf(0), [buf(0)], n=10, src_len=(12, 0)),
            make_op("row_softmax", buf(2), [buf(2)], n=64, rows=2, row_len=32),
            make_op("rope", buf(3), [buf(3)], aux=buf(4), n=64, rows=2, row_len=32),
        )
        c.submit(arr)


# ----------------------------------------------------------------------------
# ops defined at run time (register programs)

P = gpuos.make_program


def _with(p, **fields):
    for k, v in fields.items():
        setattr(p, k, v)
    return p


def _prog_op(pid, n=1000, nin=3, out=0, dtype="f32", **kw):
    ins = [buf(1 + j) for j in range(nin)]
    return make_op("program", buf(out), ins[:2], ins[2] if nin > 2 else 0, n=n, dtype=dtype,
                   dims=(pid,), **kw)


def test_program_define_encodes_the_body_into_the_descriptor():
    with ctx(fusion=2) as c:  # fusion off: no chain is lowered to a built-in descriptor
        p0 = c.program_define(P([("mul", 3, 0, 1), ("add", 3, 3, 2), ("relu", 3, 3)], 3, 3))
        # reads r5 and r6 before writing them: they start at +0 (zero mask)
        p1 = c.program_define(P([("add", 4, 0, 5), ("sel", 7, 4, 6, 9)], 1, 7, consts=(0.0, 2.5)))
        assert (p0, p1) == (0, 1)
        c.submit((gpuos.GpuosOp * 2)(_prog_op(p0), _prog_op(p1, nin=1, out=5)))
        c.flush()
        d0, d1 = desc(c, 1), desc(c, 2)
        assert d0["opcode"] == gpuos.OPCODES["program"] and d0["ntiles"] >= 1
        assert d0["pg"]["n_insns"] == 3 and d0["pg"]["result"] == 3 and d0["pg"]["n_inputs"] == 3
        assert d0["pg"]["zero_mask"] == 0
        assert d0["pg"]["ins"][:3] == [3 | 3 << 5 | 0 << 8 | 1 << 12, 1 | 3 << 5 | 3 << 8 | 2 << 12,
                                       9 | 3 << 5 | 3 << 8]
        assert d0["ptr"][:4] == [buf(0), buf(1), buf(2), buf(3)]
        assert d1["pg"]["zero_mask"] == (1 << 5) | (1 << 6)
        assert d1["pg"]["ins"][1] == 12 | 7 << 5 | 4 << 8 | 6 << 12 | 9 << 16
        assert d1["pg"]["consts"][1] == 2.5


def test_program_update_changes_only_later_ops():
    with ctx(fusion=2) as c:
        pid = c.program_define(P([("add", 3, 0, 1)], 2, 3))
        c.submit((gpuos.GpuosOp * 1)(_prog_op(pid, nin=2)))
        c.program_update(pid, P([("sub", 3, 0, 1), ("neg", 3, 3)], 2, 3))
        c.submit((gpuos.GpuosOp * 1)(_prog_op(pid, nin=2, out=6)))
        c.flush()
        a, b = desc(c, 1)["pg"], desc(c, 2)["pg"]
        assert a["n_insns"] == 1 and a["ins"][0] & 31 == gpuos.POPS["add"]
        assert b["n_insns"] == 2 and b["ins"][0] & 31 == gpuos.POPS["sub"]


@pytest.mark.parametrize("make,msg", [
    (lambda: P([("add", 3, 0, 1)], 0, 3), "n_inputs"),
    (lambda: P([("add", 3, 0, 1)], 4, 3), "n_inputs"),
    (lambda: P([], 1, 0), "n_insns"),
    (lambda: _with(P([("mov", 1, 0)] * 16, 1, 1), n_insns=17), "n_insns"),
    (lambda: P([("mov", 8, 0)], 1, 8), "destination"),
    (lambda: P([("add", 3, 0, 16)], 1, 3), "source register"),
    (lambda: P([("relu", 3, 0, 1)], 1, 3), "unused operand"),
    (lambda: P([("mov", 3, 0)], 1, 16), "result"),
])
def test_program_define_rejects_malformed_bodies(make, msg):
    with ctx() as c:
        with pytest.raises(GpuosError) as e:
            c.program_define(make())
        assert e.value.status == gpuos.EINVAL and msg in str(e.value)
    with ctx() as c:
        p = P([("mov", 3, 0)], 1, 3)
        p.insns[0].op = gpuos.POPS["sel"] + 1  # unknown instruction
        with pytest.raises(GpuosError, match="unknown op"):
            c.program_define(p)
        p = P([("mov", 3, 0)], 1, 3)
        p.insns[5].a = 1  # a slot past n_insns
        with pytest.raises(GpuosError, match="past n_insns"):
            c.program_define(p)
        p = P([("mov", 3, 0)], 1, 3)
        p.insns[0]._reserved[1] = 1
        with pytest.raises(GpuosError, match="reserved"):
            c.program_define(p)
        with pytest.raises(GpuosError, match="unknown program"):
            c.program_update(3, P([("mov", 3, 0)], 1, 3))


def test_program_op_validation():
    with ctx() as c:
        pid = c.program_define(P([("mul", 3, 0, 1)], 2, 3))
        bad = [
            (_prog_op(pid + 1, nin=2), "unknown program"),
            (_prog_op(pid, nin=1), "in[1] must be given"),
            (_prog_op(pid, nin=3), "in[2] must be null"),
            (_prog_op(pid, nin=2, dtype="i32"), "int32 is only for"),
            (_prog_op(pid, nin=2, src_len=(10, 0)), "src_len"),
            (make_op("program", buf(1), [buf(1) + 8, buf(2)], n=100, dims=(pid,)), "overlaps"),
        ]
        for op, msg in bad:
            with pytest.raises(GpuosError) as e:
                c.submit((gpuos.GpuosOp * 1)(op))
            assert e.value.status == gpuos.EINVAL and msg in str(e.value), msg
        with pytest.raises(GpuosError, match="views are only"):
            c.submit((gpuos.GpuosOp * 1)(_prog_op(pid, nin=2, n=6)),
                     views=(gpuos.GpuosView * 1)(gpuos.make_view([2, 3], [[3, 1], [3, 1], [3, 1]])))
        # in place over its own input, element for element, is fine
        c.submit((gpuos.GpuosOp * 1)(make_op("program", buf(1), [buf(1), buf(2)], n=100, dims=(pid,))))
    with pytest.raises(GpuosError, match="only in a context"):
        gpuos.baseline_run(0, (gpuos.GpuosOp * 1)(_prog_op(0, nin=2)), 1)


def test_program_ops_get_hazards_and_are_not_fused():
    with ctx() as c:
        pid = c.program_define(P([("max", 3, 0, 1), ("min", 3, 3, 2)], 3, 3))
        n = 4096
        arr = (gpuos.GpuosOp * 4)(
            make_op("relu", buf(3), [buf(9)], n=n),                 # writes the program's in[2]
            make_op("program", buf(4), [buf(1), buf(2)], buf(3), n=n, dims=(pid,)),
            make_op("relu", buf(5), [buf(4)], n=n),                 # reads the program's output
            make_op("relu", buf(6), [buf(5)], n=n),                 # fuses with the one before
        )
        c.submit(arr)
        c.flush()
        assert c.published(0) == 3
        assert desc(c, 2)["opcode"] == gpuos.OPCODES["program"] and desc(c, 2)["deps"][0] == 1
        assert desc(c, 3)["deps"][0] == 2


def test_yield_and_program_calls_follow_the_context_state():
    with ctx() as c:
        c.yield_gpu()  # nothing resident on a host-only context: returns at once
        pid = c.program_define(P([("mov", 3, 0)], 1, 3))
        c.stop()
        for call in (lambda: c.yield_gpu(), lambda: c.program_define(P([("mov", 3, 0)], 1, 3)),
                     lambda: c.program_update(pid, P([("neg", 3, 0)], 1, 3)),
                     lambda: c.submit((gpuos.GpuosOp * 1)(_prog_op(pid, nin=1)))):
            with pytest.raises(GpuosError) as e:
                call()
            assert e.value.status == gpuos.ESTATE


def test_extent_limits():
    # an operand spans at most 0xFFF00000 bytes, and n is at most 2^30
    with ctx() as c:
        n32 = 0xFFF00000 // 4
        c.submit((gpuos.GpuosOp * 1)(make_op("add", buf(0), [buf(64), buf(128)], n=n32)))
        with pytest.raises(GpuosError, match="spans more than"):
            c.submit((gpuos.GpuosOp * 1)(make_op("add", buf(0), [buf(64), buf(128)], n=n32 + 1)))
        c.submit((gpuos.GpuosOp * 1)(make_op("add", buf(200), [buf(240), buf(280)], n=1 << 30,
                                             dtype="bf16")))
        with pytest.raises(GpuosError, match="2\\^30"):
            c.submit((gpuos.GpuosOp * 1)(make_op("add", buf(200), [buf(240), buf(280)], n=(1 << 30) + 1,
                                                 dtype="bf16")))


def test_chain_programs_lower_to_builtin_descriptors():
    FUSED = 32
    with ctx() as c:
        relu_axb = c.program_define(P([("mul", 3, 0, 1), ("add", 3, 3, 2), ("relu", 3, 3)], 3, 3))
        one_add = c.program_define(P([("add", 3, 1, 0)], 2, 3))            # x1 + x0: commutative
        scale = c.program_define(P([("mul", 4, 8, 0)], 1, 4, consts=(2.5,)))
        square_exp = c.program_define(P([("mul", 3, 0, 0), ("exp", 3, 3)], 1, 3))
        interp = [
            c.program_define(P([("sub", 3, 0, 1)], 2, 3)),                  # no SUB step
            c.program_define(P([("add", 3, 0, 8)], 1, 3, consts=(1.0,))),   # ADD of a constant
            c.program_define(P([("mul", 3, 0, 1), ("add", 4, 0, 1)], 2, 4)),  # the accumulator is dropped
            c.program_define(P([("add", 3, 0, 5)], 1, 3)),                  # reads an unset register
        ]
        ops = [_prog_op(relu_axb, out=0), _prog_op(one_add, nin=2, out=5), _prog_op(scale, nin=1, out=6),
               _prog_op(square_exp, nin=1, out=7)]
        ops += [_prog_op(p, nin=2 if k in (0, 2) else 1, out=8 + k) for k, p in enumerate(interp)]
        ops.append(_prog_op(relu_axb, out=12, dtype="bf16"))                # fp32 only
        c.submit((gpuos.GpuosOp * len(ops))(*ops))
        c.flush()
        d = [desc(c, s) for s in range(1, len(ops) + 1)]
        assert d[0]["opcode"] == FUSED and d[0]["nsteps"] == 3
        assert d[0]["step_op"][:3] == [2, 1, 4]                 # MUL, ADD, RELU
        assert d[0]["ptr"][0] == buf(1)                         # the chain starts from in[0]
        assert d[1]["opcode"] == gpuos.OPCODES["add"] and d[1]["ptr"][1:3] == [buf(2), buf(1)]
        assert d[2]["opcode"] == gpuos.OPCODES["scale"] and d[2]["alpha"] == 2.5
        assert d[3]["opcode"] == FUSED and d[3]["step_fl"][0] & 0x2  # acc * acc
        for k in range(4, len(ops)):
            assert d[k]["opcode"] == gpuos.OPCODES["program"], k
        assert c.stats()["programs_lowered"] == 4
    with ctx(fusion=2) as c:  # fusion off: every program is interpreted
        pid = c.program_define(P([("mul", 3, 0, 1), ("add", 3, 3, 2), ("relu", 3, 3)], 3, 3))
        c.submit((gpuos.GpuosOp * 1)(_prog_op(pid)))
        c.flush()
        assert desc(c, 1)["opcode"] == gpuos.OPCODES["program"]


def test_submit_flush_publishes_in_the_same_call():
    """gpuos_submit_flush: the ids of gpuos_submit, and the ops published as
    by gpuos_flush; a failed submit publishes nothing."""
    with ctx() as c:
        a, b, y = buf(0), buf(1), buf(2)
        ids = c.submit(make_op("add", y, [a, b], n=4096), flush=True)
        assert ids == [1] and c.published(0) == 1
        two = (gpuos.GpuosOp * 2)(make_op("relu", buf(3), [buf(6)], n=4096, flags=gpuos.FLAG_LC),
                                  make_op("mul", buf(4), [a, b], n=4096))
        assert c.submit(two, flush=True) == [2, 3]
        assert c.published(0) == 2 and c.published(1) == 1
        bad = (gpuos.GpuosOp * 1)(make_op("add", buf(5), [a, b], n=0))
        with pytest.raises(GpuosError, match="EINVAL"):
            c.submit(bad, flush=True)
        assert c.published(0) == 2 and c.published(1) == 1


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_overlaps_every_conflict_is_ordered(seed):
    """Random elementwise ops over overlapping sub-ranges of three buffers:
    for every pair of ops whose byte ranges conflict (read after write, write
    after read, write after write), the later op's published dependencies
    order it after the earlier one, directly or through other dependencies
    (or through a wait on the retire cursor).  The hazard map may add orderings,
    never drop one."""
    import random

    rng = random.Random(seed)
    bufs = [buf(i) for i in range(3)]
    ops, ranges = [], []
    while len(ops) < 300:
        n = rng.choice([1, 7, 64, 100, 256, 1000])
        def pick():
            return rng.randrange(3), rng.randrange(0, 2048)
        (bo, oo), (b0, o0), (b1, o1) = pick(), pick(), pick()
        w = (bufs[bo] + 4 * oo, bufs[bo] + 4 * (oo + n))
        r0 = (bufs[b0] + 4 * o0, bufs[b0] + 4 * (o0 + n))
        r1 = (bufs[b1] + 4 * o1, bufs[b1] + 4 * (o1 + n))
        # an output may overlap an input only if it is exactly that input
        if any(r != w and r[0] < w[1] and w[0] < r[1] for r in (r0, r1)):
            continue
        ops.append(make_op("add", w[0], [r0[0], r1[0]], n=n))
        ranges.append((w, (r0, r1)))
    arr = (gpuos.GpuosOp * len(ops))(*ops)
    with ctx(fusion=2) as c:
        c.submit(arr)
        c.flush()
        assert c.published(0) == len(ops)
        preds = []
        for i in range(len(ops)):
            d = desc(c, i + 1)
            # decode_desc gives each dependency as its sequence number; with
            # fusion off, op k is sequence k + 1
            p = {dep - 1 for dep in d["deps"] if dep}
            if d["wait_retired"]:
                p |= set(range(d["wait_retired"]))
            preds.append(p)
    # transitive closure, in order
    reach = []
    for i in range(len(ops)):
        r = set()
        for j in preds[i]:
            r.add(j)
            r |= reach[j]
        reach.append(r)

    def overlap(a, b):
        return a[0] < b[1] and b[0] < a[1]

    for i, (wi, ri) in enumerate(ranges):
        for j in range(i):
            wj, rj = ranges[j]
            conflict = overlap(wi, wj) or any(overlap(r, wj) for r in ri) or any(overlap(wi, r) for r in rj)
            if conflict:
                assert j in reach[i], f"op {i} is not ordered after op {j}"


def test_consumer_calls_on_a_host_only_context():
    """The host-consumer entry points: the tail follows flushes, a slot is read
    only under its own sequence, retiring is bounded by the tail, and with a
    consumer attached a wait that nobody serves times out instead of failing
    at once."""
    lib = gpuos.lib()
    raw = (gpuos.C.c_uint8 * 256)()
    with ctx(ring_slots=64) as c:
        h = c.handle
        assert lib.gpuos_debug_consumer_tail(h, 0) == 0
        c.submit((gpuos.GpuosOp * 2)(make_op("add", buf(2), [buf(0), buf(1)], n=256),
                                     make_op("relu", buf(3), [buf(2)], n=256)))
        assert lib.gpuos_debug_consumer_tail(h, 0) == 0  # staged, not yet published
        c.flush()
        tail = lib.gpuos_debug_consumer_tail(h, 0)
        assert tail == c.published(0) >= 1
        assert lib.gpuos_debug_consumer_read(h, 0, 1, raw) == 0
        assert bytes(raw) == bytes(c.read_desc(0, 1))
        assert lib.gpuos_debug_consumer_read(h, 0, tail + 1, raw) == gpuos.EINVAL
        assert lib.gpuos_debug_consumer_read(h, 2, 1, raw) == gpuos.EINVAL
        assert lib.gpuos_debug_consumer_retire(h, 0, tail + 1) == gpuos.EINVAL
        # without a consumer, a sync on a host-only context fails at once
        with pytest.raises(GpuosError) as e:
            c.sync(0, 5.0)
        assert e.value.status == gpuos.ETIMEDOUT
        assert lib.gpuos_debug_consumer_attach(h) == 0
        with pytest.raises(GpuosError) as e:
            c.sync(0, 0.05)
        assert e.value.status == gpuos.ETIMEDOUT
        assert lib.gpuos_debug_consumer_retire(h, 0, tail) == 0
        c.sync(0, 1.0)


def test_environment_overrides_config_defaults(monkeypatch):
    """GPUOS_<FIELD> replaces a default; the caller's nonzero field wins; a
    malformed or out-of-range value fails the create."""
    op = make_op("relu", buf(1), [buf(0)], n=256)

    def fill(c):
        k = 0
        while True:
            try:
                c.submit((gpuos.GpuosOp * 1)(op))
                c.flush()
            except GpuosError as e:
                assert e.status == gpuos.EAGAIN
                return k
            k += 1

    monkeypatch.setenv("GPUOS_RING_SLOTS", "0x40")
    with Context(DEVICE_NONE) as c:
        assert fill(c) == 64  # the ring holds 64 descriptors, none retire
    with Context(DEVICE_NONE, ring_slots=128) as c:
        assert fill(c) == 128
    monkeypatch.setenv("GPUOS_RING_SLOTS", "48")  # not a power of two
    with pytest.raises(GpuosError, match="ring_slots"):
        Context(DEVICE_NONE)
    monkeypatch.setenv("GPUOS_RING_SLOTS", "64k")
    with pytest.raises(GpuosError, match="GPUOS_RING_SLOTS"):
        Context(DEVICE_NONE)
    monkeypatch.delenv("GPUOS_RING_SLOTS")
    monkeypatch.setenv("GPUOS_FUSION", "3")  # switch fields take 1 or 2
    with pytest.raises(GpuosError, match="switch fields"):
        Context(DEVICE_NONE)
    monkeypatch.setenv("GPUOS_FUSION", "2")
    with Context(DEVICE_NONE) as c:  # fusion off: the chain stays three descriptors
        c.submit((gpuos.GpuosOp * 3)(make_op("mul", buf(2), [buf(0), buf(1)], n=256),
                                     make_op("add", buf(3), [buf(2), buf(1)], n=256),
                                     make_op("relu", buf(4), [buf(3)], n=256)))
        c.flush()
        assert c.published(0) == 3
    monkeypatch.delenv("GPUOS_FUSION")
    with Context(DEVICE_NONE) as c:
        c.submit((gpuos.GpuosOp * 3)(make_op("mul", buf(2), [buf(0), buf(1)], n=256),
                                     make_op("add", buf(3), [buf(2), buf(1)], n=256),
                                     make_op("relu", buf(4), [buf(3)], n=256)))
        c.flush()
        assert c.published(0) == 1
