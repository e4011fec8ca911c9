"""Compiled program bodies, host half (no GPU).

gpuos_program_compile on a host-only context writes the bodies as code and
builds the kernel variant with hipRTC for gfx950 (hipRTC runs on the CPU);
nothing is loaded, and flushes only count the hand-overs between the two
kernels.  These tests check the generated code (operand order, constants
as exact bits), which descriptors carry a compiled body, where the queue
changes kernels, and the errors.  The device results are compared with the
oracle in the GPU tests.
"""

import ctypes as C

import pytest

from persistent_fusion_amd import gpuos
from persistent_fusion_amd.gpuos import Context, DEVICE_NONE, GpuosError, decode_desc, make_op
from persistent_fusion_amd.workloads import Program

BASE = 0x7F0000000000
MB = 1 << 26


def buf(i):
    return BASE + i * MB


# a body the fused tile cannot express (so it is not lowered with fusion on)
CLAMP = Program((("sub", 3, 0, 1), ("div", 4, 3, 8), ("max", 5, 4, 9), ("min", 5, 5, 10),
                 ("sel", 6, 0, 5, 1)), 2, 6, consts=(3.0, -0.5, 0.5))
SQ = Program((("mul", 3, 0, 0), ("lt", 4, 3, 1), ("neg", 4, 4)), 2, 4)


@pytest.fixture(scope="module")
def compiled():
    """One host-only context with CLAMP and SQ compiled (one hipRTC build)."""
    c = Context(DEVICE_NONE, ring_slots=1024, fusion=2)
    pc = c.program_define(gpuos.program_of(CLAMP))
    ps = c.program_define(gpuos.program_of(SQ))
    log = c.program_compile()
    yield c, pc, ps, log
    c.destroy()


def test_generated_code_keeps_operand_order_and_constant_bits(compiled):
    c, _, _, _ = compiled
    src = c.rtc_source()
    body0 = src[src.index("struct RtcBody0"):src.index("struct RtcBody1")]
    lines = [l.strip() for l in body0.splitlines() if l.strip().startswith(("r", "return"))]
    assert lines == [
        "r3 = r0 - r1;",
        "r4 = r3 / pvec(__uint_as_float(0x40400000u));",          # 3.0
        "r5 = pv_max(r4, pvec(__uint_as_float(0xbf000000u)));",   # -0.5
        "r5 = pv_min(r5, pvec(__uint_as_float(0x3f000000u)));",   # 0.5
        "r6 = pv_sel(r0, r5, r1);",
        "return r6;",
    ]
    body1 = src[src.index("struct RtcBody1"):]
    assert "r3 = r0 * r0;" in body1 and "r4 = pv_lt(r3, r1);" in body1 and "r4 = pv_neg(r4);" in body1
    assert "#define GPUOS_RTC_BODIES(X) X(0) X(1)" in src
    assert "#define GPUOS_RTC_DTYPES 0x" in src


def _prog_op(pid, out, a, b, n=4096, dtype="f32"):
    return make_op("program", out, [a, b], n=n, dtype=dtype, dims=(pid,))


def test_descriptors_carry_bodies_and_the_queue_changes_kernels(compiled):
    c, pc, ps, _ = compiled
    st0 = c.stats()
    ops = (gpuos.GpuosOp * 3)(
        _prog_op(pc, buf(2), buf(0), buf(1)),
        make_op("add", buf(3), [buf(2), buf(1)], n=4096),
        _prog_op(ps, buf(4), buf(3), buf(0)),
    )
    c.submit(ops)
    c.flush()
    s0 = c.published(0) - 2
    bodies = [decode_desc(c.read_desc(0, s0 + k))["pg"]["body"] for k in (0, 2)]
    assert bodies == [1, 2]
    st = c.stats()
    # one hand-over to the variant: everything in the flush can run there
    assert st["kernel_switches"] - st0["kernel_switches"] == 1
    assert st["programs_compiled"] - st0["programs_compiled"] == 2

    # a bf16 op sends the queue back; the program after it returns to the variant
    ops = (gpuos.GpuosOp * 2)(
        make_op("relu", buf(5), [buf(6)], n=4096, dtype="bf16"),
        _prog_op(pc, buf(7), buf(0), buf(1)),
    )
    c.submit(ops)
    c.flush()
    assert c.stats()["kernel_switches"] - st["kernel_switches"] == 2

    # a program whose body changed after the compile has no compiled body:
    # the variant cannot run it, so the queue goes back to the built-in kernel
    st = c.stats()
    upd = Program((("add", 3, 0, 1),) + CLAMP.insns[1:], 2, 6, consts=CLAMP.consts)
    c.program_update(pc, gpuos.program_of(upd))
    c.submit(_prog_op(pc, buf(8), buf(0), buf(1)))
    c.flush()
    assert decode_desc(c.read_desc(0, c.published(0)))["pg"]["body"] == 0
    st2 = c.stats()
    assert st2["kernel_switches"] - st["kernel_switches"] == 1
    assert st2["programs_compiled"] == st["programs_compiled"]
    c.program_update(pc, gpuos.program_of(CLAMP))  # restore for the other tests


def test_a_flush_with_an_op_the_variant_cannot_run_stays_built_in(compiled):
    c, pc, _, _ = compiled
    # the previous test ended on the built-in kernel
    st = c.stats()
    ops = (gpuos.GpuosOp * 2)(
        _prog_op(pc, buf(2), buf(0), buf(1)),
        make_op("row_sum", buf(9), [buf(10)], n=64 * 256, rows=64, row_len=256),
    )
    c.submit(ops)
    c.flush()
    st2 = c.stats()
    assert st2["kernel_switches"] == st["kernel_switches"]
    assert st2["programs_compiled"] - st["programs_compiled"] == 1  # carries the body, interpreted here


def test_dtype_mask_limits_the_compiled_bodies():
    c = Context(DEVICE_NONE, ring_slots=1024, fusion=2)
    try:
        pid = c.program_define(gpuos.program_of(SQ))
        c.program_compile(dtypes=["f32"])
        assert "#define GPUOS_RTC_DTYPES 0x1u" in c.rtc_source()
        c.submit((gpuos.GpuosOp * 2)(_prog_op(pid, buf(1), buf(0), buf(2)),
                                     _prog_op(pid, buf(3), buf(4), buf(5), dtype="bf16")))
        c.flush()
        last = c.published(0)
        assert decode_desc(c.read_desc(0, last - 1))["pg"]["body"] == 1
        assert decode_desc(c.read_desc(0, last))["pg"]["body"] == 0
    finally:
        c.destroy()


def test_compile_errors():
    L = gpuos.lib()
    c = Context(DEVICE_NONE, ring_slots=1024)
    try:
        with pytest.raises(GpuosError, match="EINVAL"):
            c.program_compile()                     # nothing defined
        pid = c.program_define(gpuos.program_of(SQ))
        with pytest.raises(GpuosError, match="EINVAL"):
            c.program_compile(ids=[pid + 1])        # unknown id
        log = C.create_string_buffer(64)
        rc = L.gpuos_program_compile(c.handle, None, 0, 1 << 5, log, len(log))  # not a float dtype
        assert rc == gpuos.EINVAL
        assert L.gpuos_program_compile(None, None, 0, 0, None, 0) == gpuos.EINVAL
        c.stop()
        with pytest.raises(GpuosError, match="ESTATE"):
            c.program_compile()
    finally:
        c.destroy()
