"""ctypes binding of the gpuos C ABI (``include/gpuos.h``).

Argument marshalling only: every op runs in the HIP kernels of ``libgpuos.so``.
Device buffers come from the caller (typically torch tensors, passed by
``data_ptr()``); torch does no compute on this path.  Importing this module
fails loudly when the native library has not been built.
"""

from __future__ import annotations

import ctypes as C
import os
from typing import Callable, Dict, Iterable, List, Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgpuos.so")
ABI_VERSION = 9  # GPUOS_ABI_VERSION of the header this binding follows

# status codes
OK, EINVAL, ENOMEM, EAGAIN, ETIMEDOUT, EDEVICE, ESTATE, ECOMPILE = 0, -1, -2, -3, -4, -5, -6, -7
STATUS_NAMES = {0: "OK", -1: "EINVAL", -2: "ENOMEM", -3: "EAGAIN", -4: "ETIMEDOUT",
                -5: "EDEVICE", -6: "ESTATE", -7: "ECOMPILE"}

OPCODES = {
    "nop": 0, "copy": 1, "gather": 2, "add": 3, "mul": 4, "scale": 5, "relu": 6, "exp": 7,
    "row_sum": 8, "row_softmax": 9, "rmsnorm": 10, "rope": 11, "gemv": 12,
    "attn_score": 13, "attn_av": 14, "silu_mul": 15, "spin": 16, "program": 17,
}
# instructions of a gpuos_program
POPS = {"mov": 0, "add": 1, "sub": 2, "mul": 3, "div": 4, "min": 5, "max": 6, "neg": 7,
        "abs": 8, "relu": 9, "exp": 10, "lt": 11, "sel": 12}
POP_ARITY = {k: (3 if k == "sel" else 2 if k in ("add", "sub", "mul", "div", "min", "max", "lt") else 1)
             for k in POPS}
PROG_MAX_INSNS = 16
PROG_MAX_PROGRAMS = 4096  # programs per context
DTYPES = {"f32": 0, "bf16": 1, "i32": 2, "f16": 3}
ELEM_BYTES = {"f32": 4, "bf16": 2, "i32": 4}
FLAG_TRANSIENT, FLAG_LC, FLAG_NONTEMPORAL = 0x1, 0x2, 0x4
DEVICE_NONE = -1


class GpuosOp(C.Structure):
    _fields_ = [
        ("opcode", C.c_uint16), ("dtype", C.c_uint8), ("flags", C.c_uint8),
        ("n", C.c_uint32), ("rows", C.c_uint32), ("row_len", C.c_uint32),
        ("out", C.c_void_p), ("in_", C.c_void_p * 3), ("src_len", C.c_uint64 * 2),
        ("alpha", C.c_float), ("beta", C.c_float), ("eps", C.c_float),
        ("aux", C.c_int32 * 4), ("_pad", C.c_int32), ("deps", C.c_int64 * 4),
    ]


class GpuosConfig(C.Structure):
    _fields_ = [(name, C.c_uint32) for name in (
        "ring_slots", "waves_per_cu", "tile_elems", "be_tile_elems", "fusion", "auto_deps",
        "trace", "block_on_full", "max_fuse", "priority", "idle_exit_ms", "stream_min_kib",
        "lc_waves", "tile_counts", "jitter", "reserved")]


class GpuosStats(C.Structure):
    _fields_ = [(name, C.c_uint64) for name in (
        "ops_submitted", "ops_fused", "descs_published", "descs_completed", "flushes",
        "ring_full_waits", "deps_explicit", "deps_auto", "device_error", "error_desc",
        "worker_waves", "compute_units", "kernel_ns", "launches", "lc_waves", "programs_lowered",
        "programs_compiled", "kernel_switches")]


class GpuosTraceRec(C.Structure):
    _fields_ = [("seq", C.c_uint64), ("t_claim", C.c_uint64), ("t_done", C.c_uint64),
                ("opcode", C.c_uint32), ("ntiles", C.c_uint32), ("ring", C.c_uint32),
                ("first_ops", C.c_uint32), ("t_wait", C.c_uint64), ("t_end", C.c_uint64),
                ("t_ack", C.c_uint64)]


class GpuosView(C.Structure):
    _fields_ = [("ndim", C.c_uint32), ("_reserved", C.c_uint32), ("shape", C.c_uint64 * 4),
                ("stride", (C.c_int64 * 4) * 3)]


class GpuosInsn(C.Structure):
    _fields_ = [("op", C.c_uint8), ("dst", C.c_uint8), ("a", C.c_uint8), ("b", C.c_uint8),
                ("c", C.c_uint8), ("_reserved", C.c_uint8 * 3)]


class GpuosProgram(C.Structure):
    _fields_ = [("n_insns", C.c_uint32), ("n_inputs", C.c_uint32), ("result", C.c_uint32),
                ("_reserved", C.c_uint32), ("consts", C.c_float * 8),
                ("insns", GpuosInsn * 16)]


assert C.sizeof(GpuosInsn) == 8
assert C.sizeof(GpuosProgram) == 176
assert C.sizeof(GpuosView) == 136
assert C.sizeof(GpuosOp) == 128
assert C.sizeof(GpuosConfig) == 64
assert C.sizeof(GpuosStats) == 144
assert C.sizeof(GpuosTraceRec) == 64

# Every symbol declared in include/gpuos.h and include/gpuos_debug.h.
EXPORTS = (
    "gpuos_abi_version", "gpuos_last_error", "gpuos_config_default", "gpuos_create",
    "gpuos_submit", "gpuos_flush", "gpuos_submit_flush", "gpuos_sync", "gpuos_query", "gpuos_get_stats",
    "gpuos_trace_read", "gpuos_stop", "gpuos_destroy", "gpuos_baseline_run", "gpuos_submit_views",
    "gpuos_graph_create", "gpuos_graph_launch", "gpuos_graph_destroy", "gpuos_yield",
    "gpuos_launch_overhead",
    "gpuos_program_define", "gpuos_program_update", "gpuos_program_compile",
    "gpuos_debug_read_desc", "gpuos_debug_published", "gpuos_debug_seq_of", "gpuos_debug_retire",
    "gpuos_debug_tile_counts", "gpuos_create_static", "gpuos_debug_rtc_source",
    "gpuos_debug_consumer_attach", "gpuos_debug_consumer_tail", "gpuos_debug_consumer_read",
    "gpuos_debug_consumer_retire",
)

_lib = None


def lib() -> C.CDLL:
    """Loads libgpuos.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"native library {LIB_PATH} is missing: run __graft_entry__.build() first")
    L = C.CDLL(LIB_PATH)
    P = C.c_void_p
    sig = {
        "gpuos_abi_version": (C.c_int, []),
        "gpuos_last_error": (C.c_char_p, []),
        "gpuos_config_default": (None, [C.POINTER(GpuosConfig)]),
        "gpuos_create": (C.c_int, [C.c_int, C.POINTER(GpuosConfig), C.POINTER(P)]),
        "gpuos_create_static": (C.c_int, [C.c_int, C.POINTER(GpuosConfig), P, C.c_size_t, C.POINTER(P)]),
        "gpuos_submit": (C.c_int, [P, C.POINTER(GpuosOp), C.c_uint32, C.POINTER(C.c_uint64)]),
        "gpuos_submit_views": (C.c_int, [P, C.POINTER(GpuosOp), C.POINTER(GpuosView), C.c_uint32,
                                         C.POINTER(C.c_uint64)]),
        "gpuos_flush": (C.c_int, [P]),
        "gpuos_submit_flush": (C.c_int, [P, C.POINTER(GpuosOp), C.c_uint32, C.POINTER(C.c_uint64)]),
        "gpuos_sync": (C.c_int, [P, C.c_uint64, C.c_int64]),
        "gpuos_query": (C.c_int, [P, C.c_uint64]),
        "gpuos_get_stats": (C.c_int, [P, C.POINTER(GpuosStats)]),
        "gpuos_trace_read": (C.c_int, [P, C.POINTER(GpuosTraceRec), C.c_uint32, C.POINTER(C.c_uint32)]),
        "gpuos_stop": (C.c_int, [P, C.c_int64]),
        "gpuos_yield": (C.c_int, [P, C.c_int64]),
        "gpuos_program_define": (C.c_int, [P, C.POINTER(GpuosProgram), C.POINTER(C.c_uint32)]),
        "gpuos_program_update": (C.c_int, [P, C.c_uint32, C.POINTER(GpuosProgram)]),
        "gpuos_program_compile": (C.c_int, [P, C.POINTER(C.c_uint32), C.c_uint32, C.c_uint32,
                                            C.c_char_p, C.c_size_t]),
        "gpuos_destroy": (C.c_int, [P, C.c_int64]),
        "gpuos_baseline_run": (C.c_int, [C.c_int, C.POINTER(GpuosOp), C.c_uint32, C.c_int, P]),
        "gpuos_graph_create": (C.c_int, [C.c_int, C.POINTER(GpuosOp), C.c_uint32, C.c_int, C.POINTER(P)]),
        "gpuos_graph_launch": (C.c_int, [P, P]),
        "gpuos_graph_destroy": (C.c_int, [P]),
        "gpuos_launch_overhead": (C.c_int, [C.c_int, C.c_uint32, C.POINTER(C.c_double), C.POINTER(C.c_double)]),
        "gpuos_debug_read_desc": (C.c_int, [P, C.c_int, C.c_uint64, P]),
        "gpuos_debug_published": (C.c_uint64, [P, C.c_int]),
        "gpuos_debug_seq_of": (C.c_int, [P, C.c_uint64, C.POINTER(C.c_int), C.POINTER(C.c_uint64)]),
        "gpuos_debug_retire": (C.c_int, [P, C.c_int, C.c_uint64]),
        "gpuos_debug_consumer_attach": (C.c_int, [P]),
        "gpuos_debug_consumer_tail": (C.c_uint64, [P, C.c_int]),
        "gpuos_debug_consumer_read": (C.c_int, [P, C.c_int, C.c_uint64, P]),
        "gpuos_debug_consumer_retire": (C.c_int, [P, C.c_int, C.c_uint64]),
        "gpuos_debug_tile_counts": (C.c_int, [P, C.c_int, C.POINTER(C.c_uint32), C.c_uint32]),
        "gpuos_debug_rtc_source": (C.c_size_t, [P, C.c_char_p, C.c_size_t]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


class GpuosError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = lib().gpuos_last_error().decode(errors="replace")
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def _check(rc: int, where: str) -> int:
    if rc < 0:
        raise GpuosError(rc, where)
    return rc


def config(**kw) -> GpuosConfig:
    """A config with the given fields set and every other field zero, which
    selects the library's default (or a GPUOS_<FIELD> environment override)."""
    cfg = GpuosConfig()
    for k, v in kw.items():
        if not hasattr(cfg, k):
            raise TypeError(f"unknown config field {k}")
        setattr(cfg, k, int(v))
    return cfg


def make_op(kind: str, out: int, ins: Sequence[int] = (), aux: int = 0, n: int = 0,
            dtype: str = "f32", rows: int = 0, row_len: int = 0, src_len=(0, 0),
            alpha: float = 0.0, eps: float = 0.0, dims: Sequence[int] = (),
            deps: Sequence[int] = (), flags: int = 0) -> GpuosOp:
    """Fills one gpuos_op from raw device addresses."""
    o = GpuosOp()
    o.opcode = OPCODES[kind]
    o.dtype = DTYPES[dtype]
    o.flags = flags
    o.n, o.rows, o.row_len = n, rows, row_len
    o.out = out or None
    for i, p in enumerate(ins):
        o.in_[i] = p or None
    o.in_[2] = aux or None
    o.src_len[0], o.src_len[1] = int(src_len[0]), int(src_len[1])
    o.alpha, o.eps = alpha, eps
    for i, v in enumerate(dims):
        o.aux[i] = int(v)
    for i, v in enumerate(deps):
        o.deps[i] = int(v)
    return o


def encode_ops(ops, start: int, end: int, addr: Callable, id_of: Dict[int, int],
               prog_ids: Optional[Dict] = None):
    """Encodes workload ops [start, end) as a gpuos_op array.

    ``addr(ref, dtype)`` returns the device address of a workload ``Ref``;
    ``id_of`` maps earlier op indices to the ids gpuos_submit returned.  A
    dependency inside [start, end) becomes a relative one (negative), an
    earlier one an absolute id.  ``prog_ids`` maps the ``Program`` of each
    program op to its id in the context (``define_programs``).
    """
    arr = (GpuosOp * (end - start))()
    for k, i in enumerate(range(start, end)):
        op = ops[i]
        deps = []
        for d in op.deps:
            deps.append(-(i - d) if d >= start else id_of[d])
        if len(deps) > 4:
            raise ValueError("at most 4 explicit dependencies")
        in_dt = "f32" if op.kind == "attn_av" else op.dtype
        aux_dt = {"rmsnorm": op.dtype, "rope": "f32", "gather": "i32"}.get(op.kind, "bf16")
        out_dt = "f32" if op.kind == "attn_score" else op.dtype
        flags = (FLAG_TRANSIENT if op.transient else 0) | (FLAG_LC if op.lc else 0)
        if op.kind == "program":  # up to three data inputs; in[2] is one of them
            ins = [addr(r, op.dtype) for r in op.ins]
            arr[k] = make_op("program", addr(op.out, op.dtype), ins[:2], ins[2] if len(ins) > 2 else 0,
                             n=op.n, dtype=op.dtype, dims=(prog_ids[op.prog],), deps=deps,
                             flags=flags)
            continue
        arr[k] = make_op(op.kind, addr(op.out, out_dt), [addr(r, in_dt) for r in op.ins],
                         addr(op.aux, aux_dt) if op.aux is not None else 0, n=op.n,
                         dtype=op.dtype, rows=op.rows, row_len=op.row_len, src_len=op.src_len,
                         alpha=op.alpha, eps=op.eps, dims=op.dims, deps=deps, flags=flags)
    return arr


def make_program(insns: Sequence[Sequence], n_inputs: int, result: int,
                 consts: Sequence[float] = ()) -> GpuosProgram:
    """A gpuos_program from (op name, dst, *sources) tuples, e.g.
    ``[("mul", 3, 0, 1), ("add", 3, 3, 2), ("relu", 3, 3)]``."""
    p = GpuosProgram()
    p.n_insns, p.n_inputs, p.result = len(insns), n_inputs, result
    for j, v in enumerate(consts):
        p.consts[j] = float(v)
    for s, ins in enumerate(insns):
        op, dst, *src = ins
        p.insns[s].op, p.insns[s].dst = POPS[op], dst
        for j, r in enumerate(src):
            setattr(p.insns[s], "abc"[j], r)
    return p


def program_of(prog) -> GpuosProgram:
    """The gpuos_program of a workload ``Program``."""
    return make_program(prog.insns, prog.n_inputs, prog.result, prog.consts)


def define_programs(ctx: "Context", ops) -> Dict:
    """Defines every distinct ``Program`` of the program ops in ``ops`` on
    the context, in order of first use; returns Program -> id."""
    ids: Dict = {}
    for op in ops:
        if op.kind == "program" and op.prog not in ids:
            ids[op.prog] = ctx.program_define(program_of(op.prog))
    return ids


def make_view(shape: Sequence[int], strides: Sequence[Sequence[int]]) -> GpuosView:
    """A gpuos_view: shape (outermost first) and element strides of out, in0,
    in1 (a missing operand's strides are 0)."""
    v = GpuosView()
    v.ndim = len(shape)
    for d, e in enumerate(shape):
        v.shape[d] = int(e)
    for k, st in enumerate(strides):
        for d, x in enumerate(st):
            v.stride[k][d] = int(x)
    return v


def encode_views(ops, start: int, end: int):
    """GpuosView array for workload ops [start, end), or None if no op there
    has a view (``Op.view`` = (shape, out strides, in0 strides, in1 strides))."""
    if not any(getattr(ops[i], "view", None) for i in range(start, end)):
        return None
    arr = (GpuosView * (end - start))()
    for k, i in enumerate(range(start, end)):
        v = getattr(ops[i], "view", None)
        if v:
            arr[k] = make_view(v[0], v[1:])
    return arr


STATIC_MAX_SLOTS = 4096  # GPUOS_STATIC_MAX_SLOTS


def static_host_bytes(slots: int) -> int:
    """GPUOS_STATIC_HOST_BYTES(slots): the pinned workspace a static context needs."""
    return 768 + 2 * (slots * 256 + (slots * 8 + 255) // 256 * 256) + (slots * 8 + 255) // 256 * 256


class Context:
    """One resident-kernel context (``gpuos_create`` ... ``gpuos_destroy``).
    With ``host_ws`` (the address of a pinned workspace of ``host_ws_bytes``
    bytes) the context is made by ``gpuos_create_static`` instead."""

    def __init__(self, device: int = 0, host_ws: Optional[int] = None, host_ws_bytes: int = 0, **cfg):
        self._lib = lib()
        self._cfg = config(**cfg)
        h = C.c_void_p()
        if host_ws is None:
            _check(self._lib.gpuos_create(device, C.byref(self._cfg), C.byref(h)), "gpuos_create")
        else:
            _check(self._lib.gpuos_create_static(device, C.byref(self._cfg), host_ws, host_ws_bytes,
                                                 C.byref(h)), "gpuos_create_static")
        self.handle = h
        self.device = device
        self._submit = self._lib.gpuos_submit
        self._submit_flush = self._lib.gpuos_submit_flush
        self._query = self._lib.gpuos_query
        self._id1 = (C.c_uint64 * 1)()

    def submit(self, ops, n: Optional[int] = None, views=None, flush: bool = False) -> List[int]:
        """Submits ops (and, optionally, a GpuosView array: gpuos_submit_views);
        with flush, also flushes in the same call (gpuos_submit_flush)."""
        if isinstance(ops, GpuosOp):
            ops = (GpuosOp * 1)(ops)
        n = len(ops) if n is None else n
        if n == 1 and views is None:  # one op: no per-call id array
            rc = (self._submit_flush if flush else self._submit)(self.handle, ops, 1, self._id1)
            if rc < 0:
                raise GpuosError(rc, "gpuos_submit_flush" if flush else "gpuos_submit")
            return [self._id1[0]]
        if flush and views is None:
            ids = (C.c_uint64 * max(n, 1))()
            _check(self._submit_flush(self.handle, ops, n, ids), "gpuos_submit_flush")
            return list(ids[:n])
        ids = (C.c_uint64 * max(n, 1))()
        if views is not None:
            _check(self._lib.gpuos_submit_views(self.handle, ops, views, n, ids), "gpuos_submit_views")
        else:
            _check(self._lib.gpuos_submit(self.handle, ops, n, ids), "gpuos_submit")
        if flush:
            self.flush()
        return list(ids[:n])

    def submit_noids(self, ops, n: int) -> None:
        _check(self._lib.gpuos_submit(self.handle, ops, n, None), "gpuos_submit")

    def flush(self) -> None:
        _check(self._lib.gpuos_flush(self.handle), "gpuos_flush")

    def sync(self, upto: int = 0, timeout_s: float = -1.0) -> None:
        t = -1 if timeout_s < 0 else int(timeout_s * 1e9)
        _check(self._lib.gpuos_sync(self.handle, upto, t), "gpuos_sync")

    def query(self, op_id: int) -> bool:
        rc = self._query(self.handle, op_id)
        if rc < 0:
            raise GpuosError(rc, "gpuos_query")
        return rc == 1

    def stats(self) -> dict:
        s = GpuosStats()
        _check(self._lib.gpuos_get_stats(self.handle, C.byref(s)), "gpuos_get_stats")
        return {name: getattr(s, name) for name, _ in GpuosStats._fields_ if name != "reserved"}

    def trace(self, max_records: int = 1 << 16) -> List[dict]:
        buf = (GpuosTraceRec * max_records)()
        n = C.c_uint32()
        _check(self._lib.gpuos_trace_read(self.handle, buf, max_records, C.byref(n)), "gpuos_trace_read")
        return [{k: getattr(buf[i], k) for k, _ in GpuosTraceRec._fields_} for i in range(n.value)]

    def read_desc(self, ring: int, seq: int) -> bytes:
        out = C.create_string_buffer(256)
        _check(self._lib.gpuos_debug_read_desc(self.handle, ring, seq, out), "gpuos_debug_read_desc")
        return out.raw

    def published(self, ring: int = 0) -> int:
        return self._lib.gpuos_debug_published(self.handle, ring)

    def seq_of(self, op_id: int):
        r, s = C.c_int(), C.c_uint64()
        _check(self._lib.gpuos_debug_seq_of(self.handle, op_id, C.byref(r), C.byref(s)), "gpuos_debug_seq_of")
        return r.value, s.value

    def retire(self, ring: int, upto: int) -> None:
        _check(self._lib.gpuos_debug_retire(self.handle, ring, upto), "gpuos_debug_retire")

    def tile_counts(self, ring: int, n: int) -> List[int]:
        """gpuos_debug_tile_counts: executions of tickets [0, n) of `ring`."""
        buf = (C.c_uint32 * max(n, 1))()
        _check(self._lib.gpuos_debug_tile_counts(self.handle, ring, buf, n), "gpuos_debug_tile_counts")
        return list(buf[:n])

    def tickets(self, ring: int = 0) -> int:
        """Tickets (tiles) published to `ring` so far: the first ticket after
        its last published descriptor."""
        last = self.published(ring)
        if not last:
            return 0
        d = decode_desc(self.read_desc(ring, last))
        return d["tstart"] + d["ntiles"]

    def program_define(self, prog: GpuosProgram) -> int:
        """gpuos_program_define: returns the program id (aux[0] of PROGRAM ops)."""
        pid = C.c_uint32()
        _check(self._lib.gpuos_program_define(self.handle, C.byref(prog), C.byref(pid)),
               "gpuos_program_define")
        return pid.value

    def program_update(self, pid: int, prog: GpuosProgram) -> None:
        """gpuos_program_update: ops submitted from now on run the new body."""
        _check(self._lib.gpuos_program_update(self.handle, pid, C.byref(prog)), "gpuos_program_update")

    def program_compile(self, ids: Optional[Sequence[int]] = None, dtypes: Sequence[str] = ()) -> str:
        """gpuos_program_compile: builds the kernel variant holding the current
        bodies of programs `ids` (None = all) for `dtypes` (empty = all float
        types); returns the compiler's log."""
        mask = 0
        for dt in dtypes:
            mask |= 1 << DTYPES[dt]
        arr = None if ids is None else (C.c_uint32 * max(1, len(ids)))(*ids)
        buf = C.create_string_buffer(1 << 16)
        rc = self._lib.gpuos_program_compile(self.handle, arr, 0 if ids is None else len(ids), mask,
                                             buf, len(buf))
        log = buf.value.decode(errors="replace")
        if rc < 0:
            raise GpuosError(rc, "gpuos_program_compile" + (f" (log: {log[:2000]})" if log else ""))
        return log

    def rtc_source(self) -> str:
        """The body source written by the last program_compile."""
        n = self._lib.gpuos_debug_rtc_source(self.handle, None, 0)
        buf = C.create_string_buffer(max(1, n))
        self._lib.gpuos_debug_rtc_source(self.handle, buf, len(buf))
        return buf.value.decode()

    def yield_gpu(self, timeout_s: float = 30.0) -> None:
        """gpuos_yield: let the resident kernel leave once the queue is done."""
        _check(self._lib.gpuos_yield(self.handle, int(timeout_s * 1e9)), "gpuos_yield")

    def stop(self, timeout_s: float = 30.0) -> None:
        _check(self._lib.gpuos_stop(self.handle, int(timeout_s * 1e9)), "gpuos_stop")

    def destroy(self, timeout_s: float = 30.0) -> None:
        if self.handle:
            h, self.handle = self.handle, None
            _check(self._lib.gpuos_destroy(h, int(timeout_s * 1e9)), "gpuos_destroy")

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.destroy()
        return False


def launch_overhead(device: int, n: int = 10000):
    """gpuos_launch_overhead: (host us per back-to-back empty-kernel launch,
    us per launch followed by a stream synchronize)."""
    a, s = C.c_double(), C.c_double()
    _check(lib().gpuos_launch_overhead(device, n, C.byref(a), C.byref(s)), "gpuos_launch_overhead")
    return a.value, s.value


def baseline_run(device: int, ops, n: Optional[int] = None, fuse: bool = False,
                 stream: int = 0) -> None:
    """One kernel launch per op (or per fused chain) on `stream` (0 = default)."""
    n = len(ops) if n is None else n
    _check(lib().gpuos_baseline_run(device, ops, n, 1 if fuse else 0, stream or None),
           "gpuos_baseline_run")


class Graph:
    """The per-op launches of a fixed op list, captured once as a HIP graph.

    ``launch`` replays every launch with one submission on `stream`; the
    buffers the ops name must stay allocated while the graph exists.
    """

    def __init__(self, device: int, ops, n: Optional[int] = None, fuse: bool = False):
        n = len(ops) if n is None else n
        h = C.c_void_p()
        _check(lib().gpuos_graph_create(device, ops, n, 1 if fuse else 0, C.byref(h)),
               "gpuos_graph_create")
        self.handle = h

    def launch(self, stream: int = 0) -> None:
        _check(lib().gpuos_graph_launch(self.handle, stream or None), "gpuos_graph_launch")

    def destroy(self) -> None:
        if self.handle:
            h, self.handle = self.handle, None
            _check(lib().gpuos_graph_destroy(h), "gpuos_graph_destroy")

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.destroy()
        return False


def decode_desc(raw: bytes) -> dict:
    """Splits a 256-byte device descriptor into named fields (debug/tests)."""
    import struct
    w = struct.unpack("<64I", raw)
    q = lambda i: w[i] | (w[i + 1] << 32)
    d = {
        "opcode": w[0] & 0xFF, "dtype": (w[0] >> 8) & 0xFF, "flags": (w[0] >> 16) & 0xFF,
        "nsteps": w[0] >> 24, "n": w[1], "rows": w[2], "row_len": w[3], "seq": q(4),
        "ntiles": w[6], "tile": w[7],
        "deps": [q(4) - x if x else 0 for x in list(w[8:16]) + list(w[54:60])],
        "wait_retired": q(16), "ptr": [q(18 + 2 * i) for i in range(4)],
        "src_len": [w[26], w[27]], "tstart": q(60), "user_ops": w[62], "check": w[63],
    }
    d["fused_out"] = [q(26 + 2 * s) for s in range(8)]
    d["step_op"] = [(w[42 + s // 4] >> (8 * (s % 4))) & 0xFF for s in range(8)]
    d["step_fl"] = [(w[44 + s // 4] >> (8 * (s % 4))) & 0xFF for s in range(8)]
    d["fscal"] = list(struct.unpack("<8f", raw[46 * 4:54 * 4]))
    d["alpha"] = struct.unpack("<f", raw[28 * 4:29 * 4])[0]
    # RMSNORM -> GEMV (-> SILU_MUL) descriptors
    d["ng"] = {"W": q(18), "out": q(20), "x": q(22), "g": q(24), "h": q(26), "act": q(28),
               "M": w[30], "K": w[31], "eps": struct.unpack("<f", raw[32 * 4:33 * 4])[0],
               "F": w[33], "q": q(34), "k": q(36), "v": q(38), "tabq": q(40), "tabk": q(42),
               "hd": w[44]}
    # GEMV -> residual ADD descriptors
    d["ga"] = {"out": q(18), "x": q(20), "res": q(22), "W": q(24), "res_first": w[26],
               "M": w[30], "K": w[31], "sum": q(32)}
    d["view"] = {"shape": list(w[34:38]), "stride": [list(w[38 + 4 * k:42 + 4 * k]) for k in range(3)]}
    # PROGRAM descriptors
    d["pg"] = {"n_insns": w[26] & 31, "result": (w[26] >> 8) & 15, "n_inputs": (w[26] >> 16) & 3,
               "zero_mask": w[26] >> 24, "ins": list(w[27:43]),
               "consts": list(struct.unpack("<8f", raw[43 * 4:51 * 4])), "body": w[51]}
    return d
