"""CPU oracle for queues of small tensor ops.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this
module: it is used by ``tests/``, by ``__graft_entry__.smoke()`` to check the
GPU result and by ``bench.py`` to time the CPU baseline.  It shares no code,
constant or helper with the HIP runtime; both read the same seeded
:class:`persistent_fusion_amd.workloads.Workload`.

What it computes.  The method ("GPUOS: A GPU Operating System Primitive for
Transparent Operation Fusion", section "The Paper") only removes launch
overhead: the result of a queue of small ops is the result of running the ops
one after another in submission order.  The oracle is that definition written
out: one op at a time, in order, every output written (also the ones the
runtime may keep in registers), no fusion.  Fusion itself ("Launch Overhead and
Fusion", section "Fusion") must not change the result; the pins in
``tests/test_oracle_pins.py`` check this interpreter against an independent
per-element evaluator.

Per-op definitions (where the pages are silent, the plainest reading is
taken: no FMA contraction, RELU maps -0 and NaN to +0, denormals kept,
round-to-nearest-even narrowing to bf16):

* fp32 ADD / MUL / SCALE are single IEEE operations rounded to nearest even
  (numpy float32 arithmetic, no fused multiply-add); RELU is
  ``x > 0 ? x : +0``; bf16 operands are widened exactly to fp32 and every bf16
  result is the fp32 result rounded to bf16 with round-to-nearest-even.
* EXP, ROW_SUM, ROW_SOFTMAX, RMSNORM, GEMV, ATTN_SCORE, ATTN_AV, SILU_MUL are
  evaluated in fp64 and rounded once to fp32 (then to bf16 for bf16 outputs).
* ROPE is the rotate-half rotation evaluated in fp32 with each product and each
  sum rounded, as written: ``y_i = x_i c_i - x_{i+h/2} s_i``,
  ``y_{i+h/2} = x_{i+h/2} c_i + x_i s_i``.
* A data operand whose readable length is shorter than the op's extent is read
  cyclically (index ``k mod len``); a longer one is read as a prefix.
* fp16 operands are widened exactly to fp32 and every fp16 result is the fp32
  result rounded to fp16 with round-to-nearest-even (numpy's float32 ->
  float16 conversion, which is that IEEE rounding).
* int32 ADD and MUL are two's-complement and wrap modulo 2^32 (the exact
  integer result reduced mod 2^32); int32 RELU is ``x > 0 ? x : 0``.
* An elementwise op with a view (the generic tensor abstraction of arbitrary
  shapes, strides and broadcasting in "GPUOS: A GPU Operating System
  Primitive for Transparent Operation Fusion", section "The Paper") applies
  the same per-element definition at every index (i0, .., i{d-1}) of its
  shape, reading operand k at element ``sum_j i_j * stride[k][j]`` from the
  operand's start and writing the output there; all inputs are read before
  the output is written.
* A PROGRAM op (an operator defined while the persistent kernel runs:
  runtime operator injection in "GPUOS: A GPU Operating System Primitive for
  Transparent Operation Fusion", section "The Paper") runs its register
  program at every element, one instruction at a time: registers r0..r7 hold
  fp32 values (the op's inputs widened exactly in r0..n_inputs-1, +0 in the
  rest), r8..r15 the program's constants; each instruction stores one fp32
  result rounded to nearest even (division too; no fused multiply-add); MIN
  and MAX return NaN for a NaN operand and order -0 below +0 (IEEE 754-2019
  minimum / maximum); EXP is exp evaluated in fp64 and rounded to fp32.  The
  result register is rounded once to the op's dtype.  A program with EXP is
  in the tolerance class, with |result| as the error scale; otherwise exact.

``run`` also returns, for every element written by a reduction or a
transcendental, the error scale the tolerance test uses: the sum of absolute
values of the terms for sums and dot products, ``|result|`` otherwise.

Accumulation type.  ``acc="f64"`` (the default, and the oracle's definition)
evaluates the tolerance-class ops as stated above.  ``acc="f32"`` evaluates
the same formulas with fp32 accumulation instead (numpy float32 sums, float32
BLAS products, float32 exp) and rounds the same way: a second implementation
inside the same tolerance, which lets a test measure how far two correct
evaluations of a long dependent chain drift apart through rounding alone.

Weight matrices.  A GEMV widens its bf16 weight matrix to fp64 on every call.
``run`` and ``local_check`` keep the widened matrix (and its absolute values,
for the error scale) of a GEMV whose weights sit in a buffer that no op of
the workload writes, and reuse it for every later GEMV over the same
weights.  The arithmetic is unchanged: the cached arrays are exactly the ones
the GEMV would compute again.
"""

from __future__ import annotations

from typing import Dict, List, Optional, Tuple

import numpy as np

from persistent_fusion_amd.workloads import Op, Ref, Workload

EXACT_KINDS = frozenset({"nop", "spin", "copy", "gather", "add", "mul", "scale", "relu", "rope"})
TOL_KINDS = frozenset({"exp", "row_sum", "row_softmax", "rmsnorm", "gemv", "attn_score",
                       "attn_av", "silu_mul"})


class OracleError(RuntimeError):
    """An op the definition rejects (for example a GATHER index out of range)."""


# ----------------------------------------------------------------------------
# bf16 <-> fp32, written from the format's definition: bf16 is the top half of
# an IEEE binary32 word.  Narrowing rounds to nearest, ties to even; NaN stays
# a quiet NaN with its sign.


def bf16_to_f32(u: np.ndarray) -> np.ndarray:
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    upper = bits >> np.uint64(16)
    lower = bits & np.uint64(0xFFFF)
    half = np.uint64(0x8000)
    round_up = (lower > half) | ((lower == half) & ((upper & np.uint64(1)) == np.uint64(1)))
    out = upper + round_up.astype(np.uint64)
    is_nan = np.isnan(np.asarray(x, dtype=np.float32))
    out = np.where(is_nan, upper | np.uint64(0x0040), out)
    return out.astype(np.uint16)


def _to_f32(arr: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_to_f32(arr)
    return np.asarray(arr, dtype=np.float32)  # fp16 widens exactly


def _store_from_f32(vals32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16(vals32)
    if dtype == "f16":
        with np.errstate(over="ignore"):
            return np.asarray(vals32, dtype=np.float32).astype(np.float16)
    return np.asarray(vals32, dtype=np.float32)


def _wrap_i32(v: np.ndarray) -> np.ndarray:
    """The exact integer values reduced modulo 2^32, as int32."""
    return (np.asarray(v, dtype=np.int64) & np.int64(0xFFFFFFFF)).astype(np.uint32).view(np.int32)


def _store_from_f64(vals64: np.ndarray, dtype: str) -> np.ndarray:
    with np.errstate(over="ignore", invalid="ignore"):
        vals32 = np.asarray(vals64, dtype=np.float64).astype(np.float32)
    return _store_from_f32(vals32, dtype)


# ----------------------------------------------------------------------------
# operand access


def _elem_count(bufs: Dict[str, np.ndarray], ref: Ref) -> int:
    return bufs[ref.buf].shape[0] - ref.off


def _read_cyclic(bufs: Dict[str, np.ndarray], ref: Ref, src_len: int, extent: int) -> np.ndarray:
    """Elements k mod src_len (k < extent) of the operand starting at ref."""
    if src_len == 0:
        src_len = extent
    if ref.off + src_len > bufs[ref.buf].shape[0]:
        raise OracleError(f"operand {ref} of length {src_len} overruns its buffer")
    base = bufs[ref.buf][ref.off:ref.off + src_len]
    if src_len >= extent:
        return base[:extent].copy()
    reps = -(-extent // src_len)
    return np.tile(base, reps)[:extent].copy()


def _read(bufs: Dict[str, np.ndarray], ref: Ref, count: int) -> np.ndarray:
    if ref.off + count > bufs[ref.buf].shape[0]:
        raise OracleError(f"operand {ref} of length {count} overruns its buffer")
    return bufs[ref.buf][ref.off:ref.off + count].copy()


def _write(bufs: Dict[str, np.ndarray], ref: Ref, vals: np.ndarray) -> None:
    dst = bufs[ref.buf]
    if ref.off + vals.shape[0] > dst.shape[0]:
        raise OracleError(f"output {ref} of length {vals.shape[0]} overruns its buffer")
    dst[ref.off:ref.off + vals.shape[0]] = vals.astype(dst.dtype, copy=False)


# ----------------------------------------------------------------------------
# elementwise values


def _acc_type(acc: str):
    if acc not in ("f64", "f32"):
        raise ValueError(f"accumulation type {acc!r}")
    return np.float64 if acc == "f64" else np.float32


def _ew_values(k: str, dt: str, alpha: float, xr: np.ndarray, yr: Optional[np.ndarray],
               acc: str = "f64"):
    """Stored values of elementwise op ``k`` on raw operands xr (and yr), and
    the error scale (None for the exact class)."""
    if dt == "i32":
        x = np.asarray(xr, dtype=np.int64)
        if k == "add":
            return _wrap_i32(x + np.asarray(yr, dtype=np.int64)), None
        if k == "mul":
            return _wrap_i32(x * np.asarray(yr, dtype=np.int64)), None
        if k == "relu":
            return np.where(x > 0, x, 0).astype(np.int32), None
        raise OracleError(f"{k} is not defined for int32")
    x = _to_f32(xr, dt)
    y = _to_f32(yr, dt) if yr is not None else None
    if k == "add":
        r32 = x + y
    elif k == "mul":
        r32 = x * y
    elif k == "scale":
        r32 = np.float32(alpha) * x
    elif k == "relu":
        r32 = np.where(x > np.float32(0.0), x, np.float32(0.0)).astype(np.float32)
    elif k == "exp":
        F = _acc_type(acc)
        with np.errstate(over="ignore"):
            r64 = np.exp(x.astype(F))
        return _store_from_f64(r64, dt), np.abs(r64.astype(np.float64))
    else:  # silu_mul: g / (1 + exp(-g)) * u in fp64
        F = _acc_type(acc)
        g = x.astype(F)
        u = y.astype(F)
        with np.errstate(over="ignore", invalid="ignore"):
            r64 = g / (F(1.0) + np.exp(-g)) * u
        return _store_from_f64(r64, dt), np.abs(r64.astype(np.float64))
    return _store_from_f32(r32.astype(np.float32), dt), None


def _bits(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)


def _from_bits(u: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(u, dtype=np.uint32).view(np.float32)


def _p_min(a: np.ndarray, b: np.ndarray, smaller: bool) -> np.ndarray:
    """IEEE 754-2019 minimum (smaller=True) / maximum: NaN if either operand
    is NaN; of two equal values (+0 and -0 included) minimum takes the one
    with the sign bit set, maximum the one without."""
    lt, gt = (a < b, a > b) if smaller else (a > b, a < b)
    eq_bits = (_bits(a) | _bits(b)) if smaller else (_bits(a) & _bits(b))
    r = np.where(lt, a, np.where(gt, b, _from_bits(eq_bits)))
    return np.where(np.isnan(a) | np.isnan(b), np.float32(np.nan), r).astype(np.float32)


def _program_values(prog, dt: str, raws):
    """Stored values of a PROGRAM op on its raw inputs, and the error scale
    (None unless the program uses EXP)."""
    n = raws[0].shape[0]
    regs = [np.zeros(n, np.float32) for _ in range(8)]
    for j, r in enumerate(raws):
        regs[j] = _to_f32(r, dt).astype(np.float32)
    consts = [np.float32(c) for c in prog.consts] + [np.float32(0.0)] * (8 - len(prog.consts))

    def reg(i: int) -> np.ndarray:
        return regs[i] if i < 8 else np.full(n, consts[i - 8], np.float32)

    uses_exp = False
    with np.errstate(all="ignore"):
        for ins in prog.insns:
            name, dst, src = ins[0], ins[1], ins[2:]
            a = reg(src[0])
            b = reg(src[1]) if len(src) > 1 else None
            c = reg(src[2]) if len(src) > 2 else None
            if name == "mov":
                y = a.copy()
            elif name == "add":
                y = a + b
            elif name == "sub":
                y = a - b
            elif name == "mul":
                y = a * b
            elif name == "div":
                y = a / b
            elif name == "min":
                y = _p_min(a, b, True)
            elif name == "max":
                y = _p_min(a, b, False)
            elif name == "neg":
                y = _from_bits(_bits(a) ^ np.uint32(0x80000000))
            elif name == "abs":
                y = _from_bits(_bits(a) & np.uint32(0x7FFFFFFF))
            elif name == "relu":
                y = np.where(a > np.float32(0.0), a, np.float32(0.0))
            elif name == "exp":
                y = np.exp(a.astype(np.float64)).astype(np.float32)
                uses_exp = True
            elif name == "lt":
                y = np.where(a < b, np.float32(1.0), np.float32(0.0))
            elif name == "sel":
                y = np.where(a != np.float32(0.0), b, c)
            else:
                raise OracleError(f"unknown program instruction {name}")
            regs[dst] = np.asarray(y, dtype=np.float32)
    res = reg(prog.result)
    return _store_from_f32(res, dt), (np.abs(res.astype(np.float64)) if uses_exp else None)


def view_offsets(shape, strides) -> np.ndarray:
    """Element offsets sum_j i_j * strides[j] of every index of ``shape``, in
    row-major index order."""
    idx = np.indices(tuple(shape), dtype=np.int64).reshape(len(shape), -1)
    return (idx * np.asarray(strides, dtype=np.int64)[:, None]).sum(axis=0)


def _apply_view(op: Op, bufs: Dict[str, np.ndarray]) -> Optional[np.ndarray]:
    """An elementwise op over a view: op.view = (shape, out strides, in0
    strides, in1 strides)."""
    shape, so, s0, s1 = op.view
    k = op.kind
    if k not in ("copy", "add", "mul", "scale", "relu", "exp", "silu_mul"):
        raise OracleError(f"views are not defined for {k}")
    if int(np.prod(shape)) != op.n:
        raise OracleError("view extents do not multiply to n")

    def gather(ref: Ref, strides) -> np.ndarray:
        off = ref.off + view_offsets(shape, strides)
        if off.size and off.max() >= bufs[ref.buf].shape[0]:
            raise OracleError(f"view of {ref} overruns its buffer")
        return bufs[ref.buf][off].copy()

    xr = gather(op.ins[0], s0)
    if k == "copy":
        vals, scale = xr, None
    else:
        yr = gather(op.ins[1], s1) if k in ("add", "mul", "silu_mul") else None
        vals, scale = _ew_values(k, op.dtype, op.alpha, xr, yr)
    out_off = op.out.off + view_offsets(shape, so)
    dst = bufs[op.out.buf]
    if out_off.size and out_off.max() >= dst.shape[0]:
        raise OracleError("view output overruns its buffer")
    if np.unique(out_off).size != out_off.size:
        raise OracleError("view output addresses an element twice")
    dst[out_off] = vals.astype(dst.dtype, copy=False)
    return scale


# ----------------------------------------------------------------------------
# one op


def out_len(op: Op) -> int:
    """Number of elements an op writes."""
    if op.kind in ("nop", "spin"):
        return 0
    if op.kind == "row_sum":
        return op.rows
    return op.n


def out_positions(op: Op) -> np.ndarray:
    """Element indices (in the output buffer) an op writes, in the order of
    its results."""
    if getattr(op, "view", None) is not None:
        return op.out.off + view_offsets(op.view[0], op.view[1])
    return np.arange(op.out.off, op.out.off + out_len(op), dtype=np.int64)


class WeightCache:
    """Widened weight matrices of GEMVs over buffers that no op writes
    (``frozen``): (buffer, offset, M, K) -> (W, |W|) in fp64."""

    def __init__(self, frozen):
        self.frozen = frozenset(frozen)
        self.mats: Dict[tuple, Tuple[np.ndarray, np.ndarray]] = {}

    @staticmethod
    def for_workload(wl: Workload) -> "WeightCache":
        written = {op.out.buf for op in wl.ops}
        return WeightCache(set(wl.buffers) - written)


def _gemv_weights(bufs: Dict[str, np.ndarray], ref: Ref, M: int, K: int,
                  cache: Optional[WeightCache], acc: str = "f64") -> Tuple[np.ndarray, np.ndarray]:
    key = (ref.buf, ref.off, M, K, acc)
    if cache is not None and key in cache.mats:
        return cache.mats[key]
    W = bf16_to_f32(_read(bufs, ref, M * K)).astype(_acc_type(acc)).reshape(M, K)
    absW = np.abs(W)
    if cache is not None and ref.buf in cache.frozen:
        cache.mats[key] = (W, absW)
    return W, absW


def apply_op(op: Op, bufs: Dict[str, np.ndarray], dtypes: Dict[str, str],
             wcache: Optional[WeightCache] = None, acc: str = "f64") -> Optional[np.ndarray]:
    """Executes one op on ``bufs`` in place.

    Returns the error-scale array of the elements written (tolerance class),
    or None for ops whose result is exact.  ``wcache`` (optional) keeps the
    widened weights of GEMVs over buffers no op writes; ``acc`` is the
    accumulation type of the tolerance-class ops (see the module docstring).
    """
    k = op.kind
    dt = op.dtype
    n = op.n
    F = _acc_type(acc)
    if k in ("nop", "spin"):
        return None

    if getattr(op, "view", None) is not None:
        return _apply_view(op, bufs)

    if k == "copy":
        _write(bufs, op.out, _read_cyclic(bufs, op.ins[0], op.src_len[0], n))
        return None

    if k == "gather":
        idx = _read(bufs, op.aux, n).astype(np.int64)
        src_n = op.src_len[0] or _elem_count(bufs, op.ins[0])
        if np.any(idx < 0) or np.any(idx >= src_n):
            raise OracleError("gather index out of range")
        src = _read(bufs, op.ins[0], src_n)
        _write(bufs, op.out, src[idx])
        return None

    if k == "program":
        if len(op.ins) != op.prog.n_inputs:
            raise OracleError("program op with a wrong number of inputs")
        vals, scale = _program_values(op.prog, dt, [_read(bufs, r, n) for r in op.ins])
        _write(bufs, op.out, vals)
        return scale

    if k in ("add", "mul", "scale", "relu", "exp", "silu_mul"):
        xr = _read_cyclic(bufs, op.ins[0], op.src_len[0], n)
        yr = _read_cyclic(bufs, op.ins[1], op.src_len[1], n) if k in ("add", "mul", "silu_mul") else None
        vals, scale = _ew_values(k, dt, op.alpha, xr, yr, acc)
        _write(bufs, op.out, vals)
        return scale

    if k in ("row_sum", "row_softmax", "rmsnorm"):
        rows, L = op.rows, op.row_len
        if rows * L != n:
            raise OracleError("row op with n != rows * row_len")
        x64 = _to_f32(_read_cyclic(bufs, op.ins[0], op.src_len[0], n), dt).astype(F)
        x64 = x64.reshape(rows, L)
        if k == "row_sum":
            s = x64.sum(axis=1)
            _write(bufs, op.out, _store_from_f64(s, dt))
            return np.abs(x64.astype(np.float64)).sum(axis=1)
        if k == "row_softmax":
            m = x64.max(axis=1, keepdims=True)  # NaN propagates through max
            with np.errstate(invalid="ignore", over="ignore"):
                e = np.exp(x64 - m)
                y = e / e.sum(axis=1, keepdims=True)
            _write(bufs, op.out, _store_from_f64(y.reshape(-1), dt))
            return np.abs(y.astype(np.float64)).reshape(-1)
        g = _to_f32(_read(bufs, op.aux, L), dt).astype(F)
        ms = (x64 * x64).sum(axis=1) / F(L)
        inv = F(1.0) / np.sqrt(ms + F(np.float32(op.eps)))
        y = x64 * inv[:, None] * g[None, :]
        _write(bufs, op.out, _store_from_f64(y.reshape(-1), dt))
        return np.abs(y.astype(np.float64)).reshape(-1)

    if k == "rope":
        heads, hd = op.rows, op.row_len
        if heads * hd != n or hd % 2:
            raise OracleError("rope needs n = heads * head_dim with an even head_dim")
        half = hd // 2
        x = _to_f32(_read(bufs, op.ins[0], n), dt).reshape(heads, hd)
        tab = _read(bufs, op.aux, hd).astype(np.float32)
        c, s = tab[:half], tab[half:]
        x1, x2 = x[:, :half], x[:, half:]
        y1 = (x1 * c) - (x2 * s)
        y2 = (x2 * c) + (x1 * s)
        y = np.concatenate([y1, y2], axis=1).astype(np.float32).reshape(-1)
        _write(bufs, op.out, _store_from_f32(y, dt))
        return None

    if k == "gemv":
        M, K = op.dims[0], op.dims[1]
        if M != n:
            raise OracleError("gemv needs n == M")
        W, absW = _gemv_weights(bufs, op.aux, M, K, wcache, acc)
        x = _to_f32(_read(bufs, op.ins[0], K), dt).astype(F)
        y = W @ x
        _write(bufs, op.out, _store_from_f64(y, dt))
        return (absW @ np.abs(x)).astype(np.float64)

    if k == "attn_score":
        H, Dh, S = op.dims[0], op.dims[1], op.dims[2]
        if H * S != n:
            raise OracleError("attn_score needs n == H * S")
        q = _to_f32(_read(bufs, op.ins[0], H * Dh), dt).astype(F).reshape(H, Dh)
        Kc = bf16_to_f32(_read(bufs, op.aux, S * H * Dh)).astype(F).reshape(S, H, Dh)
        a = F(np.float32(op.alpha))
        sc = np.empty((H, S), F)
        scale = np.empty((H, S))
        for h in range(H):
            sc[h] = a * (Kc[:, h, :] @ q[h])
            scale[h] = abs(a) * (np.abs(Kc[:, h, :]) @ np.abs(q[h]))
        _write(bufs, op.out, _store_from_f64(sc.reshape(-1), "f32"))
        return scale.reshape(-1)

    if k == "attn_av":
        H, Dh, S = op.dims[0], op.dims[1], op.dims[2]
        if H * Dh != n:
            raise OracleError("attn_av needs n == H * D")
        p = _read(bufs, op.ins[0], H * S).astype(F).reshape(H, S)
        Vc = bf16_to_f32(_read(bufs, op.aux, S * H * Dh)).astype(F).reshape(S, H, Dh)
        o = np.empty((H, Dh), F)
        scale = np.empty((H, Dh))
        for h in range(H):
            o[h] = Vc[:, h, :].T @ p[h]
            scale[h] = np.abs(Vc[:, h, :]).T @ np.abs(p[h])
        _write(bufs, op.out, _store_from_f64(o.reshape(-1), dt))
        return scale.reshape(-1)

    raise OracleError(f"unknown op kind {k!r}")


# ----------------------------------------------------------------------------
# a whole queue


def run(wl: Workload, upto: Optional[int] = None, scales: bool = False,
        buffers: Optional[Dict[str, np.ndarray]] = None, start: int = 0,
        wcache: Optional[WeightCache] = None, acc: str = "f64"):
    """Runs ops [start, upto) of the workload in submission order, from the
    workload's initial buffers or from ``buffers`` (the state after ops
    [0, start), for a run taken in pieces).

    Returns the final buffers (copies; the workload is not modified).  With
    ``scales=True`` also returns ``{buffer: scale array or None}``: for every
    buffer, an fp64 array of error scales where the last writer of an element
    in the run was a tolerance-class op, NaN where it was an exact op or the
    initial contents.  ``wcache`` (optional) carries widened weights from one
    piece of a run to the next.  ``acc`` is the accumulation type of the
    tolerance-class ops ("f64", the definition, or "f32"; see the module
    docstring).
    """
    bufs = {k: v.copy() for k, v in (buffers or wl.buffers).items()}
    sc: Dict[str, np.ndarray] = {}
    ops = wl.ops[start:] if upto is None else wl.ops[start:upto]
    cache = wcache if wcache is not None else WeightCache.for_workload(wl)
    for op in ops:
        s = apply_op(op, bufs, wl.dtypes, cache, acc)
        if not scales or op.kind in ("nop", "spin"):
            continue
        name = op.out.buf
        if name not in sc:
            sc[name] = np.full(bufs[name].shape[0], np.nan)
        sc[name][out_positions(op)] = np.nan if s is None else s
    if scales:
        return bufs, sc
    return bufs


def local_check(wl: Workload, gpu: Dict[str, np.ndarray], compare_fn, only=None):
    """Checks each op on the GPU's own inputs.

    Requires a workload in which every element is written at most once (its
    verification form), so the GPU's final buffers hold every op's output.
    The state before op i is the initial buffers with the GPU outputs of ops
    0..i-1 written into their ranges; op i is re-run by the oracle on that
    state and its output compared with the GPU's.  With ``only`` (a set of op
    indices) just those ops are re-run; the others only advance the state.
    Returns a list of (op index, buffer, Mismatch) for every op whose output
    differs.
    """
    state = {k: v.copy() for k, v in wl.buffers.items()}
    bad = []
    cache = WeightCache.for_workload(wl)
    for i, op in enumerate(wl.ops):
        if out_len(op) == 0:
            continue
        name, pos = op.out.buf, out_positions(op)
        if only is not None and i not in only:
            state[name][pos] = gpu[name][pos]
            continue
        s = apply_op(op, state, wl.dtypes, cache)
        want = state[name][pos].copy()
        got = gpu[name][pos]
        r = compare_fn(got, want, wl.dtypes[name], s)
        if not r.ok:
            bad.append((i, name, r))
        state[name][pos] = got
    return bad
