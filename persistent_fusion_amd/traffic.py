"""Algorithmic HBM byte model for queues of small ops.

Bytes an op stream must move at minimum, used to turn measured times into
effective GB/s and a roofline fraction.  The model is the one "Launch Overhead
and Fusion" uses in its section "Fusion" and in the byte counts its "Code"
section prints: unfused, every op reads each vector operand and writes its
output; fused, a chain reads each distinct external vector once and writes
only the outputs that survive (transient intermediates stay in registers).
Scalars cost nothing.  For y = relu(a*x + b) with scalar a, b this gives 24 vs
8 bytes per fp32 element; with vector a, b it gives 32 vs 16.
"""

from __future__ import annotations

from typing import Iterable, Sequence, Set

from .workloads import ELEM_BYTES, Op

_EW = {"copy", "add", "mul", "scale", "relu", "exp", "silu_mul"}


def op_bytes(op: Op, scalar_bufs: Set[str] = frozenset()) -> int:
    """Bytes one op moves when run on its own."""
    eb = ELEM_BYTES[op.dtype]
    n = op.n
    k = op.kind
    if k in _EW:
        reads = sum(1 for r in op.ins if r.buf not in scalar_bufs)
        return eb * n * (reads + 1)
    if k == "row_sum":
        return eb * (n + op.rows)
    if k == "row_softmax":
        return eb * 2 * n
    if k == "rmsnorm":
        return eb * (2 * n + op.row_len)
    if k == "rope":
        return eb * 2 * n + 4 * op.row_len
    if k == "gemv":
        M, K = op.dims[0], op.dims[1]
        return 2 * M * K + eb * (K + M)
    if k == "attn_score":
        H, D, S = op.dims
        return 2 * S * H * D + eb * H * D + 4 * H * S
    if k == "attn_av":
        H, D, S = op.dims
        return 2 * S * H * D + 4 * H * S + eb * H * D
    if k == "gather":
        return (eb + 4) * n + eb * n
    if k == "program":
        return eb * n * (len(op.ins) + 1)
    return 0


def unfused_bytes(ops: Iterable[Op], scalar_bufs: Set[str] = frozenset()) -> int:
    return sum(op_bytes(op, scalar_bufs) for op in ops)


def fused_chain_bytes(ops: Sequence[Op], scalar_bufs: Set[str] = frozenset()) -> int:
    """Bytes of one register-resident pass over an elementwise chain."""
    produced = set()
    inputs = set()
    for op in ops:
        for r in op.ins:
            if r.buf not in produced and r.buf not in scalar_bufs:
                inputs.add(r.buf)
        produced.add(op.out.buf)
    eb = ELEM_BYTES[ops[0].dtype]
    n = ops[0].n
    outs = {op.out.buf for op in ops if not op.transient}
    return eb * n * (len(inputs) + len(outs))


def launch_model(launches: int, per_launch_s: float, compute_s: float) -> dict:
    """Host launch cost against device work for one step ("Launch Overhead and
    Fusion", section "Code": a decode step issues a fixed number of launches,
    each costing a fixed host time, on top of its compute).  Launches are
    issued one after another on one host thread, so their cost adds to the
    compute instead of overlapping it; the share is the launches' part of the
    total."""
    if launches < 0 or per_launch_s < 0 or compute_s < 0:
        raise ValueError("launch model: negative input")
    overhead = launches * per_launch_s
    total = overhead + compute_s
    return {"overhead_s": overhead, "total_s": total,
            "share": overhead / total if total > 0 else 0.0}
