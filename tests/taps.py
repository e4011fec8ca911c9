"""Tap ops: snapshots of sampled ops' inputs and outputs taken inside a queue.

A queue whose buffers are reused (a ring of output slots) keeps no op's
inputs to the end, so its ops cannot be re-checked one by one afterwards.
``add_taps`` inserts, around each sampled op, COPY ops that copy every input
operand's readable range into a fresh buffer just before the op and its
output range into another just after it.  The runtime orders the copies like
any other op (read-after-write on the producer, write-after-read for the next
writer of the slot), and COPY is a bit copy, so the snapshots are exactly
what the sampled op read and wrote.  ``check_taps`` re-runs each sampled op
in the oracle on its snapshot inputs and compares with its snapshot output.
"""

from __future__ import annotations

from dataclasses import replace
from typing import Dict, List, Sequence, Tuple

import numpy as np

import oracle
from persistent_fusion_amd.workloads import NP_DTYPE, Op, Ref, Workload


def _in_len(op: Op, k: int) -> int:
    # readable length of data operand k: src_len if shorter than the extent
    sl = op.src_len[k] if k < len(op.src_len) else 0
    return sl if sl and sl < op.n else op.n


def add_taps(wl: Workload, sample: Sequence[int]) -> Tuple[Workload, List[dict]]:
    sample = set(int(i) for i in sample)
    bufs = dict(wl.buffers)
    dts = dict(wl.dtypes)
    ops: List[Op] = []
    new_index: Dict[int, int] = {}
    taps: List[dict] = []
    for i, op in enumerate(wl.ops):
        tin = []
        if i in sample:
            for k, ref in enumerate(op.ins):
                cnt = _in_len(op, k)
                name = f"tap_in{i}_{k}"
                dt = wl.dtypes[ref.buf]
                bufs[name] = np.zeros(cnt, NP_DTYPE[dt])
                dts[name] = dt
                ops.append(Op("copy", Ref(name), (ref,), n=cnt, dtype=dt))
                tin.append(name)
        deps = tuple(new_index[d] for d in op.deps)
        new_index[i] = len(ops)
        ops.append(replace(op, deps=deps))
        if i in sample:
            cnt = oracle.out_len(op)
            dt = wl.dtypes[op.out.buf]
            name = f"tap_out{i}"
            bufs[name] = np.zeros(cnt, NP_DTYPE[dt])
            dts[name] = dt
            ops.append(Op("copy", Ref(name), (op.out,), n=cnt, dtype=dt))
            taps.append({"index": i, "op": op, "ins": tin, "out": name})
    groups = [(new_index[g0] - _taps_before(wl, sample, g0), _group_end(new_index, wl, sample, g1))
              for g0, g1 in wl.groups]
    outs = [t["out"] for t in taps] + [n for t in taps for n in t["ins"]]
    return Workload(wl.name + "+taps", bufs, dts, ops, groups=groups, outputs=outs,
                    meta=dict(wl.meta)), taps


def _taps_before(wl, sample, i):
    # tap-in copies inserted right before op i
    return len(wl.ops[i].ins) if i in sample else 0


def _group_end(new_index, wl, sample, g1):
    last = g1 - 1
    return new_index[last] + 1 + (1 if last in sample else 0)


def check_taps(wl: Workload, taps: List[dict], got: Dict[str, np.ndarray]) -> List[tuple]:
    """Re-runs each tapped op on its snapshot inputs; returns the mismatches."""
    bad = []
    for t in taps:
        op = t["op"]
        bufs = {name: got[name] for name in t["ins"]}
        dts = {name: wl.dtypes[name] for name in t["ins"]}
        out_dt = wl.dtypes[t["out"]]
        cnt = oracle.out_len(op)
        bufs["_y"] = np.zeros(cnt, NP_DTYPE[out_dt])
        dts["_y"] = out_dt
        aux = op.aux
        if aux is not None:
            bufs[aux.buf] = wl.buffers[aux.buf]
            dts[aux.buf] = wl.dtypes[aux.buf]
        src_len = tuple(_in_len(op, k) if k < len(op.ins) else 0 for k in range(2))
        mini = replace(op, out=Ref("_y"), ins=tuple(Ref(n) for n in t["ins"]), deps=(),
                       src_len=src_len)
        s = oracle.apply_op(mini, bufs, dts)
        r = oracle.compare(got[t["out"]], bufs["_y"], out_dt, s)
        if not r.ok:
            bad.append((t["index"], op.kind, r))
    return bad
