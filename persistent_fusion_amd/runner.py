"""Running a seeded workload through the native runtime.

Device memory for the workload's buffers comes from torch (allocation and
host<->device copies only); every op runs in the HIP kernels behind
:mod:`persistent_fusion_amd.gpuos`.  A wait on the whole device
(``torch.cuda.synchronize()``) while a context is open also waits for the
resident kernel, which leaves only after its idle period (or in
``gpuos_stop`` / ``gpuos_destroy``); destroy contexts first.
"""

from __future__ import annotations

from typing import Dict, Iterable, List, Optional

import numpy as np

from . import gpuos
from .workloads import ELEM_BYTES, Ref, Workload

_TORCH_DT = {"f32": "float32", "bf16": "int16", "i32": "int32"}


def to_device(wl: Workload, device: int = 0, names: Optional[Iterable[str]] = None) -> Dict[str, "object"]:
    """Uploads the workload's buffers; bf16 buffers travel as raw 16-bit words."""
    import torch

    out = {}
    for name in (names or wl.buffers):
        arr = wl.buffers[name]
        dt = wl.dtypes[name]
        host = arr.view(np.int16) if dt == "bf16" else arr
        t = torch.from_numpy(np.ascontiguousarray(host)).to(f"cuda:{device}")
        out[name] = t
    return out


def download(tensors: Dict[str, "object"], wl: Workload, names: Iterable[str]) -> Dict[str, np.ndarray]:
    res = {}
    for name in names:
        a = tensors[name].cpu().numpy()
        if wl.dtypes[name] == "bf16":
            a = a.view(np.uint16)
        res[name] = a
    return res


def addr_fn(tensors: Dict[str, "object"], wl: Workload):
    base = {k: t.data_ptr() for k, t in tensors.items()}

    def addr(ref: Ref, dtype: str) -> int:
        return base[ref.buf] + ref.off * ELEM_BYTES[wl.dtypes[ref.buf]]

    return addr


def submit_workload(ctx: gpuos.Context, wl: Workload, addr, groups=None, flush_each: bool = True,
                    encoded=None, compile_programs: bool = False) -> List[int]:
    """Submits every group of the workload (flushing after each); returns the
    ids.  With compile_programs, the workload's programs are compiled
    (gpuos_program_compile) before the first submission."""
    ids: List[int] = [0] * len(wl.ops)
    id_of = {}
    prog_ids = gpuos.define_programs(ctx, wl.ops) if encoded is None else None
    if compile_programs and prog_ids:
        ctx.program_compile()
    for gi, (g0, g1) in enumerate(groups or wl.groups):
        arr = encoded[gi] if encoded is not None else \
            gpuos.encode_ops(wl.ops, g0, g1, addr, id_of, prog_ids)
        got = ctx.submit(arr, g1 - g0, views=gpuos.encode_views(wl.ops, g0, g1))
        for k, i in enumerate(range(g0, g1)):
            ids[i] = got[k]
            id_of[i] = got[k]
        if flush_each:
            ctx.flush()
    return ids


def run_resident(wl: Workload, device: int = 0, outputs: Optional[Iterable[str]] = None,
                 tensors=None, timeout_s: float = 60.0, compile_programs: bool = False,
                 stats: Optional[dict] = None, **cfg) -> Dict[str, np.ndarray]:
    """Runs the workload on a fresh resident context and returns the outputs
    (the context's final counters go into `stats` if given)."""
    tensors = tensors if tensors is not None else to_device(wl, device)
    addr = addr_fn(tensors, wl)
    ctx = gpuos.Context(device, **cfg)
    try:
        submit_workload(ctx, wl, addr, compile_programs=compile_programs)
        ctx.sync(0, timeout_s)
        if stats is not None:
            stats.update(ctx.stats())
    finally:
        ctx.destroy()
    return download(tensors, wl, outputs or wl.outputs)


def run_per_op(wl: Workload, device: int = 0, outputs: Optional[Iterable[str]] = None,
               tensors=None, fuse: bool = False) -> Dict[str, np.ndarray]:
    """Runs the workload as one kernel launch per op (stream order)."""
    import torch

    tensors = tensors if tensors is not None else to_device(wl, device)
    addr = addr_fn(tensors, wl)
    stream = torch.cuda.current_stream(device).cuda_stream
    for g0, g1 in wl.groups:
        arr = gpuos.encode_ops(wl.ops, g0, g1, addr, {i: 0 for i in range(g0)})
        gpuos.baseline_run(device, arr, g1 - g0, fuse=fuse, stream=stream)
    torch.cuda.current_stream(device).synchronize()
    return download(tensors, wl, outputs or wl.outputs)


def _out_elems(op) -> int:
    """Number of output elements an op writes."""
    if op.kind == "row_sum":
        return op.rows
    if op.kind == "gemv":
        return op.dims[0]
    if op.kind == "attn_score":
        H, _, S = op.dims
        return H * S
    if op.kind == "attn_av":
        H, D, _ = op.dims
        return H * D
    return op.n


def poisonable(wl: Workload, outputs: Iterable[str]) -> List[str]:
    """The `outputs` whose first use in op order is a write of the whole buffer
    (so no op can observe their contents before the workload sets them)."""
    first = {}
    for op in wl.ops:
        reads = {r.buf for r in op.ins}
        if op.aux is not None:
            reads.add(op.aux.buf)
        for b in reads:
            first.setdefault(b, False)
        if op.out.buf not in first:
            whole = op.out.off == 0 and _out_elems(op) >= len(wl.buffers[op.out.buf])
            first[op.out.buf] = whole
    return [b for b in outputs if first.get(b, False)]


def restore(tensors: Dict[str, "object"], wl: Workload, outputs: Iterable[str]) -> None:
    """Re-uploads every buffer's initial contents, then fills the outputs that
    the workload overwrites whole before any read (see `poisonable`) with NaN
    (all-ones words for bf16 and i32), on torch's current stream."""
    import torch

    for name, t in tensors.items():
        arr = wl.buffers[name]
        host = arr.view(np.int16) if wl.dtypes[name] == "bf16" else arr
        t.copy_(torch.from_numpy(np.ascontiguousarray(host)))
    for name in poisonable(wl, outputs):
        t = tensors[name]
        t.fill_(float("nan") if wl.dtypes[name] in ("f32", "f16") else -1)


def capture_graph(wl: Workload, tensors, device: int = 0, fuse: bool = False) -> gpuos.Graph:
    """Captures the workload's per-op launches (all groups, in order) as one graph."""
    addr = addr_fn(tensors, wl)
    arr = gpuos.encode_ops(wl.ops, 0, len(wl.ops), addr, {})
    return gpuos.Graph(device, arr, len(wl.ops), fuse=fuse)


def run_graph(wl: Workload, device: int = 0, outputs: Optional[Iterable[str]] = None,
              fuse: bool = False, replays: int = 3) -> List[Dict[str, np.ndarray]]:
    """Replays the captured per-op launches `replays` times; before each replay
    the buffers are restored and the outputs poisoned by ordinary torch work,
    and after it the device is synchronised.  Returns each replay's outputs."""
    import torch

    outputs = list(outputs or wl.outputs)
    tensors = to_device(wl, device)
    stream = torch.cuda.current_stream(device)
    res = []
    with capture_graph(wl, tensors, device, fuse) as g:
        for _ in range(replays):
            restore(tensors, wl, outputs)
            torch.cuda.synchronize(device)
            g.launch(stream.cuda_stream)
            torch.cuda.synchronize(device)
            res.append(download(tensors, wl, outputs))
    return res
