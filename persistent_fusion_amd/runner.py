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
                    encoded=None) -> List[int]:
    """Submits every group of the workload (flushing after each); returns the ids."""
    ids: List[int] = [0] * len(wl.ops)
    id_of = {}
    for gi, (g0, g1) in enumerate(groups or wl.groups):
        arr = encoded[gi] if encoded is not None else gpuos.encode_ops(wl.ops, g0, g1, addr, id_of)
        got = ctx.submit(arr, g1 - g0)
        for k, i in enumerate(range(g0, g1)):
            ids[i] = got[k]
            id_of[i] = got[k]
        if flush_each:
            ctx.flush()
    return ids


def run_resident(wl: Workload, device: int = 0, outputs: Optional[Iterable[str]] = None,
                 tensors=None, timeout_s: float = 60.0, **cfg) -> Dict[str, np.ndarray]:
    """Runs the workload on a fresh resident context and returns the outputs."""
    tensors = tensors if tensors is not None else to_device(wl, device)
    addr = addr_fn(tensors, wl)
    ctx = gpuos.Context(device, **cfg)
    try:
        submit_workload(ctx, wl, addr)
        ctx.sync(0, timeout_s)
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
