"""Replaying what the PyTorch front end queued through the oracle.

``RecordingMode`` is a GpuosMode that also writes down every op it queues:
the op kind, dtype, scalar, program body, and for every operand the tensor
(kept alive, so no storage is freed and reused while recording).  After the
run, ``to_workload`` turns the record into an oracle Workload: one buffer per
distinct device storage (the initial contents of a storage that existed
before the mode are the snapshot taken by ``snapshot``; storages the mode
allocated start as zeros and are written before they are read), every op an
oracle Op over that storage at the tensor's element offset, with its view.
``final_storages`` downloads the same storages after the run, so that the
oracle's final buffers can be compared with the device's element by element.
"""

from __future__ import annotations

from typing import Dict, List

import numpy as np

from persistent_fusion_amd import gpuos
from persistent_fusion_amd.torch_mode import GpuosMode
from persistent_fusion_amd.workloads import Op, Program, Ref, Workload

_DT_NAME = {v: k for k, v in gpuos.DTYPES.items()}
_KIND = {v: k for k, v in gpuos.OPCODES.items()}
_NP = {"f32": np.float32, "bf16": np.uint16, "f16": np.float16, "i32": np.int32}


def _flat(t):
    """The whole storage of tensor t as a flat tensor of its dtype."""
    import torch

    es = t.element_size()
    n = t.untyped_storage().nbytes() // es
    return torch.empty(0, dtype=t.dtype, device=t.device).set_(t.untyped_storage(), 0, (n,), (1,))


def _to_numpy(flat, dt):
    import torch

    if dt == "bf16":
        return flat.view(torch.int16).cpu().numpy().view(np.uint16)
    return flat.cpu().numpy()


def snapshot(tensors) -> Dict[int, np.ndarray]:
    """Contents of the storages of `tensors` (before the mode runs)."""
    import torch

    torch.cuda.synchronize()
    out = {}
    for t in tensors:
        dt = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16",
              torch.int32: "i32"}[t.dtype]
        out[t.untyped_storage().data_ptr()] = _to_numpy(_flat(t), dt)
    return out


class RecordingMode(GpuosMode):
    def __init__(self, *a, **kw):
        super().__init__(*a, **kw)
        self.record: List[dict] = []

    def _queue(self, kind, dt, alpha, out, tens, vshape=None, vstr=None, pid=0) -> None:
        prog = None
        if kind == "program":
            for (key, consts), p in self._pids.items():
                if p == pid:
                    insns, nin = key
                    prog = Program(tuple(tuple(i) for i in insns), nin, 3, tuple(consts))
        self.record.append({"kind": kind, "dt": _DT_NAME[dt], "alpha": alpha, "out": out,
                            "ins": tuple(tens), "vshape": None if vshape is None else list(vshape),
                            "vstr": None if vstr is None else [list(v) for v in vstr], "prog": prog})
        super()._queue(kind, dt, alpha, out, tens, vshape, vstr, pid)


def to_workload(record: List[dict], initial: Dict[int, np.ndarray]) -> Workload:
    bufs: Dict[str, np.ndarray] = {}
    dts: Dict[str, str] = {}
    names: Dict[int, str] = {}
    flats = {}

    def ref(t, dt) -> Ref:
        st = t.untyped_storage()
        base = st.data_ptr()
        if base not in names:
            name = f"s{len(names)}"
            names[base] = name
            n = st.nbytes() // t.element_size()
            bufs[name] = initial[base].copy() if base in initial else np.zeros(n, _NP[dt])
            dts[name] = dt
            flats[name] = _flat(t)
        assert dts[names[base]] == dt, "a storage read with two dtypes"
        off = (t.data_ptr() - base) // t.element_size()
        return Ref(names[base], off)

    ops: List[Op] = []
    for r in record:
        dt = r["dt"]
        out = r["out"]
        ins = tuple(ref(t, dt) for t in r["ins"])
        o = ref(out, dt)
        view = None
        if r["vshape"] is not None:
            sh = tuple(r["vshape"])
            so, s0, s1 = (tuple(v) for v in r["vstr"])
            view = (sh, so, s0, s1)
        kind = r["kind"]
        n = out.numel()
        ops.append(Op(kind, o, ins if kind not in ("scale", "relu", "exp", "copy") else ins[:1],
                      n=n, dtype=dt, alpha=r["alpha"], view=view, prog=r["prog"]))
    wl = Workload("torch_mode_record", bufs, dts, ops, outputs=sorted(bufs))
    wl.meta["flats"] = flats
    return wl


def final_storages(wl: Workload) -> Dict[str, np.ndarray]:
    import torch

    torch.cuda.synchronize()
    return {name: _to_numpy(flat, wl.dtypes[name]) for name, flat in wl.meta["flats"].items()}
