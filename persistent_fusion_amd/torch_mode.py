"""PyTorch front end: eager elementwise ops batched into the resident queue.

Idea (4) of "GPUOS: A GPU Operating System Primitive for Transparent
Operation Fusion" (section "The Paper") is to intercept PyTorch's dispatch so
that an unmodified eager program's small ops are batched into the persistent
kernel's queue instead of being launched one by one.  :class:`GpuosMode` is
that interception, as a ``TorchDispatchMode``:

* An elementwise op on CUDA tensors of the mode's device (``add``, ``mul``
  by a tensor or a scalar, ``relu``, ``exp``, ``clone``, and the in-place
  ``add_``, ``mul_``, ``relu_``), in fp32, bf16, fp16 or (add, mul, relu)
  int32, with broadcastable shapes of at most 4 non-trivial dimensions, is
  not run: its output tensor is allocated (torch supplies memory only) and
  the op is queued as a gpuos op with a view (strides from the broadcast),
  and the output tensor is returned at once.
* ``sub`` and ``div`` of two tensors, ``add``, ``sub`` and ``rsub`` with a
  Python number, ``neg`` and ``abs`` have no built-in opcode: over
  contiguous operands of one shape (fp32, bf16, fp16) each becomes an op
  defined at run time (a one-instruction register program, defined once per
  body and constant in the mode's context), the pages' runtime operator
  injection for the intercepted ops.
* An op that only makes a new view of existing memory (``t``, ``view``,
  ``expand``, ``slice`` and the like) runs at once: it touches no element.
* An op none of whose arguments is a CUDA tensor or names a CUDA device
  runs at once: it can neither read a queued result nor start a GPU kernel.
* Any other op, and leaving the mode, first flushes and waits for the queued
  ops and lets the resident kernel leave (``gpuos_yield``: while it is
  resident it holds every compute unit's registers, so no PyTorch kernel
  could start), then runs in PyTorch.  So every value PyTorch code can
  observe is final, and the ordering among queued ops comes from the
  runtime's hazard tracking.  The next queued op relaunches the kernel.
* Before the first queued op after PyTorch work, the current stream is
  synchronised, so the queue never reads a tensor a PyTorch kernel is still
  writing.  Every tensor a queued op touches is kept alive until the wait,
  so the caching allocator cannot hand its memory to another tensor first.

The decision whether and how to queue an op (:func:`plan_op`) only looks at
tensor metadata and is testable without a GPU.
"""

from __future__ import annotations

from typing import Optional, Sequence

from . import gpuos

_DTYPES = {}  # torch dtype -> gpuos dtype name (filled lazily: torch is optional at import)


def _dtype_name(t) -> Optional[str]:
    import torch

    if not _DTYPES:
        _DTYPES.update({torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16",
                        torch.int32: "i32"})
    return _DTYPES.get(t.dtype)


_TABLE: dict = {}


def _ops():
    if _TABLE:
        return _TABLE
    import torch

    a = torch.ops.aten
    _TABLE.update({
        a.add.Tensor: ("add", False), a.mul.Tensor: ("mul", False), a.mul.Scalar: ("scale", False),
        a.relu.default: ("relu", False), a.exp.default: ("exp", False),
        a.clone.default: ("copy", False),
        a.add_.Tensor: ("add", True), a.mul_.Tensor: ("mul", True), a.relu_.default: ("relu", True),
    })
    return _TABLE


_PTABLE: dict = {}


def _program_ops():
    """aten ops with no built-in opcode that run as programs defined at run
    time: func -> (name, in place).  See :func:`program_plan`."""
    if _PTABLE:
        return _PTABLE
    import torch

    a = torch.ops.aten
    _PTABLE.update({
        a.sub.Tensor: ("sub", False), a.sub_.Tensor: ("sub", True),
        a.div.Tensor: ("div", False), a.div_.Tensor: ("div", True),
        a.rsub.Scalar: ("rsub", False), a.add.Tensor: ("add", False),
        a.neg.default: ("neg", False), a.abs.default: ("abs", False),
    })
    return _PTABLE


def program_plan(name, args, kwargs):
    """The register program for an aten op of :func:`_program_ops`: (body
    key, constants, tensor operands), or None.  The key is (instructions,
    inputs) with the result in r3; constants sit in r8.. .  Tensor-tensor
    ``sub`` and ``div``, tensor-number ``add``, ``sub`` and ``rsub``, and
    ``neg``, ``abs``.  Division by a number is left to PyTorch (it may use a
    reciprocal, which would not give the same bits)."""
    kwargs = kwargs or {}
    if set(kwargs) - {"alpha"} or kwargs.get("alpha", 1) != 1:
        return None
    num = (int, float)
    if name in ("neg", "abs"):
        return ((((name, 3, 0),), 1), (), (args[0],)) if len(args) == 1 else None
    if len(args) != 2:
        return None
    x, y = args
    if type(y) in num:
        if name == "add":
            return (((("add", 3, 0, 8),), 1), (float(y),), (x,))
        if name == "sub":
            return (((("sub", 3, 0, 8),), 1), (float(y),), (x,))
        if name == "rsub":
            return (((("sub", 3, 8, 0),), 1), (float(y),), (x,))
        return None
    if name in ("sub", "div"):
        return ((((name, 3, 0, 1),), 2), (), (x, y))
    return None


def _touches_cuda(args, kwargs) -> bool:
    """Whether any argument is a CUDA tensor or names a CUDA device (then the
    op may read queued results or start a GPU kernel)."""
    import torch
    from torch.utils._pytree import tree_leaves

    for leaf in tree_leaves((args, kwargs or {})):
        if isinstance(leaf, torch.Tensor):
            if leaf.is_cuda:
                return True
        elif isinstance(leaf, torch.device):
            if leaf.type == "cuda":
                return True
        elif isinstance(leaf, str) and leaf.startswith("cuda"):
            return True
    return False


_META: set = set()


def _metadata_ops():
    """aten ops that only make a new view of existing memory: they read and
    write no element, so they run at once, with no wait for the queue."""
    if _META:
        return _META
    import torch

    a = torch.ops.aten
    for name, overloads in (("t", ("default",)), ("transpose", ("int",)), ("permute", ("default",)),
                            ("view", ("default",)), ("_unsafe_view", ("default",)),
                            ("expand", ("default",)), ("slice", ("Tensor",)), ("select", ("int",)),
                            ("unsqueeze", ("default",)), ("squeeze", ("default", "dim", "dims")),
                            ("as_strided", ("default",)), ("detach", ("default",)),
                            ("alias", ("default",)), ("split", ("Tensor",)), ("unbind", ("int",)),
                            ("diagonal", ("default",))):
        op = getattr(a, name, None)
        for ov in overloads:
            f = getattr(op, ov, None) if op is not None else None
            if f is not None:
                _META.add(f)
    return _META


def _broadcast(shapes):
    """The broadcast shape of ``shapes`` (numpy's rule), or None."""
    nd = max(len(s) for s in shapes)
    out = [1] * nd
    for s in shapes:
        for i, e in enumerate(s):
            d = nd - len(s) + i
            if e != 1:
                if out[d] != 1 and out[d] != e:
                    return None
                out[d] = e
    return out


def _strides_over(t, shape):
    """Element strides of tensor ``t`` read over the broadcast ``shape``
    (0 along every broadcast dimension)."""
    off = len(shape) - t.dim()
    st = [0] * len(shape)
    ts = t.stride()
    for i, e in enumerate(t.shape):
        if e != 1:
            st[off + i] = ts[i]
    return st


def _squeeze(shape: Sequence[int], strides: Sequence[Sequence[int]]):
    """Drops extent-1 dimensions (their strides never matter)."""
    keep = [d for d, e in enumerate(shape) if e != 1]
    return [shape[d] for d in keep], [[st[d] for d in keep] for st in strides]


def _dense_strides(shape, strides) -> bool:
    """Whether a tensor of ``shape`` with element ``strides`` addresses a
    dense block of prod(shape) elements, each once (a permuted contiguous
    layout)."""
    dims = sorted((st, e) for st, e in zip(strides, shape) if e != 1)
    acc = 1
    for st, e in dims:
        if st != acc:
            return False
        acc *= e
    return True


def eager_out_strides(func, args, kwargs, device):
    """The strides PyTorch itself gives the output of an out-of-place call:
    the same call on meta tensors (same shapes, strides and dtypes as the
    arguments on ``device``), which runs PyTorch's own layout rule and touches
    no element.  None if the call fails on meta tensors or its output is not
    a dense permuted layout."""
    import torch
    from torch.utils._pytree import tree_map

    def meta(a):
        if isinstance(a, torch.Tensor) and a.device == device:
            return torch.empty_strided(a.shape, a.stride(), dtype=a.dtype, device="meta")
        return a

    try:
        r = func(*tree_map(meta, tuple(args)), **tree_map(meta, dict(kwargs or {})))
    except Exception:  # an argument combination the meta kernels refuse
        return None
    if not isinstance(r, torch.Tensor) or not _dense_strides(r.shape, r.stride()):
        return None
    return tuple(r.stride())


def plan_op(func, args, kwargs, device):
    """How an aten call on tensors of ``device`` (a torch.device) would be
    queued: None if it is not interceptable, else (kind, dtype name, alpha,
    out shape, in-place, inputs, view shape, view strides [out, in0, in1],
    full-rank output strides).
    An out-of-place op's output gets the strides PyTorch would give it
    (:func:`eager_out_strides`): a dense input's layout is kept, as eager
    PyTorch keeps it, so later view ops behave the same in the mode.
    Pure metadata: no GPU work."""
    import torch

    table = _ops()
    if func not in table:
        return None
    kind, inplace = table[func]
    kwargs = kwargs or {}
    if kind == "add" and kwargs.get("alpha", 1) != 1:
        return None
    fmt = kwargs.get("memory_format", None)
    if kind == "copy" and fmt not in (None, torch.preserve_format, torch.contiguous_format):
        return None
    extra = set(kwargs) - {"alpha", "memory_format"}
    if extra:
        return None
    alpha = 0.0
    if kind == "scale":
        x, s = args[0], args[1]
        if not isinstance(s, (int, float)) or isinstance(s, bool):
            return None
        alpha, tens = float(s), [x]
    elif kind == "mul" and len(args) == 2 and type(args[1]) in (int, float):
        # ``x * 0.5`` reaches the dispatcher as mul.Tensor with a Python number
        if not isinstance(args[0], torch.Tensor):
            return None
        kind, alpha, tens = "scale", float(args[1]), [args[0]]
    elif kind in ("add", "mul"):
        if len(args) != 2 or not all(isinstance(a, torch.Tensor) for a in args):
            return None
        tens = list(args)
        # a Python number multiplying a tensor arrives wrapped as a 0-dim CPU
        # tensor: that is SCALE
        if kind == "mul" and args[1].dim() == 0 and args[1].device.type == "cpu" and \
                args[0].device == device and args[1].dtype in (torch.float32, torch.float64):
            if args[0].dtype not in (torch.float32, torch.bfloat16, torch.float16):
                return None
            kind, alpha, tens = "scale", float(args[1].item()), [args[0]]
    else:
        if len(args) != 1:
            return None
        tens = [args[0]]
    dev = device
    dt = _dtype_name(tens[0])
    if dt is None:
        return None
    for t in tens:
        if t.device != dev or t.dtype != tens[0].dtype or t.requires_grad:
            return None
    if dt == "i32" and kind not in ("add", "mul", "relu", "copy"):
        return None
    if any(t.numel() == 0 for t in tens):
        return None
    shape = _broadcast([t.shape for t in tens])
    if shape is None:
        return None
    shape = tuple(shape)
    n = 1
    for e in shape:
        n *= e
    if n > (1 << 30):
        return None
    if inplace and tuple(tens[0].shape) != shape:
        return None
    # strides of each operand over the output's index space (0 = broadcast)
    if inplace:
        out_strides = list(tens[0].stride())
    else:
        st = eager_out_strides(func, args, kwargs, dev)
        if st is None or len(st) != len(shape):
            return None
        out_strides = list(st)
    ins = [_strides_over(t, shape) for t in tens]
    if any(s < 0 for st in [out_strides] + ins for s in st):
        return None
    if inplace:
        # the runtime takes an in-place output only over itself under the same
        # view, and never one that names an element twice
        o = tens[0]
        if any(st == 0 and e > 1 for st, e in zip(out_strides, shape)):
            return None
        for t, st in zip(tens[1:], ins[1:]):
            if t.untyped_storage().data_ptr() == o.untyped_storage().data_ptr() and \
                    (t.data_ptr() != o.data_ptr() or st != out_strides):
                return None
    while len(ins) < 2:
        ins.append([0] * len(shape))
    vshape, vstr = _squeeze(list(shape), [out_strides] + ins)
    if len(vshape) > 4:
        return None
    if not vshape:  # a single element
        vshape, vstr = [1], [[1], [1 if len(tens) > 0 else 0], [1 if len(tens) > 1 else 0]]
    return kind, dt, alpha, shape, inplace, tens, vshape, vstr, tuple(out_strides)


class GpuosMode:
    """Context manager: ``with GpuosMode(): ...`` runs the block's eligible
    elementwise ops through one resident gpuos context (see the module
    docstring).  ``stats`` counts queued and passed-through ops.

    Queued ops are written into a preallocated gpuos_op / gpuos_view batch
    and handed to ``gpuos_submit_views`` and flushed ``batch`` at a time (and
    before any wait), so an error the runtime finds in an op surfaces at that
    call, and the device works on one batch while Python fills the next.
    Queued ops keep their tensors referenced until the next wait; once
    ``max_kept`` are held, a batch submission also waits for the queue."""

    def __init__(self, device: int = 0, batch: int = 64, max_kept: int = 1 << 16, **cfg):
        from torch.utils._python_dispatch import TorchDispatchMode

        outer = self

        class _Mode(TorchDispatchMode):
            def __torch_dispatch__(self, func, types, args=(), kwargs=None):
                return outer._dispatch(func, args, kwargs)

        import torch

        self._mode = _Mode()
        self.device = device
        self._torch_device = torch.device("cuda", device)
        self.ctx = gpuos.Context(device, **cfg)
        self._batch = max(1, batch)
        self.max_kept = max_kept
        self._ops = (gpuos.GpuosOp * self._batch)()
        self._views = (gpuos.GpuosView * self._batch)()
        self._k = 0         # ops in the batch
        self._unsynced = False  # flushed ops not yet waited for
        self._keep: list = []
        self._torch_dirty = True
        self._table = _ops()
        self._ptable = _program_ops()
        self._pids: dict = {}  # (body key, constants) -> program id
        self._meta = _metadata_ops()
        self._opcode = {k: gpuos.OPCODES[k] for k in ("add", "mul", "scale", "relu", "exp", "copy", "program")}
        self._dtype = {torch.float32: gpuos.DTYPES["f32"], torch.bfloat16: gpuos.DTYPES["bf16"],
                       torch.float16: gpuos.DTYPES["f16"], torch.int32: gpuos.DTYPES["i32"]}
        self._i32 = torch.int32
        self._empty_like = torch.empty_like
        self._empty_strided = torch.empty_strided
        self._tensor = torch.Tensor
        self.stats = {"queued": 0, "programs": 0, "metadata": 0, "host_ops": 0, "passed_through": 0,
                      "syncs": 0}

    # ------------------------------------------------------------------
    def _submit_batch(self) -> None:
        k = self._k
        if not k:
            return
        self._k = 0
        lib = self.ctx._lib
        rc = lib.gpuos_submit_views(self.ctx.handle, self._ops, self._views, k, None)
        if rc < 0:
            raise gpuos.GpuosError(rc, "gpuos_submit_views")
        # published at once, so the device runs this batch while Python queues
        # the next
        self.ctx.flush()
        self._unsynced = True
        if len(self._keep) >= self.max_kept:
            # the tensors of queued ops stay referenced until a wait: bound them
            self.sync()

    def sync(self) -> None:
        """Makes every queued op's result final."""
        self._submit_batch()
        if self._unsynced:
            self.ctx.sync(0, 120.0)
            self.stats["syncs"] += 1
            self._unsynced = False
        self._keep.clear()

    def _fast(self, func, args, kwargs):
        """(kind, dtype code, alpha, in-place, inputs) for the common case:
        contiguous operands of one shape and dtype on the mode's device, or
        None (then :func:`plan_op` decides)."""
        if kwargs:
            return None
        ent = self._table.get(func)
        if ent is None:
            return None
        kind, inplace = ent
        x = args[0]
        if type(x) is not self._tensor or x.get_device() != self.device or \
                x.requires_grad or not x.is_contiguous():
            return None
        dt = self._dtype.get(x.dtype)
        if dt is None:
            return None
        alpha = 0.0
        if kind == "mul" and type(args[1]) in (float, int):
            kind = "scale"
        if kind == "scale":
            s = args[1]
            if type(s) is not float and type(s) is not int:
                return None
            alpha, tens = float(s), (x,)
        elif kind in ("add", "mul"):
            y = args[1]
            if type(y) is not self._tensor or y.get_device() != self.device or \
                    y.requires_grad or not y.is_contiguous() or y.dtype != x.dtype or y.shape != x.shape:
                return None
            if inplace and y.data_ptr() != x.data_ptr() and \
                    y.untyped_storage().data_ptr() == x.untyped_storage().data_ptr():
                return None  # in place over a shifted part of itself
            tens = (x, y)
        else:
            tens = (x,)
        if x.dtype == self._i32 and kind not in ("add", "mul", "relu", "copy"):
            return None
        n = x.numel()
        if n == 0 or n > (1 << 30):
            return None
        return kind, dt, alpha, inplace, tens

    def _queue(self, kind, dt, alpha, out, tens, vshape=None, vstr=None, pid=0) -> None:
        """Writes one op (and its view, or none) into the next batch slot.
        Every field a slot's earlier op may have set is written again."""
        k = self._k
        o = self._ops[k]
        o.opcode = self._opcode[kind]
        o.dtype = dt
        o.n = out.numel()
        o.out = out.data_ptr()
        o.in_[0] = tens[0].data_ptr()
        o.in_[1] = tens[1].data_ptr() if len(tens) > 1 else None
        o.alpha = alpha
        o.aux[0] = pid  # the program id of a PROGRAM op, else 0
        v = self._views[k]
        if vshape is None:
            v.ndim = 0
        else:
            v.ndim = len(vshape)
            for d, e in enumerate(vshape):
                v.shape[d] = e
            for j in range(3):
                st = vstr[j]
                for d in range(len(vshape)):
                    v.stride[j][d] = st[d]
        self._keep.extend(tens)
        self._keep.append(out)
        self._k = k + 1
        if self._k == self._batch:
            self._submit_batch()

    def _dispatch(self, func, args, kwargs):
        fast = self._fast(func, args, kwargs)
        if fast is not None:
            kind, dt, alpha, inplace, tens = fast
            if self._torch_dirty:
                self._sync_torch()
            out = tens[0] if inplace else self._empty_like(tens[0])
            self._queue(kind, dt, alpha, out, tens)
            self.stats["queued"] += 1
            return out
        if func in self._ptable:
            done = self._try_program(func, args, kwargs)
            if done is not None:
                return done
        if func in self._meta:
            self.stats["metadata"] += 1
            return func(*args, **(kwargs or {}))
        plan = plan_op(func, args, kwargs, self._torch_device)
        if plan is None:
            if not _touches_cuda(args, kwargs):
                # a host-only op cannot observe the queue or start a GPU kernel
                self.stats["host_ops"] += 1
                return func(*args, **(kwargs or {}))
            # the queue finishes and the resident kernel gives the GPU back
            # (while it is resident no other kernel can start)
            self.sync()
            self.ctx.yield_gpu()
            self.stats["passed_through"] += 1
            self._torch_dirty = True
            return func(*args, **(kwargs or {}))
        kind, dt, alpha, shape, inplace, tens, vshape, vstr, ostr = plan
        if self._torch_dirty:
            self._sync_torch()
        out = tens[0] if inplace else self._empty_strided(shape, ostr, dtype=tens[0].dtype,
                                                           device=tens[0].device)
        self._queue(kind, gpuos.DTYPES[dt], alpha, out, tens, vshape, vstr)
        self.stats["queued"] += 1
        return out

    def _try_program(self, func, args, kwargs):
        """Queues an op of :func:`_program_ops` as a PROGRAM op over contiguous
        operands of one shape and a float dtype; None if it does not apply."""
        name, inplace = self._ptable[func]
        plan = program_plan(name, args, kwargs)
        if plan is None:
            return None
        key, consts, tens = plan
        x = tens[0]
        for t in tens:
            if type(t) is not self._tensor or t.get_device() != self.device or t.requires_grad or \
                    not t.is_contiguous() or t.dtype != x.dtype or t.shape != x.shape:
                return None
        dt = self._dtype.get(x.dtype)
        n = x.numel()
        if dt is None or x.dtype == self._i32 or n == 0 or n > (1 << 30):
            return None
        if inplace and len(tens) > 1 and tens[1].data_ptr() != x.data_ptr() and \
                tens[1].untyped_storage().data_ptr() == x.untyped_storage().data_ptr():
            return None
        pid = self._pids.get((key, consts))
        if pid is None:
            if len(self._pids) >= gpuos.PROG_MAX_PROGRAMS - 1:
                return None  # every program id is taken: PyTorch runs it
            insns, nin = key
            pid = self.ctx.program_define(gpuos.make_program(insns, nin, 3, consts))
            self._pids[(key, consts)] = pid
        if self._torch_dirty:
            self._sync_torch()
        out = x if inplace else self._empty_like(x)
        self._queue("program", dt, 0.0, out, tens, pid=pid)
        self.stats["queued"] += 1
        self.stats["programs"] += 1
        return out

    def _sync_torch(self) -> None:
        import torch

        torch.cuda.current_stream(self.device).synchronize()
        self._torch_dirty = False

    # ------------------------------------------------------------------
    def __enter__(self):
        self._mode.__enter__()
        return self

    def __exit__(self, *exc):
        try:
            self.sync()
            self.ctx.yield_gpu()
        finally:
            self._mode.__exit__(*exc)
        return False

    def close(self) -> None:
        self.ctx.destroy()
