"""Host logic of the PyTorch front end: which aten calls are queued, and the
views they become (metadata only, CPU tensors)."""

import pytest

torch = pytest.importorskip("torch")

from persistent_fusion_amd.torch_mode import plan_op  # noqa: E402

A = torch.ops.aten
CPU = torch.device("cpu")
_B = torch.zeros(8)
_S = torch.zeros(4, 4)


def test_broadcast_add_becomes_a_view():
    x = torch.zeros(6, 40)
    b = torch.zeros(40)
    kind, dt, alpha, shape, inplace, tens, vshape, vstr, _ = plan_op(A.add.Tensor, (x, b), {}, CPU)
    assert (kind, dt, shape, inplace) == ("add", "f32", (6, 40), False)
    assert vshape == [6, 40]
    assert vstr == [[40, 1], [40, 1], [0, 1]]


def test_scalar_mul_is_scale_and_transposed_input_keeps_strides():
    x = torch.zeros(8, 5).t()  # (5, 8), strides (1, 5)
    kind, dt, alpha, shape, inplace, tens, vshape, vstr, _ = plan_op(A.mul.Scalar, (x, 2.5), {}, CPU)
    assert (kind, alpha, shape) == ("scale", 2.5, (5, 8))
    # the output keeps the transposed layout, as eager PyTorch's does
    assert vstr[0] == [1, 5] and vstr[1] == [1, 5] and vstr[2] == [0, 0]
    assert list((x * 2.5).stride()) == vstr[0]


def test_in_place_and_unit_dimensions():
    x = torch.zeros(3, 1, 7, dtype=torch.float16)
    y = torch.zeros(1, 1, 7, dtype=torch.float16)
    kind, dt, alpha, shape, inplace, tens, vshape, vstr, _ = plan_op(A.add_.Tensor, (x, y), {}, CPU)
    assert (kind, dt, inplace, shape) == ("add", "f16", True, (3, 1, 7))
    assert vshape == [3, 7] and vstr == [[7, 1], [7, 1], [0, 1]]


@pytest.mark.parametrize("call", [
    lambda: (A.add.Tensor, (torch.zeros(4), torch.zeros(4)), {"alpha": 2}),          # alpha
    lambda: (A.add.Tensor, (torch.zeros(4), torch.zeros(4, dtype=torch.float64)), {}),  # mixed dtypes
    lambda: (A.add.Tensor, (torch.zeros(4, dtype=torch.float64), torch.zeros(4, dtype=torch.float64)), {}),
    lambda: (A.exp.default, (torch.zeros(4, dtype=torch.int32),), {}),                # exp on int32
    lambda: (A.mm.default, (torch.zeros(2, 2), torch.zeros(2, 2)), {}),               # not elementwise
    lambda: (A.add.Tensor, (torch.zeros(2, 2, 2, 2, 2), torch.zeros(2, 2, 2, 2, 2)), {}),  # 5-D
    lambda: (A.add.Tensor, (torch.zeros(0), torch.zeros(0)), {}),                     # empty
    lambda: (A.add_.Tensor, (torch.zeros(4), torch.zeros(3, 4)), {}),                 # in-place broadcast of self
    lambda: (A.add_.Tensor, (_B[:4], _B[1:5]), {}),                                   # in place over a shifted self
    lambda: (A.add_.Tensor, (_S, _S.t()), {}),                                        # in place over a transposed self
    lambda: (A.relu_.default, (torch.zeros(1, 4).expand(3, 4),), {}),                 # output names elements twice
    lambda: (A.clone.default, (torch.zeros(3, 4),), {"memory_format": torch.channels_last}),
])
def test_not_intercepted(call):
    func, args, kwargs = call()
    assert plan_op(func, args, kwargs, CPU) is None


def test_other_device_is_not_intercepted():
    x = torch.zeros(4)
    assert plan_op(A.relu.default, (x,), {}, torch.device("cuda", 0)) is None


def test_python_scalar_multiplier_is_scale():
    x = torch.zeros(10)
    kind, dt, alpha, shape, inplace, tens, vshape, vstr, _ = plan_op(A.mul.Tensor, (x, torch.tensor(0.25)), {}, CPU)
    assert (kind, alpha, shape) == ("scale", 0.25, (10,))


def test_in_place_over_itself_is_intercepted():
    x = torch.zeros(4, 4)
    plan = plan_op(A.add_.Tensor, (x, x), {}, CPU)
    assert plan is not None and plan[4] is True


def test_python_number_in_mul_tensor_is_scale():
    # ``x * 0.5`` reaches the dispatcher as mul.Tensor(x, 0.5)
    x = torch.zeros(6)
    kind, dt, alpha, shape, inplace, tens, vshape, vstr, _ = plan_op(A.mul.Tensor, (x, 0.5), {}, CPU)
    assert (kind, alpha, inplace, len(tens)) == ("scale", 0.5, False, 1)
    kind, dt, alpha, shape, inplace, tens, vshape, vstr, _ = plan_op(A.mul_.Tensor, (x, 3), {}, CPU)
    assert (kind, alpha, inplace) == ("scale", 3.0, True)
    assert plan_op(A.mul.Tensor, (torch.zeros(6, dtype=torch.int32), 2), {}, CPU) is None


def test_metadata_only_ops_are_listed():
    from persistent_fusion_amd.torch_mode import _metadata_ops

    meta = _metadata_ops()
    for f in (A.t.default, A.view.default, A.expand.default, A.slice.Tensor, A.transpose.int):
        assert f in meta
    for f in (A.add.Tensor, A.clone.default, A.sum.default, A.mm.default, A._to_copy.default):
        assert f not in meta


def test_program_plans_for_ops_without_an_opcode():
    from persistent_fusion_amd.torch_mode import _program_ops, program_plan

    x, y = torch.zeros(4), torch.ones(4)
    assert program_plan("sub", (x, y), {}) == (((("sub", 3, 0, 1),), 2), (), (x, y))
    assert program_plan("div", (x, y), {}) == (((("div", 3, 0, 1),), 2), (), (x, y))
    assert program_plan("add", (x, 2), {})[:2] == (((("add", 3, 0, 8),), 1), (2.0,))
    assert program_plan("sub", (x, 0.5), {})[:2] == (((("sub", 3, 0, 8),), 1), (0.5,))
    assert program_plan("rsub", (x, 1), {})[:2] == (((("sub", 3, 8, 0),), 1), (1.0,))  # 1 - x
    assert program_plan("neg", (x,), {})[:2] == (((("neg", 3, 0),), 1), ())
    assert program_plan("abs", (x,), {})[:2] == (((("abs", 3, 0),), 1), ())
    assert program_plan("div", (x, 2.0), {}) is None        # may be a reciprocal multiply in torch
    assert program_plan("add", (x, y), {}) is None          # a built-in ADD
    assert program_plan("sub", (x, y), {"alpha": 2}) is None
    table = _program_ops()
    assert table[A.sub_.Tensor] == ("sub", True) and table[A.rsub.Scalar] == ("rsub", False)


def test_host_only_arguments_are_recognised():
    from persistent_fusion_amd.torch_mode import _touches_cuda

    x = torch.zeros(3)
    assert not _touches_cuda((x, 2.0), {})
    assert not _touches_cuda(([x, x],), {"dim": 0})
    assert _touches_cuda((), {"device": torch.device("cuda", 0)})
    assert _touches_cuda((), {"device": "cuda:0"})
    assert not _touches_cuda((), {"device": torch.device("cpu")})


def test_contiguous_clone_of_a_transpose_is_a_transposed_copy():
    """x.t().contiguous() reaches the dispatcher as clone(contiguous_format):
    a COPY whose view reads the input down the output's columns."""
    x = torch.zeros(3, 5)
    kind, dt, alpha, shape, inplace, tens, vshape, vstr, _ = plan_op(
        A.clone.default, (x.t(),), {"memory_format": torch.contiguous_format}, CPU)
    assert (kind, dt, shape, inplace) == ("copy", "f32", (5, 3), False)
    assert vshape == [5, 3] and vstr[0] == [3, 1] and vstr[1] == [1, 5]


def _layouts():
    base = torch.zeros(6, 10)
    cube = torch.zeros(3, 4, 5)
    return [
        (A.relu.default, (base.t(),), {}),
        (A.exp.default, (cube.permute(2, 0, 1),), {}),
        (A.add.Tensor, (base.t(), base.t()), {}),
        (A.add.Tensor, (base.t(), torch.zeros(10, 6)), {}),     # mixed layouts
        (A.add.Tensor, (torch.zeros(10, 6), base.t()), {}),
        (A.mul.Tensor, (base.t(), torch.zeros(6)), {}),        # broadcast + transposed
        (A.mul.Tensor, (torch.zeros(6), base.t()), {}),
        (A.add.Tensor, (cube.transpose(0, 2), cube.transpose(0, 2)), {}),
        (A.clone.default, (base.t(),), {}),                     # preserve_format keeps it
        (A.clone.default, (base.t(),), {"memory_format": torch.contiguous_format}),
        (A.clone.default, (cube[:, ::2],), {}),                 # not dense: contiguous
        (A.mul.Tensor, (base.t(), 0.25), {}),
    ]


@pytest.mark.parametrize("case", range(len(_layouts())))
def test_output_layout_is_eagers(case):
    """Every queued out-of-place op's output has the strides eager PyTorch
    gives it, so views taken of it later (.view, .t()) behave the same."""
    func, args, kwargs = _layouts()[case]
    plan = plan_op(func, args, kwargs, CPU)
    assert plan is not None
    want = func(*args, **kwargs)
    assert plan[8] == tuple(want.stride()), (plan[8], want.stride())
    assert plan[3] == tuple(want.shape)
