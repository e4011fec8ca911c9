"""GPU: the graph-replay comparator (per-op launches captured once as a HIP graph).

Each test captures a workload's launches, replays the graph several times with
ordinary torch work (re-upload of every input, NaN poisoning of the outputs)
and a device synchronisation between replays, and checks every replay: against
the oracle, and bit for bit against the same launches issued eagerly.
"""

import numpy as np
import pytest

import oracle
from persistent_fusion_amd import gpuos, runner, workloads

pytestmark = pytest.mark.gpu


def _need_gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gpuos.lib()


def say(msg):
    print(msg, flush=True)


def _same_bits(a, b):
    return a.tobytes() == b.tobytes()


@pytest.mark.parametrize("fuse", [False, True])
def test_graph_fused_chain(fuse):
    _need_gpu()
    say(f"graph fused chain n=1000003 fuse={fuse}")
    wl = workloads.gen_fused_chain(seed=5, n=1_000_003)
    eager = runner.run_per_op(wl, outputs=["y"], fuse=fuse)
    want, scales = oracle.run(wl, scales=True)
    reps = runner.run_graph(wl, outputs=["y"], fuse=fuse, replays=3)
    for r, got in enumerate(reps):
        assert _same_bits(got["y"], eager["y"]), f"replay {r} differs from eager"
        res = oracle.compare(got["y"], want["y"], "f32", scales.get("y"))
        assert res.ok, f"replay {r}: {res}"


@pytest.mark.parametrize("fuse", [False, True])
def test_graph_elementwise_queue(fuse):
    _need_gpu()
    say(f"graph elementwise queue 1000x4096 fuse={fuse}")
    wl = workloads.gen_elementwise_queue(seed=6)
    eager = runner.run_per_op(wl, fuse=fuse)
    want, scales = oracle.run(wl, scales=True)
    reps = runner.run_graph(wl, fuse=fuse, replays=3)
    for r, got in enumerate(reps):
        for name in wl.outputs:
            assert _same_bits(got[name], eager[name]), f"replay {r} {name} differs from eager"
            res = oracle.compare(got[name], want[name], wl.dtypes[name], scales.get(name))
            assert res.ok, f"replay {r} {name}: {res}"


@pytest.mark.parametrize("fuse", [False, True])
def test_graph_decode(fuse):
    _need_gpu()
    say(f"graph decode 2 layers x 3 tokens fuse={fuse}")
    wl = workloads.gen_decode(seed=7, layers=2, tokens=3, distinct=True)
    eager = runner.run_per_op(wl, fuse=fuse)
    reps = runner.run_graph(wl, fuse=fuse, replays=3)
    for r, got in enumerate(reps):
        for name in wl.outputs:
            assert _same_bits(got[name], eager[name]), f"replay {r} {name} differs from eager"
        bad = oracle.local_check(wl, got, oracle.compare)
        assert not bad, [(i, wl.ops[i].kind, n, str(x)) for i, n, x in bad[:5]]


def test_graph_empty_and_errors():
    _need_gpu()
    import torch

    say("graph: empty op list, bad op, null handles")
    with gpuos.Graph(0, (gpuos.GpuosOp * 1)(), 0) as g:
        g.launch(torch.cuda.current_stream(0).cuda_stream)
        torch.cuda.synchronize()
    bad = (gpuos.GpuosOp * 1)()
    bad[0].opcode = 250
    with pytest.raises(gpuos.GpuosError):
        gpuos.Graph(0, bad, 1)
    assert gpuos.lib().gpuos_graph_launch(None, None) < 0
    assert gpuos.lib().gpuos_graph_destroy(None) < 0
