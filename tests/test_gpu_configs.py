"""GPU parity of the full-size synthetic configurations, by sampled local
checks: each checked op is re-run by the oracle on exactly the inputs the GPU
gave it and compared element by element (bit-exact for COPY, ADD, MUL, SCALE,
RELU, ROPE; 1e-5 / 1e-2 relative to the oracle's error scale otherwise).

* Decode at full size: every op, and end to end, in test_gpu_fullsize.py.
* Dynamic DAG: 100,000 ops, sizes 256..1,048,576, outputs in a 64-slot ring
  (so the 65,536-slot descriptor ring wraps).  Tap ops snapshot a sample of
  ops' inputs and outputs inside the queue (the per-op arbiter; the untapped
  stream's final slots are compared end to end in test_gpu_fullsize.py);
  plus a 5,000-op write-once stream checked op by op in full.
* Priority mix: 200 rounds of one 64M-element fp32 best-effort op and ten
  4,096-element bf16 latency-critical ops.
"""

import numpy as np
import pytest

import oracle
from persistent_fusion_amd import gpuos, runner, workloads
from taps import add_taps, check_taps

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def _need_gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gpuos.lib()


def test_dynamic_dag_write_once_5000():
    _need_gpu()
    say("dynamic DAG, 5,000 ops with one output buffer each")
    wl = workloads.gen_dynamic_dag(seed=1, n_ops=5000, distinct_outputs=True)
    got = runner.run_resident(wl, timeout_s=120.0)
    bad = oracle.local_check(wl, got, oracle.compare)
    assert not bad, f"{len(bad)} ops differ, first: {bad[:3]}"


def test_dynamic_dag_full_size_tapped():
    _need_gpu()
    say("dynamic DAG, 100,000 ops in a 64-slot output ring, tapped")
    wl = workloads.gen_dynamic_dag(seed=0)
    rng = np.random.default_rng(12)
    sample = sorted(int(i) for i in rng.choice(len(wl.ops), 400, replace=False))
    sample += [len(wl.ops) - 1]
    twl, taps = add_taps(wl, sample)
    got = runner.run_resident(twl, timeout_s=120.0)
    bad = check_taps(twl, taps, got)
    assert not bad, f"{len(bad)} of {len(taps)} tapped ops differ, first: {bad[:3]}"


def _priority_oracle_subset(wl):
    # the final best-effort outputs come from the last op writing each of the
    # two output buffers; the latency-critical ops read only their own inputs
    last = {}
    for i, op in enumerate(wl.ops):
        if not op.lc:
            last[op.out.buf] = i
    keep = sorted(set(last.values()) | {i for i, op in enumerate(wl.ops) if op.lc})
    return workloads.Workload("priority_subset", wl.buffers, wl.dtypes,
                              [wl.ops[i] for i in keep], outputs=wl.outputs)


@pytest.mark.parametrize("priority", [1, 2])
def test_priority_mix_full_size(priority):
    _need_gpu()
    say(f"priority mix 200 rounds, priority={priority}")
    wl = workloads.gen_priority_mix(seed=0)
    if priority == 2:
        # no priority ring: the same ops, all in submission order
        from dataclasses import replace
        wl = workloads.Workload(wl.name, wl.buffers, wl.dtypes,
                                [replace(op, lc=False) for op in wl.ops], outputs=wl.outputs)
    got = runner.run_resident(wl, timeout_s=120.0, priority=priority)
    want, scales = oracle.run(_priority_oracle_subset(wl), scales=True)
    for name in wl.outputs:
        r = oracle.compare(got[name], want[name], wl.dtypes[name], scales.get(name))
        assert r.ok, f"{name}: {r}"
