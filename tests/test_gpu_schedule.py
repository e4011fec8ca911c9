"""GPU: scheduler guarantees of the resident kernel.

* Exactly once: with config.tile_counts the kernel counts, per ticket, how
  many times a wave ran that tile; after the queue has completed every
  published ticket must show exactly 1 and every later one 0 (the "each block
  runs exactly once" invariant of LithOS's kernel atomizer, section 5.4,
  Algorithm 1, here for the resident kernel's ticket ranges).  Checked on the
  1,000-op elementwise queue, on a 5,000-op write-once dynamic DAG (both
  against the oracle) and on the priority ring.
* Schedule jitter: with config.jitter every tile first waits a pseudo-random
  delay drawn from its ticket, so tiles start and finish in another order.
  Each op's tiles compute disjoint outputs with a fixed reduction order, so
  every result, of the exact and of the tolerance class, must be bit-identical
  to the run without jitter, and match the oracle.
* The grid checks in: gpuos_create returns only once every wave of the
  resident grid has started; the relaunch after a yield checks in again.
* Dependencies in time: with config.trace the kernel stamps each descriptor
  (one global 100 MHz clock); on a 2-layer decode, whose descriptors chain
  through their dependencies, every descriptor's first tile starts after the
  completion stamp of each dependency, and each record's stamps are in order
  (poll start, claim, completion; last store issued, acknowledged, counted).
"""

import numpy as np
import pytest

import oracle
from persistent_fusion_amd import gpuos, runner, workloads

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def _need_gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gpuos.lib()


def _run(wl, **cfg):
    """Runs wl on a fresh context; returns (outputs, ticket counts per ring)."""
    tensors = runner.to_device(wl, 0)
    addr = runner.addr_fn(tensors, wl)
    ctx = gpuos.Context(0, **cfg)
    try:
        runner.submit_workload(ctx, wl, addr)
        ctx.sync(0, 120.0)
        counts = {}
        if cfg.get("tile_counts"):
            for ring in (0, 1):
                n = ctx.tickets(ring)
                assert n + 64 <= cfg["tile_counts"], "raise tile_counts for this workload"
                counts[ring] = (n, np.array(ctx.tile_counts(ring, n + 64)))
    finally:
        ctx.destroy()
    return runner.download(tensors, wl, wl.outputs), counts


def _exactly_once(counts):
    for ring, (n, c) in counts.items():
        assert np.all(c[:n] == 1), f"ring {ring}: tickets run {sorted(set(c[:n].tolist()))} times"
        assert np.all(c[n:] == 0), f"ring {ring}: unpublished tickets ran"


def test_every_tile_runs_once_elementwise_queue():
    _need_gpu()
    say("exactly once: 1,000-op queue")
    wl = workloads.gen_elementwise_queue(seed=0)
    got, counts = _run(wl, tile_counts=1 << 16)
    assert counts[0][0] >= len(wl.ops)
    _exactly_once(counts)
    want = oracle.run(wl)
    for name in wl.outputs:
        assert oracle.compare(got[name], want[name], "f32").ok, name


def test_every_tile_runs_once_dynamic_dag():
    _need_gpu()
    say("exactly once: 5,000-op write-once dynamic DAG")
    wl = workloads.gen_dynamic_dag(seed=1, n_ops=5000, distinct_outputs=True)
    got, counts = _run(wl, tile_counts=1 << 21)
    say(f"  {counts[0][0]} tickets")
    _exactly_once(counts)
    bad = oracle.local_check(wl, got, oracle.compare)
    assert not bad, f"{len(bad)} ops differ, first: {bad[:3]}"


def test_every_tile_runs_once_priority_ring():
    _need_gpu()
    say("exactly once: priority mix, 20 rounds with 1M-element best-effort ops")
    wl = workloads.gen_priority_mix(seed=2, rounds=20, be_n=1 << 20)
    got, counts = _run(wl, tile_counts=1 << 16, priority=1)
    assert counts[1][0] >= 200
    _exactly_once(counts)


@pytest.mark.parametrize("which", ["queue", "chain", "dag", "decode"])
def test_jitter_changes_no_result(which):
    _need_gpu()
    say(f"jitter: {which}")
    wl = {"queue": lambda: workloads.gen_elementwise_queue(seed=3),
          "chain": lambda: workloads.gen_fused_chain(seed=3, n=1_000_003),
          "dag": lambda: workloads.gen_dynamic_dag(seed=3, n_ops=2000, distinct_outputs=True),
          "decode": lambda: workloads.gen_decode(seed=3, layers=2, tokens=3, distinct=True)}[which]()
    plain, _ = _run(wl)
    jit, counts = _run(wl, jitter=40, tile_counts=1 << 21)
    _exactly_once(counts)
    for name in wl.outputs:
        assert np.array_equal(plain[name].view(np.uint8), jit[name].view(np.uint8)), name
    if which in ("dag", "decode"):
        bad = oracle.local_check(wl, jit, oracle.compare)
        assert not bad, f"{len(bad)} ops differ, first: {bad[:3]}"
    else:
        want, scales = oracle.run(wl, scales=True)
        for name in wl.outputs:
            r = oracle.compare(jit[name], want[name], wl.dtypes[name], scales.get(name))
            assert r.ok, f"{name}: {r}"


def test_relaunch_after_yield_checks_in_again():
    _need_gpu()
    say("grid check-in on relaunch")
    wl = workloads.gen_elementwise_queue(seed=4, n_ops=300)
    tensors = runner.to_device(wl, 0)
    addr = runner.addr_fn(tensors, wl)
    ctx = gpuos.Context(0, tile_counts=1 << 14)
    try:
        half = [(0, 150), (150, 300)]
        ids = {}
        for g0, g1 in half:
            arr = gpuos.encode_ops(wl.ops, g0, g1, addr, ids)
            got = ctx.submit(arr, g1 - g0)
            ids.update({i: got[i - g0] for i in range(g0, g1)})
            ctx.flush()
            ctx.sync(0, 60.0)
            ctx.yield_gpu()
        assert ctx.stats()["launches"] == 2
        n = ctx.tickets(0)
        _exactly_once({0: (n, np.array(ctx.tile_counts(0, n + 64)))})
    finally:
        ctx.destroy()
    got = runner.download(tensors, wl, wl.outputs)
    want = oracle.run(wl)
    for name in wl.outputs:
        assert oracle.compare(got[name], want[name], "f32").ok, name


def test_trace_orders_every_dependency_in_time():
    _need_gpu()
    say("trace: dependencies in time, 2-layer decode")
    wl = workloads.gen_decode(seed=5, layers=2, tokens=3, distinct=True)
    tensors = runner.to_device(wl, 0)
    addr = runner.addr_fn(tensors, wl)
    ctx = gpuos.Context(0, trace=1)
    try:
        runner.submit_workload(ctx, wl, addr)
        ctx.sync(0, 60.0)
        recs = {r["seq"]: r for r in ctx.trace(1 << 16) if r["ring"] == 0}
        n = ctx.published(0)
        assert sorted(recs) == list(range(1, n + 1)), "a completed descriptor has no trace record"
        checked = 0
        for seq, r in recs.items():
            assert 0 < r["t_wait"] <= r["t_claim"] <= r["t_done"], (seq, r)
            assert 0 < r["t_end"] <= r["t_ack"] <= r["t_done"], (seq, r)
            for dep in (x for x in gpuos.decode_desc(ctx.read_desc(0, seq))["deps"] if x):
                assert r["t_claim"] > recs[dep]["t_done"], (seq, dep)
                checked += 1
        say(f"  {n} descriptors, {checked} dependencies")
        assert checked >= n // 2
    finally:
        ctx.destroy()
    bad = oracle.local_check(wl, runner.download(tensors, wl, wl.outputs), oracle.compare)
    assert not bad, f"{len(bad)} ops differ, first: {bad[:3]}"
