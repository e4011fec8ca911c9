#!/usr/bin/env python3
"""Benchmark of the persistent small-op kernel on one MI355X.

The headline is the fused chain y = relu(a*x + b) on 16,777,216-element fp32
vectors through the resident kernel.  A step is one pass of the whole path
over one batch: gpuos_submit of the three descriptors, gpuos_flush (fusion
pass, ring publication, doorbell), the resident kernel's claim, dispatch and
completion, and (once, after the last step) gpuos_sync.  Four independent
replicas of x, a, b, y (1 GiB) rotate across steps so the 256 MB infinity
cache cannot serve a pass from the previous one.  The warm-up and timed passes
run in one launch of the resident kernel, whose duration (HIP events on its
stream) gives the roofline's achieved bandwidth.  Beside it: one kernel launch
per op, a stand-alone fused kernel, graph replay, a plain copy kernel.

The same line carries the other small-op streams (`configs`): the 1,000-op
elementwise queue, the 24-layer decode, the 100,000-op dynamic DAG and the
two-priority mix, each with ops/s, GB/s, its roofline fraction, the per-op
launch comparator and the CPU oracle (untuned, one thread pinned to one core)
on a bounded sample.

Prints one JSON line (rank 0).  Only one GPU is supported.
"""

from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

N_ELEMS = 16_777_216
REPLICAS = 4
HBM_PEAK_GBS = 8000.0
METRIC = "small ops/sec and effective HBM GB/s vs per-op launch, 1× MI355X"
# sources whose change invalidates the committed HBM byte counts
KERNEL_SOURCES = ("kernels.hip", "tile_ops.h", "device_common.h", "gpuos_internal.h")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def fused_chain_leg(steps, warmup, device=0, warm_s=0.5):
    """One resident launch: warm-up passes (at least `warmup`, and at least
    `warm_s` seconds of them, so that the GPU's clocks and memory system are
    at their sustained state), then `steps` timed passes."""
    import torch

    from persistent_fusion_amd import gpuos, runner, traffic, workloads

    wl = workloads.gen_fused_chain(seed=0, n=N_ELEMS)
    fused_bytes = traffic.fused_chain_bytes(wl.ops)
    unfused_bytes = traffic.unfused_bytes(wl.ops)
    reps = []
    for r in range(REPLICAS):
        reps.append(runner.to_device(wl, device))
    arrs = []
    for t in reps:
        addr = runner.addr_fn(t, wl)
        arrs.append(gpuos.encode_ops(wl.ops, 0, 3, addr, {}))
    torch.cuda.synchronize()

    # the launch covers the warm-up passes and the timed passes; the HIP events
    # recorded around it on its stream give the kernel's duration
    ctx = gpuos.Context(device, trace=1)
    # warm-up: at least `warmup` passes and warm_s seconds of them, submitted
    # back to back; the host stays at most 128 passes ahead of the device (it
    # waits for pass k - 128 before submitting pass k), so the device never
    # idles and the host never queues seconds of work.  Then the queue drains.
    w0 = time.perf_counter()
    k = 0
    last = []
    while k < warmup or time.perf_counter() - w0 < warm_s:
        if len(last) >= 128:
            oid = last.pop(0)
            while not ctx.query(oid):
                pass
        last.append(ctx.submit(arrs[k % REPLICAS], 3)[-1])
        ctx.flush()
        k += 1
    ctx.sync(0, 60.0)
    warm_passes = k
    log(f"bench: fused chain, one resident launch: {warm_passes} warm-up passes "
        f"({time.perf_counter() - w0:.2f} s) + {steps} timed passes")
    t0 = time.perf_counter()
    for k in range(steps):
        ctx.submit_noids(arrs[(warm_passes + k) % REPLICAS], 3)
        ctx.flush()
    ctx.sync(0, 120.0)
    t1 = time.perf_counter()
    ctx.stop()
    st = ctx.stats()
    tr = ctx.trace()
    ctx.destroy()
    torch.cuda.synchronize()
    wall = t1 - t0
    if st["launches"] != 1:
        raise RuntimeError(f"the resident kernel was launched {st['launches']} times in one session")
    kernel_s = st["kernel_ns"] * 1e-9
    # device-side busy span of the timed passes from the in-kernel trace (100 MHz)
    fused = sorted((r for r in tr if r["opcode"] == 32), key=lambda r: r["seq"])[-steps:]
    dev_span = None
    if fused:
        dev_span = (max(r["t_done"] for r in fused) - min(r["t_claim"] for r in fused)) * 1e-8
    per_pass_dev = sorted((r["t_done"] - r["t_claim"]) * 1e-8 for r in fused)

    # output of the last pass (checked against the oracle in the CPU leg)
    y = reps[(warm_passes + steps - 1) % REPLICAS]["y"].cpu().numpy()

    # per-op launches (3 kernels per pass) and one stand-alone fused kernel
    log("bench: fused chain baselines (per-op launches, stand-alone fused kernel, graph replay)")
    stream = torch.cuda.current_stream(device)
    res = {}
    for label, fuse in (("per_op_launch", False), ("standalone_fused_kernel", True)):
        for k in range(warmup):
            gpuos.baseline_run(device, arrs[k % REPLICAS], 3, fuse=fuse, stream=stream.cuda_stream)
        stream.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for k in range(steps):
            gpuos.baseline_run(device, arrs[k % REPLICAS], 3, fuse=fuse, stream=stream.cuda_stream)
        e1.record(stream)
        stream.synchronize()
        w = time.perf_counter() - t0
        gpu_s = e0.elapsed_time(e1) * 1e-3
        launches = steps * (1 if fuse else 3)
        res[label] = {"gb_per_s": round(steps * fused_bytes / w / 1e9, 1),
                      "ms_per_step": round(w / steps * 1e3, 4),
                      "launches_per_step": 1 if fuse else 3,
                      "avg_kernel_us_events": round(gpu_s / launches * 1e6, 2),
                      "hbm_bytes_per_step": fused_bytes if fuse else unfused_bytes}
    # the same launches captured once per buffer replica as HIP graphs
    for label, fuse in (("graph_replay", False), ("graph_replay_fused", True)):
        graphs = [gpuos.Graph(device, a, 3, fuse=fuse) for a in arrs]
        try:
            for k in range(warmup):
                graphs[k % REPLICAS].launch(stream.cuda_stream)
            stream.synchronize()
            t0 = time.perf_counter()
            for k in range(steps):
                graphs[k % REPLICAS].launch(stream.cuda_stream)
            stream.synchronize()
            w = time.perf_counter() - t0
        finally:
            for g in graphs:
                g.destroy()
        res[label] = {"gb_per_s": round(steps * fused_bytes / w / 1e9, 1),
                      "ms_per_step": round(w / steps * 1e3, 4),
                      "launches_per_step": 1 if fuse else 3,
                      "hbm_bytes_per_step": fused_bytes if fuse else unfused_bytes}
    del reps
    torch.cuda.empty_cache()
    return {
        "wall_s": wall, "kernel_s": kernel_s, "dev_span_s": dev_span, "y": y, "warmup_passes": warm_passes,
        "fused_bytes": fused_bytes, "unfused_bytes": unfused_bytes,
        "per_pass_dev_us": per_pass_dev[len(per_pass_dev) // 2] * 1e6 if per_pass_dev else None,
        "stats": st, "baselines": res,
    }


def copy_leg(device=0, reps=10):
    """A plain device copy of 1 GiB (torch's copy kernel): the bandwidth a
    simple streaming kernel reaches on this GPU, and the known-size kernel the
    HBM byte counters are calibrated with."""
    import torch

    n = 1 << 28  # 268,435,456 fp32 = 1 GiB
    src = torch.empty(n, dtype=torch.float32, device=f"cuda:{device}").uniform_()
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    s = e0.elapsed_time(e1) * 1e-3 / reps
    del src, dst
    torch.cuda.empty_cache()
    return {"bytes_per_launch": 2 * 4 * n, "gb_per_s": round(2 * 4 * n / s / 1e9, 1),
            "kernel": "torch copy_ (1 GiB -> 1 GiB)"}


def queue_leg(reps_n, device=0):
    """1,000 fp32 elementwise ops on 4,096-element vectors: ops/s."""
    import torch

    from persistent_fusion_amd import gpuos, runner, workloads

    wl = workloads.gen_elementwise_queue(seed=0)
    t = runner.to_device(wl, device)
    addr = runner.addr_fn(t, wl)
    arr = gpuos.encode_ops(wl.ops, 0, len(wl.ops), addr, {})
    n_ops = len(wl.ops)
    torch.cuda.synchronize()
    ctx = gpuos.Context(device)
    ctx.submit_noids(arr, n_ops)
    ctx.sync(0, 60.0)  # warm-up
    times = []
    for _ in range(reps_n):
        t0 = time.perf_counter()
        ctx.submit_noids(arr, n_ops)
        ctx.sync(0, 60.0)
        times.append(time.perf_counter() - t0)
    ctx.destroy()
    # one more queue with the in-kernel trace on (not timed), for the gaps
    ctx = gpuos.Context(device, trace=1)
    ctx.submit_noids(arr, n_ops)
    ctx.sync(0, 60.0)
    gaps = handoff_gaps(ctx, ctx.trace())
    ctx.destroy()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(device)
    gpuos.baseline_run(device, arr, n_ops, stream=stream.cuda_stream)
    stream.synchronize()
    btimes = []
    for _ in range(reps_n):
        t0 = time.perf_counter()
        gpuos.baseline_run(device, arr, n_ops, stream=stream.cuda_stream)
        stream.synchronize()
        btimes.append(time.perf_counter() - t0)
    med = sorted(times)[len(times) // 2]
    bmed = sorted(btimes)[len(btimes) // 2]
    gtimes, gbuild = _time_graph(device, arr, n_ops, False, reps_n)
    gmed = sorted(gtimes)[len(gtimes) // 2]
    del t
    return {"ops": n_ops, "elems": 4096, "resident_ops_per_s": round(n_ops / med),
            "per_op_launch_ops_per_s": round(n_ops / bmed),
            "speedup_vs_per_op_launch": round(bmed / med, 2),
            "graph_replay_ops_per_s": round(n_ops / gmed),
            "speedup_vs_graph_replay": round(gmed / med, 2),
            "graph_replay_us_per_queue_median": round(gmed * 1e6, 1),
            "graph_capture_and_instantiate_ms": round(gbuild * 1e3, 2),
            "per_op_launch_us_per_op": round(bmed / n_ops * 1e6, 2),
            "resident_trace": gaps,
            "resident_us_per_queue_median": round(med * 1e6, 1),
            "resident_us_per_queue_p10_p90": [round(_pct(times, 0.1) * 1e6, 1), round(_pct(times, 0.9) * 1e6, 1)],
            "per_op_launch_us_per_queue_median": round(bmed * 1e6, 1),
            "per_op_launch_us_per_queue_p10_p90": [round(_pct(btimes, 0.1) * 1e6, 1),
                                                   round(_pct(btimes, 0.9) * 1e6, 1)],
            "effective_gb_per_s": round(wl.meta["bytes"] / med / 1e9, 1),
            "roofline": {"bound": "latency (16 MB working set, cache-resident)",
                         "frac_of_hbm_peak": _frac(wl.meta["bytes"] / med / 1e9)}}


def _pct(xs, q):
    """The q-quantile of xs (nearest rank)."""
    v = sorted(xs)
    return v[min(len(v) - 1, int(q * len(v)))]


def launch_rate_leg(device=0, n=10000):
    """The pages' launch-overhead measurement, in C++ HIP: an empty kernel
    launched n times back to back (host time per launch), and n times each
    followed by a stream synchronize (time per launch-and-wait round trip)."""
    from persistent_fusion_amd import gpuos

    a, s = gpuos.launch_overhead(device, n)
    return {"kernel": "empty kernel, one wave", "launches": n,
            "us_per_launch_back_to_back": round(a, 2), "us_per_launch_and_sync": round(s, 2)}


class _NoIds(dict):
    """Ids of earlier groups for per-op launches: none (stream order already
    covers every dependency)."""

    def __missing__(self, key):
        return 0


def _time_per_op(device, groups_encoded, sizes):
    """The same submission groups as one launch per op on one stream."""
    import torch

    from persistent_fusion_amd import gpuos

    stream = torch.cuda.current_stream(device)
    stream.synchronize()
    t0 = time.perf_counter()
    for arr, k in zip(groups_encoded, sizes):
        gpuos.baseline_run(device, arr, k, stream=stream.cuda_stream)
    stream.synchronize()
    return time.perf_counter() - t0


def _time_graph(device, arr, n, fuse, reps):
    """The per-op launches of arr[0, n) captured once as a HIP graph: one
    untimed replay, then `reps` replays each timed from launch to the end of a
    stream synchronisation."""
    import torch

    from persistent_fusion_amd import gpuos

    stream = torch.cuda.current_stream(device)
    t0 = time.perf_counter()
    g = gpuos.Graph(device, arr, n, fuse=fuse)
    build_s = time.perf_counter() - t0
    try:
        g.launch(stream.cuda_stream)
        stream.synchronize()
        times = []
        for _ in range(reps):
            t0 = time.perf_counter()
            g.launch(stream.cuda_stream)
            stream.synchronize()
            times.append(time.perf_counter() - t0)
    finally:
        g.destroy()
    return times, build_s


def handoff_gaps(ctx, recs):
    """Idle gaps between dependent ops inside the resident kernel, from its
    trace (100 MHz timestamps): for every descriptor whose dependencies are all
    in `recs`, the time from the last dependency's completion to the claim of
    the descriptor's first tile, and whether that tile's wave was already
    polling when the dependency completed; and each descriptor's own
    claim-to-done time, split at the completing wave's last store issue and
    its acknowledgement (work, store acknowledgement, completion count)."""
    from persistent_fusion_amd import gpuos

    by_seq = {r["seq"]: r for r in recs if r["ring"] == 0}
    gaps, busy, waiting = [], [], 0
    for seq, r in by_seq.items():
        busy.append((r["t_done"] - r["t_claim"]) * 1e-2)
        deps = [x for x in gpuos.decode_desc(ctx.read_desc(0, seq))["deps"] if x]
        if not deps or any(x not in by_seq for x in deps):
            continue
        last_done = max(by_seq[x]["t_done"] for x in deps)
        gaps.append((r["t_claim"] - last_done) * 1e-2)
        waiting += 0 < r["t_wait"] <= last_done
    gaps.sort()
    busy.sort()
    pick = lambda v, q: round(v[min(len(v) - 1, int(q * len(v)))], 2) if v else None
    return {"descriptors": len(by_seq), "with_deps": len(gaps),
            "handoff_us_p50": pick(gaps, 0.5), "handoff_us_p90": pick(gaps, 0.9),
            "first_tile_polling_at_dep_done_frac": round(waiting / len(gaps), 3) if gaps else None,
            "busy_us_p50": pick(busy, 0.5), "busy_us_p90": pick(busy, 0.9)}


def critical_path_split(recs, names):
    """Median split of each descriptor kind's claim-to-done time (µs): work up
    to the completing wave's last store issue, that store's acknowledgement,
    and the completion count (tile counter atomics)."""
    by_op = {}
    for x in recs:
        if not (x["t_claim"] <= x["t_end"] <= x["t_ack"] <= x["t_done"]):
            continue
        by_op.setdefault(names.get(x["opcode"], str(x["opcode"])), []).append(
            ((x["t_end"] - x["t_claim"]) * 1e-2, (x["t_ack"] - x["t_end"]) * 1e-2, (x["t_done"] - x["t_ack"]) * 1e-2))
    med = lambda v: round(sorted(v)[len(v) // 2], 2)
    return {k: {"work_us": med([w for w, _, _ in v]), "store_ack_us": med([a for _, a, _ in v]),
                "count_us": med([c for _, _, c in v]), "n": len(v)} for k, v in sorted(by_op.items())}


def decode_leg(device=0, reps=3):
    """Batch-1 decode: 24 layers, 64 tokens, 360 ops per token, one flush per
    token, one sync at the end."""
    import torch

    from persistent_fusion_amd import gpuos, runner, workloads

    wl = workloads.gen_decode(seed=0)
    t = runner.to_device(wl, device)
    addr = runner.addr_fn(t, wl)
    enc = [gpuos.encode_ops(wl.ops, g0, g1, addr, {}) for g0, g1 in wl.groups]
    sizes = [g1 - g0 for g0, g1 in wl.groups]
    torch.cuda.synchronize()
    ctx = gpuos.Context(device, trace=1)
    times = []
    for r in range(reps + 1):
        t0 = time.perf_counter()
        for arr, k in zip(enc, sizes):
            ctx.submit_noids(arr, k)
            ctx.flush()
        ctx.sync(0, 120.0)
        if r:
            times.append(time.perf_counter() - t0)
    tr = ctx.trace(1 << 16)
    descs_per_run = ctx.stats()["descs_published"] // (reps + 1)
    last_run = sorted(tr, key=lambda x: x["seq"])[-descs_per_run:]
    gaps = handoff_gaps(ctx, last_run)
    # median claim-to-completion time of each descriptor kind in the last run
    names = {v: k for k, v in gpuos.OPCODES.items()}
    names.update({32: "fused_ew", 33: "norm_gemv", 34: "gemv_add", 35: "softmax_av"})
    by_op = {}
    for x in last_run:
        by_op.setdefault(names.get(x["opcode"], str(x["opcode"])), []).append((x["t_done"] - x["t_claim"]) * 1e-2)
    busy_by_op = {k: round(sorted(v)[len(v) // 2], 2) for k, v in sorted(by_op.items())}
    split = critical_path_split(last_run, names)
    ctx.destroy()
    torch.cuda.synchronize()
    per_op = []
    for r in range(reps + 1):
        w = _time_per_op(device, enc, sizes)
        if r:
            per_op.append(w)
    # the whole 64-token run (every group, in order) captured as one graph:
    # the most favourable case for replay, since no launch is issued per token
    whole = gpuos.encode_ops(wl.ops, 0, len(wl.ops), addr, {})
    graph = {}
    for label, fuse in (("graph_replay", False), ("graph_replay_fused", True)):
        gt, gb = _time_graph(device, whole, len(wl.ops), fuse, reps)
        graph[label] = (min(gt), gb)
    tokens = wl.meta["tokens"]
    ops = len(wl.ops)
    byt = (wl.meta["weight_bytes"] + wl.meta["kv_bytes"]) * tokens
    best, best_b = min(times), min(per_op)
    # device-side span of the last run from the trace (fused descriptors
    # carry several ops, so count descriptors, not ops)
    recs = sorted(tr, key=lambda x: x["seq"])[-descs_per_run:]
    dev_s = (max(x["t_done"] for x in recs) - min(x["t_claim"] for x in recs)) * 1e-8 if recs else None
    del t
    torch.cuda.empty_cache()
    return {"workload": "decode 24 layers, hidden 896, 14x64 heads, FFN 4864, KV 512, 64 tokens",
            "ops": ops, "tokens": tokens,
            "resident_tok_per_s": round(tokens / best, 1),
            "resident_ops_per_s": round(ops / best),
            "resident_gb_per_s": round(byt / best / 1e9, 1),
            "resident_device_span_ms": round(dev_s * 1e3, 3) if dev_s else None,
            "per_op_launch_tok_per_s": round(tokens / best_b, 1),
            "per_op_launch_ops_per_s": round(ops / best_b),
            "speedup_vs_per_op_launch": round(best_b / best, 2),
            "graph_replay_tok_per_s": round(tokens / graph["graph_replay"][0], 1),
            "graph_replay_fused_tok_per_s": round(tokens / graph["graph_replay_fused"][0], 1),
            "speedup_vs_graph_replay": round(graph["graph_replay"][0] / best, 2),
            "speedup_vs_graph_replay_fused": round(graph["graph_replay_fused"][0] / best, 2),
            "graph_capture_and_instantiate_ms": round(graph["graph_replay"][1] * 1e3, 1),
            "per_op_launch_us_per_op": round(best_b / ops * 1e6, 2),
            "resident_trace_last_run": gaps,
            "resident_busy_us_by_descriptor": busy_by_op,
            "resident_critical_path_us_by_descriptor": split,
            "bytes_per_token": byt // tokens,
            "roofline": {"bound": "hbm (weights and KV cache stream every token)",
                         "frac_of_hbm_peak": _frac(byt / best / 1e9)}}


def dag_leg(device=0, reps=2):
    """100,000 ops, log-uniform sizes, random DAG, 64-slot output ring;
    submitted in groups of 1,000 with a flush each, one sync at the end."""
    import torch

    from persistent_fusion_amd import gpuos, runner, workloads

    wl = workloads.gen_dynamic_dag(seed=0, group=1000)
    t = runner.to_device(wl, device)
    addr = runner.addr_fn(t, wl)
    n = len(wl.ops)
    # a context numbers ops 1, 2, 3, ... in submission order, so pass r's op i
    # gets id r * n + i + 1: encode every pass beforehand
    passes = []
    for r in range(reps + 1):
        ids = {i: r * n + i + 1 for i in range(n)}
        passes.append([(gpuos.encode_ops(wl.ops, g0, g1, addr, ids), g1 - g0) for g0, g1 in wl.groups])
    torch.cuda.synchronize()
    ctx = gpuos.Context(device)
    times = []
    for r in range(reps + 1):
        t0 = time.perf_counter()
        first = None
        for arr, k in passes[r]:
            got = ctx.submit(arr, k)
            first = got[0] if first is None else first
            ctx.flush()
        ctx.sync(0, 300.0)
        if first != r * n + 1:
            raise RuntimeError("unexpected op ids")
        if r:
            times.append(time.perf_counter() - t0)
    ctx.destroy()
    torch.cuda.synchronize()
    # one more pass with the in-kernel trace on (not timed): hand-off gaps of
    # the last 65,536 descriptors, and whether the wave holding each one's
    # first tile was already waiting when its last dependency completed (a
    # wave still busy with earlier tickets arrives late)
    ctx = gpuos.Context(device, trace=1)
    for arr, k in passes[0]:
        ctx.submit_noids(arr, k)
        ctx.flush()
    ctx.sync(0, 300.0)
    tr = ctx.trace(1 << 16)
    gaps = handoff_gaps(ctx, tr)
    late = []
    by_seq = {r["seq"]: r for r in tr if r["ring"] == 0}
    for seq, r in by_seq.items():
        deps = [x for x in gpuos.decode_desc(ctx.read_desc(0, seq))["deps"] if x]
        if deps and all(x in by_seq for x in deps):
            last_done = max(by_seq[x]["t_done"] for x in deps)
            if r["t_wait"] > last_done:
                late.append((r["t_wait"] - last_done) * 1e-2)
    late.sort()
    gaps["late_first_wave_us_p50"] = round(late[len(late) // 2], 2) if late else None
    gaps["late_first_wave_us_p90"] = round(late[int(0.9 * len(late))], 2) if late else None
    ctx.destroy()
    torch.cuda.synchronize()
    # per-op launches: stream order covers every dependency
    enc_b = [gpuos.encode_ops(wl.ops, g0, g1, addr, _NoIds()) for g0, g1 in wl.groups]
    sizes = [g1 - g0 for g0, g1 in wl.groups]
    per_op = [_time_per_op(device, enc_b, sizes) for _ in range(reps)]
    best, best_b = min(times), min(per_op)
    del t
    torch.cuda.empty_cache()
    return {"workload": "dynamic DAG: 100,000 ops, n log-uniform 256..1,048,576, add/mul/relu/exp/"
                        "row_sum/row_softmax, 0-2 deps among the previous 8, 64-slot output ring",
            "ops": n, "algorithmic_bytes": wl.meta["bytes"],
            "resident_ops_per_s": round(n / best),
            "resident_gb_per_s": round(wl.meta["bytes"] / best / 1e9, 1),
            "per_op_launch_ops_per_s": round(n / best_b),
            "per_op_launch_gb_per_s": round(wl.meta["bytes"] / best_b / 1e9, 1),
            "speedup_vs_per_op_launch": round(best_b / best, 2),
            "resident_trace": gaps,
            "roofline": {"bound": "hbm and dependency latency",
                         "frac_of_hbm_peak": _frac(wl.meta["bytes"] / best / 1e9)}}


def priority_leg(device=0, rounds=200):
    """Two-priority mix: per round one 64M-element fp32 best-effort op (no
    wait), then ten bf16 4,096-element latency-critical ops, each submitted,
    flushed and waited for (closed loop)."""
    import torch

    from persistent_fusion_amd import gpuos, runner, workloads, traffic

    wl = workloads.gen_priority_mix(seed=0, rounds=rounds)
    t = runner.to_device(wl, device)
    addr = runner.addr_fn(t, wl)
    enc = [gpuos.encode_ops(wl.ops, i, i + 1, addr, {}) for i in range(len(wl.ops))]
    be_bytes = sum(traffic.op_bytes(op) for op in wl.ops if not op.lc)
    lc_bytes = sum(traffic.op_bytes(op) for op in wl.ops if op.lc)
    torch.cuda.synchronize()
    res = {}
    for label, prio in (("priority_ring", 1), ("single_ring", 2)):
        ctx = gpuos.Context(device, priority=prio)
        lat = []
        t0 = time.perf_counter()
        for i, op in enumerate(wl.ops):
            if not op.lc:
                ctx.submit_noids(enc[i], 1)
                ctx.flush()
                continue
            a = enc[i]
            if prio == 2:
                a[0].flags &= ~gpuos.FLAG_LC
            s0 = time.perf_counter()
            oid = ctx.submit(a, 1, flush=True)[0]
            while not ctx.query(oid):
                pass
            lat.append(time.perf_counter() - s0)
            if prio == 2:
                a[0].flags |= gpuos.FLAG_LC
        ctx.sync(0, 120.0)
        wall = time.perf_counter() - t0
        ctx.destroy()
        lat.sort()
        res[label] = {"lc_p50_us": round(lat[len(lat) // 2] * 1e6, 1),
                      "lc_p99_us": round(lat[int(len(lat) * 0.99)] * 1e6, 1),
                      "lc_max_us": round(lat[-1] * 1e6, 1),
                      "aggregate_gb_per_s": round((be_bytes + lc_bytes) / wall / 1e9, 1)}
    torch.cuda.synchronize()
    # best-effort ops alone, back to back
    ctx = gpuos.Context(device)
    t0 = time.perf_counter()
    for i, op in enumerate(wl.ops):
        if not op.lc:
            ctx.submit_noids(enc[i], 1)
            ctx.flush()
    ctx.sync(0, 120.0)
    res["best_effort_alone_gb_per_s"] = round(be_bytes / (time.perf_counter() - t0) / 1e9, 1)
    ctx.destroy()
    # per-op launches: best-effort ops on one stream, latency-critical ops on a
    # second stream (both at the default priority), each LC op waited for
    s_be = torch.cuda.Stream(device)
    s_lc = torch.cuda.Stream(device)
    lat = []
    t0 = time.perf_counter()
    for i, op in enumerate(wl.ops):
        if not op.lc:
            gpuos.baseline_run(device, enc[i], 1, stream=s_be.cuda_stream)
            continue
        s0 = time.perf_counter()
        gpuos.baseline_run(device, enc[i], 1, stream=s_lc.cuda_stream)
        s_lc.synchronize()
        lat.append(time.perf_counter() - s0)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    lat.sort()
    res["per_op_launch_two_streams"] = {"lc_p50_us": round(lat[len(lat) // 2] * 1e6, 1),
                                        "lc_p99_us": round(lat[int(len(lat) * 0.99)] * 1e6, 1),
                                        "lc_max_us": round(lat[-1] * 1e6, 1),
                                        "aggregate_gb_per_s": round((be_bytes + lc_bytes) / wall / 1e9, 1)}
    del t
    torch.cuda.empty_cache()
    res["workload"] = (f"{rounds} rounds of one fp32[67,108,864] best-effort op and ten "
                       "bf16[4096] latency-critical ops (closed loop)")
    res["ops"] = len(wl.ops)
    res["roofline"] = {"bound": "hbm (best-effort ops); latency (latency-critical ops)",
                       "frac_of_hbm_peak": _frac(res["priority_ring"]["aggregate_gb_per_s"])}
    return res


def torch_frontend_leg(device=0, reps=5, n_ops=1000, sizes=(4096, 1 << 20)):
    """The same eager PyTorch program (n_ops elementwise ops on fp32 tensors
    of each size in ``sizes``, each reading one or two earlier results: add,
    mul, relu, scale, and sub and neg, which have no built-in opcode) run by
    PyTorch itself and under GpuosMode, which queues the ops into the
    resident kernel; host wall time per program including the final
    synchronisation that brings the result to the host."""
    import numpy as np
    import torch

    from persistent_fusion_amd.torch_mode import GpuosMode

    rng = np.random.default_rng(0)
    prog = []
    for i in range(n_ops):
        kind = int(rng.integers(0, 6))
        a, b = int(rng.integers(0, 2 + i)), int(rng.integers(0, 2 + i))
        prog.append((kind, a, b, float(rng.uniform(-1, 1))))

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            r = fn()
            float(r)  # the result reaches the host
            ts.append(time.perf_counter() - t0)
        return sorted(ts)[len(ts) // 2], float(r)

    res = {"workload": f"{n_ops} eager elementwise ops (add/mul/relu/scale by a Python float, and sub/neg, "
                       "which the mode runs as programs defined at run time), fp32"}
    mode = GpuosMode(device)
    try:
        for size in sizes:
            torch.manual_seed(0)
            base = [torch.rand(size, device=f"cuda:{device}") * 2 - 1 for _ in range(2)]

            def run():
                vals = list(base)
                for kind, a, b, s in prog:
                    x, y = vals[a], vals[b]
                    vals.append(x + y if kind == 0 else x * y if kind == 1 else
                                torch.relu(x) if kind == 2 else x * s if kind == 3 else
                                x - y if kind == 4 else -x)
                return vals[-1].sum()

            def in_mode():
                with mode:
                    return run()

            eager_s, eager_r = timed(run)
            mode_s, mode_r = timed(in_mode)
            res[f"n{size}"] = {
                "eager_pytorch_us_per_op": round(eager_s / n_ops * 1e6, 2),
                "gpuos_mode_us_per_op": round(mode_s / n_ops * 1e6, 2),
                "speedup_vs_eager_pytorch": round(eager_s / mode_s, 2),
                "same_result": bool(abs(eager_r - mode_r) <= 1e-3 * max(1.0, abs(eager_r)))}
            print(f"torch front end n={size}: {res[f'n{size}']}", file=sys.stderr, flush=True)
            del base
    finally:
        mode.close()
    return res


def views_leg(device=0, steps=100, warmup=30, R=4096, C=4096):
    """Elementwise ops over strided and broadcast views: fp32 [R x C], 4
    rotating replicas, one resident launch per case, host wall time over
    `steps` passes.  Cases: a bias add y = x + b[None, :] (reads x and a
    C-element bias, writes y), a row scale y = x * s[:, None], a transposed
    copy y = x.T (reads x down its columns), a batched transposed copy
    y[b] = x[b].T of 16 [2048 x 512] blocks (the same bytes), and the
    contiguous y = x + z for reference.  GB/s counts each operand's bytes
    once."""
    import torch

    from persistent_fusion_amd import gpuos

    n = R * C
    E = 4
    BR, BC = 512, 2048  # the batched transpose's output block: [n / (BR * BC), BR, BC]
    assert n % (BR * BC) == 0
    out = {"workload": f"views over fp32 [{R} x {C}], 4 rotating replicas"}
    cases = {
        "bias_add": ("add", [[C, 1], [C, 1], [0, 1]], (n + C + n) * E),
        "row_scale": ("mul", [[C, 1], [C, 1], [1, 0]], (n + R + n) * E),
        "transpose_copy": ("copy", [[C, 1], [1, R], [0, 0]], 2 * n * E),
        "batched_transpose_copy": ("copy", [[BR * BC, BC, 1], [BR * BC, 1, BR], [0, 0, 0]], 2 * n * E),
        "contiguous_add": ("add", None, 3 * n * E),
    }
    for name, (kind, strides, byt) in cases.items():
        shape = [n // (BR * BC), BR, BC] if name.startswith("batched") else [R, C]
        reps = []
        for r in range(REPLICAS):
            x = torch.rand(n, device=f"cuda:{device}")
            second = torch.rand(n if name == "contiguous_add" else max(R, C), device=f"cuda:{device}")
            y = torch.empty(n, device=f"cuda:{device}")
            ins = [x.data_ptr()] + ([] if kind == "copy" else [second.data_ptr()])
            op = gpuos.make_op(kind, y.data_ptr(), ins, n=n)
            view = gpuos.make_view(shape, strides) if strides else None
            reps.append((x, second, y, (gpuos.GpuosOp * 1)(op),
                         (gpuos.GpuosView * 1)(view) if view is not None else None))
        torch.cuda.synchronize()
        ctx = gpuos.Context(device)
        try:
            def one(k):
                _, _, _, arr, varr = reps[k % REPLICAS]
                ctx.submit(arr, 1, views=varr)
                ctx.flush()
            for k in range(warmup):
                one(k)
            ctx.sync(0, 60.0)
            t0 = time.perf_counter()
            for k in range(steps):
                one(warmup + k)
            ctx.sync(0, 120.0)
            wall = time.perf_counter() - t0
        finally:
            ctx.destroy()
        # spot check of the last pass against PyTorch on the same tensors
        x, second, y, _, _ = reps[(warmup + steps - 1) % REPLICAS]
        X = x.view(R, C)
        want = {"bias_add": lambda: X + second[:C][None, :], "row_scale": lambda: X * second[:R][:, None],
                "transpose_copy": lambda: X.t().contiguous().view(R, C) if R == C else None,
                "batched_transpose_copy": lambda: x.view(-1, BC, BR).transpose(1, 2).contiguous().view(R, C),
                "contiguous_add": lambda: X + second.view(R, C)}[name]()
        gbs = steps * byt / wall / 1e9
        out[name] = {"gb_per_s": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                     "same_as_torch": bool(want is None or torch.equal(y.view(R, C), want))}
        log(f"bench: views leg {name}: {out[name]}")
        del reps
        torch.cuda.empty_cache()
    return out


def program_leg(device=0, steps=200, warmup=100):
    """The fused chain y = relu(a*x + b) at 16,777,216 fp32 elements computed
    by one op defined at run time (a 3-instruction register program) instead
    of the built-in fused descriptor: one resident launch, the same rotating
    replicas and passes as the headline, 16 algorithmic bytes per element.
    The program runs interpreted (fusion off), compiled at run time into the
    kernel variant (gpuos_program_compile, fusion off) and lowered to the
    fused micro-program (fusion on, the default); the built-in fused chain is
    timed the same way in the same process."""
    import numpy as np
    import torch

    from persistent_fusion_amd import gpuos, runner, workloads

    ys = {}
    out = {"workload": "relu(a*x+b), 16,777,216 fp32 elements, 3-instruction program (interpreted; "
                       "compiled at run time; lowered) vs built-in fused chain, 4 rotating replicas"}
    prog_wl = workloads.gen_program_chain(seed=0, n=N_ELEMS)
    for label, wl, fusion in (("program", prog_wl, 2), ("program_compiled", prog_wl, 2),
                              ("program_lowered", prog_wl, 1),
                              ("builtin_fused", workloads.gen_fused_chain(seed=0, n=N_ELEMS), 1)):
        reps = [runner.to_device(wl, device) for _ in range(REPLICAS)]
        ctx = gpuos.Context(device, trace=1, fusion=fusion)
        try:
            pids = gpuos.define_programs(ctx, wl.ops)
            if label == "program_compiled":
                t0 = time.perf_counter()
                ctx.program_compile(dtypes=["f32"])
                out["compile_s"] = round(time.perf_counter() - t0, 2)
            arrs = [gpuos.encode_ops(wl.ops, 0, len(wl.ops), runner.addr_fn(t, wl), {}, pids) for t in reps]
            torch.cuda.synchronize()
            for k in range(warmup):
                ctx.submit_noids(arrs[k % REPLICAS], len(wl.ops))
                ctx.flush()
            ctx.sync(0, 60.0)
            t0 = time.perf_counter()
            for k in range(steps):
                ctx.submit_noids(arrs[(warmup + k) % REPLICAS], len(wl.ops))
                ctx.flush()
            ctx.sync(0, 120.0)
            wall = time.perf_counter() - t0
            tr = ctx.trace()
        finally:
            ctx.destroy()
        op_code = gpuos.OPCODES["program"] if label in ("program", "program_compiled") else 32  # 32: fused
        recs = sorted((r for r in tr if r["opcode"] == op_code), key=lambda r: r["seq"])[-steps:]
        per_pass = sorted((r["t_done"] - r["t_claim"]) * 1e-8 for r in recs)
        out[label] = {"gb_per_s": round(steps * 16 * N_ELEMS / wall / 1e9, 1),
                      "median_pass_device_us": round(per_pass[len(per_pass) // 2] * 1e6, 2) if per_pass else None}
        log(f"bench: program leg {label}: {out[label]}")
        ys[label] = reps[(warmup + steps - 1) % REPLICAS]["y"].cpu().numpy()
        del reps
    out["program_vs_builtin"] = round(out["program"]["gb_per_s"] / out["builtin_fused"]["gb_per_s"], 3)
    out["program_compiled_vs_builtin"] = round(out["program_compiled"]["gb_per_s"] /
                                               out["builtin_fused"]["gb_per_s"], 3)
    out["program_lowered_vs_builtin"] = round(out["program_lowered"]["gb_per_s"] /
                                              out["builtin_fused"]["gb_per_s"], 3)
    out["bit_identical"] = bool(all(np.array_equal(ys[k].view(np.uint32), ys["builtin_fused"].view(np.uint32))
                                    for k in ("program", "program_compiled", "program_lowered")))
    return out


# ---------------------------------------------------------------------------
# CPU baseline: the oracle, untuned, single-threaded, pinned to one core, in a
# child process (so that BLAS is limited to one thread before numpy loads and
# the pinning does not touch the GPU process).


def _cpu_info():
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "usable_cores": len(os.sched_getaffinity(0)), "cpu_model": model}


def _oracle_sample(cfg, budget_s):
    """Runs the oracle on a bounded sample of config `cfg` in this process;
    returns the measured sample."""
    import numpy as np

    import oracle
    from persistent_fusion_amd import traffic, workloads

    np.seterr(all="ignore")
    t_end = None

    def over(t0):
        return time.perf_counter() - t0 >= budget_s

    if cfg == "fused_chain":
        wl = workloads.gen_fused_chain(seed=0, n=N_ELEMS)
        fb = traffic.fused_chain_bytes(wl.ops)
        n, t0 = 0, time.perf_counter()
        while True:
            out = oracle.run(wl)
            n += 1
            if over(t0) or n >= 200:
                break
        el = time.perf_counter() - t0
        return {"value": round(n * fb / el / 1e9, 3), "unit": "GB/s",
                "sample": f"{n} passes of the 16,777,216-element relu(a*x+b) chain, op by op (3 numpy "
                          f"passes each), {el:.1f} s", "_y": out["y"]}
    if cfg == "elementwise_queue":
        wl = workloads.gen_elementwise_queue(seed=0)
        n, t0 = 0, time.perf_counter()
        while True:
            oracle.run(wl)
            n += 1
            if over(t0):
                break
        el = time.perf_counter() - t0
        return {"value": round(n * len(wl.ops) / el), "unit": "ops/s",
                "gb_per_s": round(n * wl.meta["bytes"] / el / 1e9, 3),
                "sample": f"{n} whole 1,000-op queues, {el:.1f} s"}
    if cfg == "decode":
        wl = workloads.gen_decode(seed=0)
        per = wl.meta["ops_per_token"]
        byt = wl.meta["weight_bytes"] + wl.meta["kv_bytes"]
        cache = oracle.WeightCache.for_workload(wl)
        bufs, n, t0 = None, 0, time.perf_counter()
        while n < wl.meta["tokens"]:
            bufs = oracle.run(wl, upto=(n + 1) * per, buffers=bufs, start=n * per, wcache=cache)
            n += 1
            if over(t0):
                break
        el = time.perf_counter() - t0
        return {"value": round(n / el, 3), "unit": "tok/s", "ops_per_s": round(n * per / el),
                "gb_per_s": round(n * byt / el / 1e9, 3),
                "sample": f"the first {n} tokens of the 64-token decode ({n * per} ops, weights widened "
                          f"to fp64 once and reused), {el:.1f} s"}
    if cfg == "dynamic_dag":
        wl = workloads.gen_dynamic_dag(seed=0)
        ob = wl.meta["out_len"]
        bufs, n, byt, t0 = None, 0, 0, time.perf_counter()
        step = 250
        while n < len(wl.ops):
            bufs = oracle.run(wl, upto=n + step, buffers=bufs, start=n)
            for i in range(n, min(n + step, len(wl.ops))):
                op = wl.ops[i]
                byt += 4 * (op.n * len(op.ins) + ob[i])
            n = min(n + step, len(wl.ops))
            if over(t0):
                break
        el = time.perf_counter() - t0
        return {"value": round(n / el), "unit": "ops/s", "gb_per_s": round(byt / el / 1e9, 3),
                "sample": f"the first {n} of the 100,000 ops, {el:.1f} s"}
    if cfg == "priority_mix":
        wl = workloads.gen_priority_mix(seed=0)
        per = 1 + wl.meta["lc_per_round"]
        bufs, n, byt, t0 = None, 0, 0, time.perf_counter()
        while n < wl.meta["rounds"]:
            bufs = oracle.run(wl, upto=(n + 1) * per, buffers=bufs, start=n * per)
            byt += sum(traffic.op_bytes(op) for op in wl.ops[n * per:(n + 1) * per])
            n += 1
            if over(t0):
                break
        el = time.perf_counter() - t0
        return {"value": round(byt / el / 1e9, 3), "unit": "GB/s", "ops_per_s": round(n * per / el),
                "sample": f"the first {n} of the 200 rounds ({n} best-effort and {n * (per - 1)} "
                          f"latency-critical ops), {el:.1f} s"}
    raise ValueError(cfg)


def cpu_child_main(cfg, budget_s, core, y_path):
    """Entry of the child process: pin, run the sample, print one JSON line."""
    os.sched_setaffinity(0, {core})
    res = _oracle_sample(cfg, budget_s)
    y = res.pop("_y", None)
    if y is not None and y_path:
        import numpy as np

        np.save(y_path, y)
    print(json.dumps(res), flush=True)


def cpu_baseline(cfg, budget_s, gpu_y=None):
    """The oracle on a bounded sample of config `cfg`, in a child process
    pinned to one core with one BLAS / OpenMP thread."""
    import tempfile

    core = sorted(os.sched_getaffinity(0))[0]
    env = dict(os.environ)
    for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS",
              "NUMEXPR_NUM_THREADS", "VECLIB_MAXIMUM_THREADS"):
        env[k] = "1"
    y_path = None
    if gpu_y is not None:
        fd, y_path = tempfile.mkstemp(suffix=".npy")
        os.close(fd)
    try:
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-child", cfg,
                            "--cpu-budget", str(budget_s), "--cpu-core", str(core),
                            "--cpu-y", y_path or ""],
                           env=env, capture_output=True, text=True, timeout=max(300, 10 * budget_s))
        if r.returncode != 0:
            raise RuntimeError(f"oracle child for {cfg} failed:\n{r.stderr[-2000:]}")
        res = json.loads(r.stdout.strip().splitlines()[-1])
        parity = None
        if gpu_y is not None:
            import numpy as np

            import oracle

            parity = oracle.compare(gpu_y, np.load(y_path), "f32").ok
    finally:
        if y_path:
            os.unlink(y_path)
    res.update({"cores": 1, "kind": "oracle", "threads": 1, "pinned_core": core, **_cpu_info()})
    res["sample"] += ", one thread pinned to one core"
    return res, parity


def traffic_per_launch(passes):
    """HBM bytes of one fused-chain launch from the committed counter summary,
    or None when the kernel sources have changed since the counters were
    taken (or none were taken)."""
    import hashlib

    path = os.path.join(ROOT, "profiles", "gpuos_resident_fused_chain_16M_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].strip().split(": ", 1)
                fields[k.strip("`")] = v.strip().strip("`")
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "persistent_fusion_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    if fields.get("kernel_sources_sha256") != h.hexdigest():
        return None
    try:
        return int(round(float(fields["hbm_bytes_per_pass"]) * passes))
    except (KeyError, ValueError):
        return None


def _frac(gbs):
    return round(gbs / HBM_PEAK_GBS, 4)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--device-warmup-s", type=float, default=0.5,
                    help="the fused chain's warm-up continues until this many seconds have passed")
    ap.add_argument("--queue-reps", type=int, default=50)
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle work for the headline's CPU baseline (other configs: "
                         "proportionally less)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-launch-rate", action="store_true",
                    help="leave out the launch-rate measurement (20,000 empty-kernel launches), e.g. "
                         "under a profiler that serialises every dispatch")
    ap.add_argument("--configs", default="all",
                    help="comma-separated configs besides the headline: queue, decode, dag, priority (or all)")
    ap.add_argument("--extra", default="",
                    help="comma-separated extra legs: torch, program, views (or all)")
    ap.add_argument("--cpu-child", default="", help=argparse.SUPPRESS)
    ap.add_argument("--cpu-core", type=int, default=0, help=argparse.SUPPRESS)
    ap.add_argument("--cpu-y", default="", help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.cpu_child:
        cpu_child_main(args.cpu_child, args.cpu_budget, args.cpu_core, args.cpu_y)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only (the resident kernel runs on one "
              "device; --gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.synchronize()
    fc = fused_chain_leg(args.steps, args.warmup, warm_s=args.device_warmup_s)
    log("bench: copy kernel reference")
    cp = copy_leg()
    lr = None
    if not args.no_launch_rate:
        log("bench: launch rate (empty kernel)")
        lr = launch_rate_leg()
    names = ("queue", "decode", "dag", "priority") if args.configs == "all" else \
        tuple(x for x in args.configs.split(",") if x)
    cfgs = {}
    for name in names:
        log(f"bench: config {name}")
        if name == "queue":
            cfgs["C1_elementwise_queue_1000x4096"] = queue_leg(args.queue_reps)
        elif name == "decode":
            cfgs["C3_decode_24_layers_64_tokens"] = decode_leg()
        elif name == "dag":
            cfgs["C4_dynamic_dag_100000_ops"] = dag_leg()
        elif name == "priority":
            cfgs["C5_priority_mix_200_rounds"] = priority_leg()
        else:
            raise SystemExit(f"unknown config {name}")
    c3 = cfgs.get("C3_decode_24_layers_64_tokens")
    if c3 and c3.get("resident_device_span_ms") and lr:
        # the pages' launch-cost model with this GPU's figures: every op of a
        # token launched on its own, each costing the measured host time of a
        # back-to-back launch, on top of the resident kernel's device time
        from persistent_fusion_amd import traffic

        per_tok = c3["ops"] // c3["tokens"]
        comp = c3["resident_device_span_ms"] * 1e-3 / c3["tokens"]
        m = traffic.launch_model(per_tok, lr["us_per_launch_back_to_back"] * 1e-6, comp)
        c3["launch_model"] = {
            "launches_per_token": per_tok, "us_per_launch": lr["us_per_launch_back_to_back"],
            "compute_us_per_token": round(comp * 1e6, 1),
            "modelled_per_op_launch_us_per_token": round(m["total_s"] * 1e6, 1),
            "measured_per_op_launch_us_per_token": round(1e6 / c3["per_op_launch_tok_per_s"], 1),
            "launch_share": round(m["share"], 3)}
    extra_names = ("torch", "program", "views") if args.extra == "all" else \
        tuple(x for x in args.extra.split(",") if x)
    extra = {}
    for name in extra_names:
        log(f"bench: extra leg {name}")
        extra[name] = {"torch": torch_frontend_leg, "program": program_leg, "views": views_leg}[name]()
    cpu, parity = None, None
    if not args.no_cpu:
        log("bench: CPU oracle baselines")
        cpu, parity = cpu_baseline("fused_chain", args.cpu_budget, fc["y"])
        share = {"C1_elementwise_queue_1000x4096": ("elementwise_queue", 0.3),
                 "C3_decode_24_layers_64_tokens": ("decode", 1.5),
                 "C4_dynamic_dag_100000_ops": ("dynamic_dag", 0.8),
                 "C5_priority_mix_200_rounds": ("priority_mix", 0.8)}
        for key, res in cfgs.items():
            which, f = share[key]
            res["cpu_baseline"], _ = cpu_baseline(which, max(2.0, f * args.cpu_budget))

    steps = args.steps
    value = steps * fc["fused_bytes"] / fc["wall_s"] / 1e9
    passes = fc["warmup_passes"] + steps
    launch_bytes = passes * fc["fused_bytes"]
    achieved = launch_bytes / fc["kernel_s"] / 1e9
    tr = traffic_per_launch(passes)
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(fc["wall_s"] / steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "fused chain y=relu(a*x+b), 16,777,216 fp32 elements, 3 descriptors "
                               "fused into 1 pass, 4 rotating replicas",
                   "elements": N_ELEMS, "descriptors_per_step": 3},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": tr,
                     "traffic_source": (f"profiles/gpuos_resident_fused_chain_16M_traffic.md: calibrated "
                                        f"FETCH_SIZE + WRITE_SIZE per pass x {passes} passes (counters "
                                        f"taken in a separate run of the same kernel sources)")
                     if tr is not None else None,
                     "kernel": "gpuos_resident", "passes_per_launch": passes,
                     "device_warmup_passes": fc["warmup_passes"],
                     "bytes_per_launch": launch_bytes,
                     "launch_s_hip_events": round(fc["kernel_s"], 6)},
        "ops_per_s": round(3 * steps / fc["wall_s"]),
        "parity_last_pass_bit_exact": parity,
        "device_span_gb_per_s": (round(steps * fc["fused_bytes"] / fc["dev_span_s"] / 1e9, 1)
                                 if fc["dev_span_s"] else None),
        "median_pass_device_us": (round(fc["per_pass_dev_us"], 2) if fc["per_pass_dev_us"] else None),
        "per_op_launch": fc["baselines"]["per_op_launch"],
        "standalone_fused_kernel": fc["baselines"]["standalone_fused_kernel"],
        "graph_replay": fc["baselines"]["graph_replay"],
        "graph_replay_fused": fc["baselines"]["graph_replay_fused"],
        "plain_copy_kernel": cp,
        "launch_overhead": lr,
        "configs": cfgs,
        **({"extra_configs": extra} if extra else {}),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
