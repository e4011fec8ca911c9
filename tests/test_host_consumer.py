"""The host runtime under a concurrent consumer, built with the sanitizers.

``tests/native/host_consumer.cpp`` runs the runtime's submit / flush / sync
path on a host-only context while a second thread plays the resident kernel
on the same ring protocol: it follows the published tails, runs descriptors
whose published dependencies have run, in random order, and retires each ring
in order.  The ring is small, so it fills and wraps and the producer blocks on
back-pressure; a tenth of the ops go to the latency-critical ring, so byte-range
hazards across the two rings are waited for on the host.  The buffers' final
contents must equal the oracle's program-order run of the same queue, element
for element (int32 ADD / MUL / COPY are exact).

The runtime and the C++ test program are compiled from source with g++ under
AddressSanitizer + UndefinedBehaviorSanitizer, and under ThreadSanitizer (the
consumer shares the ring, the tails and the retire cursors with the producer).
They are linked with the library's kernel objects, which a host-only context
never launches.  Everything here runs on the CPU.
"""

from __future__ import annotations

import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from persistent_fusion_amd.workloads import Op, Ref, Workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OBJDIR = os.path.join(ROOT, "_build")
CSRC = os.path.join(ROOT, "persistent_fusion_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "native", "host_consumer.cpp")
KERNEL_OBJS = ["kernels.o", "single_kernel.o", "static_scratch.o", "rtc_sources.o"]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

SANITIZERS = {
    "asan_ubsan": ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                   "-fno-omit-frame-pointer"],
    "tsan": ["-fsanitize=thread"],
}

B, L = 6, 4096


def _compile(kind: str, outdir: str) -> str:
    if shutil.which("g++") is None:
        pytest.skip("g++ is not installed")
    objs = [os.path.join(OBJDIR, o) for o in KERNEL_OBJS]
    missing = [o for o in objs if not os.path.exists(o)]
    assert not missing, f"build the library first (__graft_entry__.build()): missing {missing}"
    flags = ["-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
             *SANITIZERS[kind]]
    exe = os.path.join(outdir, f"host_consumer_{kind}")
    units = []
    for src in (os.path.join(CSRC, "runtime.cpp"), DRIVER):
        obj = os.path.join(outdir, f"{kind}_{os.path.basename(src)}.o")
        r = subprocess.run(["g++", *flags, "-c", "-o", obj, src], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        units.append(obj)
    link = ["g++", *SANITIZERS[kind], "-o", exe, *units, *objs, f"-L{ROCM}/lib", "-lamdhip64",
            "-lhiprtc", f"-Wl,-rpath,{ROCM}/lib", "-lpthread"]
    r = subprocess.run(link, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return exe


@pytest.fixture(scope="module")
def drivers(tmp_path_factory):
    d = str(tmp_path_factory.mktemp("host_consumer"))
    return {k: _compile(k, d) for k in SANITIZERS}


def gen_queue(seed: int, n_ops: int, lc_frac: float = 0.1):
    """int32 ADD / MUL / COPY over ranges of B buffers of L elements: random
    extents (1..1024, log-uniform) at random offsets, so ranges overlap
    partially; an output is either exactly its first input (in place) or
    disjoint from every input of its op."""
    rng = np.random.default_rng(seed)
    init = rng.integers(-(1 << 31), 1 << 31, size=(B, L), dtype=np.int64).astype(np.int32)
    ops = []
    for _ in range(n_ops):
        kind = int(rng.integers(0, 3))
        n = int(np.exp(rng.uniform(0, np.log(1024)))) or 1
        lc = bool(rng.random() < lc_frac)

        def rnd():
            return int(rng.integers(0, B)), int(rng.integers(0, L - n + 1))

        i0, i1 = rnd(), rnd()
        if rng.random() < 0.15:
            o = i0
            while kind != 2 and i1[0] == o[0] and not (o[1] + n <= i1[1] or i1[1] + n <= o[1]):
                i1 = rnd()
        else:
            while True:
                o = rnd()
                if all(o[0] != b or o[1] + n <= off or off + n <= o[1] for b, off in (i0, i1)):
                    break
        ops.append((kind, int(lc), o[0], o[1], i0[0], i0[1], i1[0], i1[1], n))
    return init, ops


def write_inputs(tmp, init, ops):
    opsf, initf, outf = (os.path.join(tmp, x) for x in ("ops.txt", "init.bin", "out.bin"))
    with open(opsf, "w") as f:
        f.write(f"buffers {B} {L}\n")
        for o in ops:
            f.write("op " + " ".join(str(v) for v in o) + "\n")
    init.astype("<i4").tofile(initf)
    return opsf, initf, outf


def oracle_final(init, ops):
    kinds = ("add", "mul", "copy")
    bufs = {f"b{i}": init[i].copy() for i in range(B)}
    wops = []
    for kind, lc, ob, oo, b0, o0, b1, o1, n in ops:
        ins = (Ref(f"b{b0}", o0),) if kind == 2 else (Ref(f"b{b0}", o0), Ref(f"b{b1}", o1))
        wops.append(Op(kinds[kind], Ref(f"b{ob}", oo), ins, n=n, dtype="i32", lc=bool(lc)))
    wl = Workload("host_consumer", bufs, {k: "i32" for k in bufs}, wops)
    out = oracle.run(wl)
    return np.stack([out[f"b{i}"] for i in range(B)])


def run_driver(exe, tmp, init, ops, slots, batch, flush_every, seed, auto_deps=1):
    opsf, initf, outf = write_inputs(tmp, init, ops)
    env = dict(os.environ)
    # the HIP runtime library is not built with the sanitizers; its one-time
    # allocations at load are not the runtime's leaks
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["TSAN_OPTIONS"] = "halt_on_error=1:second_deadlock_stack=1"
    r = subprocess.run([exe, opsf, initf, outf, str(slots), str(batch), str(flush_every), str(seed),
                        str(auto_deps)], capture_output=True, text=True, env=env, timeout=240)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-6000:])
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-6000:]
    assert "WARNING: ThreadSanitizer" not in r.stderr, r.stderr[-6000:]
    stats = dict(zip(r.stdout.split()[0::2], r.stdout.split()[1::2]))
    got = np.fromfile(outf, dtype="<i4").reshape(B, L)
    return got, r.stdout, stats


@pytest.mark.parametrize("kind", sorted(SANITIZERS))
@pytest.mark.parametrize("slots,batch,flush_every,seed,lc_frac", [
    (64, 1, 1, 1, 0.0),     # one op per flush: the ring wraps every 64 ops
    (64, 7, 3, 2, 0.0),     # flushes of 21 ops, ragged against the ring
    (64, 200, 1, 3, 0.0),   # flushes larger than the ring: publication blocks mid-flush
    (256, 64, 2, 4, 0.1),   # both rings: cross-ring hazards wait on the host
    (64, 7, 1, 6, 0.1),
])
def test_consumer_matches_oracle(drivers, tmp_path, kind, slots, batch, flush_every, seed, lc_frac):
    init, ops = gen_queue(seed, 1500 if kind == "tsan" else 3000, lc_frac)
    want = oracle_final(init, ops)
    got, line, st = run_driver(drivers[kind], str(tmp_path), init, ops, slots, batch, flush_every, seed)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} elements differ, first {bad[:5].tolist()}; {line}"
    # the schedule really ran out of order under published dependencies
    assert int(st["out_of_order"]) > 0 and int(st["deps"]) > 0, line
    ran_lc = int(st["+"])
    if lc_frac:
        assert ran_lc > 0, line
    else:
        # one ring, kept busy: the producer waited for ring space
        assert ran_lc == 0 and int(st["ring_full_waits"]) > 0, line


def test_consumer_without_dependencies_diverges(drivers, tmp_path):
    """With the hazard dependencies off, the out-of-order consumer breaks
    program order and the comparison catches it: the test above has teeth."""
    init, ops = gen_queue(5, 3000, lc_frac=0.0)
    want = oracle_final(init, ops)
    got, line, _ = run_driver(drivers["asan_ubsan"], str(tmp_path), init, ops, 64, 16, 1, 5, auto_deps=2)
    assert (got != want).any(), line
