"""Builds libgpuos.so in-tree with hipcc for gfx950."""

from __future__ import annotations

import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgpuos.so")
# Each kernel is its own translation unit; the units compile in parallel and
# are linked into one shared library.
SOURCES = ["kernels.hip", "single_kernel.hip", "static_scratch.hip", "runtime.cpp"]
OBJDIR = os.path.join(os.path.dirname(HERE), "_build")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # exact-class ops must be single IEEE operations: no a*b+c contraction
    "-ffp-contract=off",
    # keep fp32 subnormals (no flush to zero)
    "-fno-gpu-flush-denormals-to-zero",
    # no packed fp32 instructions are generated
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


# The resident kernel is launched with 8 waves per CU by default (2 per
# SIMD): it must keep that occupancy and use no scratch memory.
MIN_WAVES_PER_SIMD = 2


def kernel_resources(stderr: str) -> dict:
    """Per-kernel resource usage from the compiler's resource-usage remarks."""
    res, cur = {}, None
    pat = re.compile(r"remark:\s+(.*?):\s+(\S+) \[-Rpass-analysis=kernel-resource-usage\]")
    for line in stderr.splitlines():
        m = pat.search(line)
        if not m:
            continue
        key, val = m.group(1).strip(), m.group(2)
        if key == "Function Name":
            cur = res.setdefault(val, {})
        elif cur is not None:
            cur[key] = val
    return res


def _filter(stderr: str):
    return [l for l in stderr.splitlines()
            if "packed-fp32-ops" not in l and "kernel-resource-usage" not in l and l.strip()
            and not l.strip().startswith(("|", "^")) and not l[:8].strip().isdigit()]


def build(verbose: bool = False, only=None) -> str:
    """Compiles every source (or, with `only`, just those sources, linking
    them with the objects already in _build/) and links libgpuos.so."""
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = []
    for src in SOURCES:
        obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
        if only is not None and src not in only:
            if not os.path.exists(obj):
                raise RuntimeError(f"{obj} is missing: build everything first")
            jobs.append((src, obj, None))
            continue
        cmd = [hipcc(), *FLAGS, "-c", "-Rpass-analysis=kernel-resource-usage", "-o", obj,
               os.path.join(CSRC, src)]
        if verbose:
            print(" ".join(cmd), flush=True)
        jobs.append((src, obj, subprocess.Popen(cmd, cwd=CSRC, stdout=subprocess.PIPE,
                                                stderr=subprocess.PIPE, text=True)))
    res, errs = {}, []
    for src, obj, p in jobs:
        if p is None:
            continue
        _, err = p.communicate()
        if p.returncode != 0:
            errs.append(f"{src}:\n" + "\n".join(_filter(err)))
        res.update(kernel_resources(err))
    if errs:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
    for name, k in res.items():
        if "gpuos_resident" not in name and "gpuos_single" not in name:
            continue
        waves = int(k.get("Occupancy [waves/SIMD]", "0"))
        scratch = int(k.get("ScratchSize [bytes/lane]", "0"))
        if verbose:
            print(f"{name}: VGPRs {k.get('VGPRs')} occupancy {waves} waves/SIMD scratch {scratch}",
                  flush=True)
        if waves < MIN_WAVES_PER_SIMD or scratch:
            raise RuntimeError(f"{name}: {k.get('VGPRs')} VGPRs, {waves} waves/SIMD, "
                               f"{scratch} B scratch: below {MIN_WAVES_PER_SIMD} waves/SIMD "
                               "or using scratch")
    tmp = LIB + ".tmp"
    link = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + \
        [obj for _, obj, _ in jobs]
    r = subprocess.run(link, cwd=CSRC, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
