"""Host checks of the measurement code: the committed traffic profile is used
only while it belongs to the kernel sources in the tree, and more than one
GPU is refused."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_traffic_is_reported_for_the_profiled_kernel_only(tmp_path, monkeypatch):
    per_launch = bench.traffic_per_launch(1500)
    assert isinstance(per_launch, int) and per_launch > 1500 * 268_435_456  # at least the algorithmic bytes
    # the same profile against different kernel sources: no traffic
    fake = tmp_path / "persistent_fusion_amd" / "csrc"
    fake.mkdir(parents=True)
    for name in bench.KERNEL_SOURCES:
        shutil.copy(os.path.join(ROOT, "persistent_fusion_amd", "csrc", name), fake / name)
    (fake / bench.KERNEL_SOURCES[0]).write_text((fake / bench.KERNEL_SOURCES[0]).read_text() + "\n// edited\n")
    (tmp_path / "profiles").mkdir()
    shutil.copy(os.path.join(ROOT, "profiles", "gpuos_resident_fused_chain_16M_traffic.md"), tmp_path / "profiles")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_per_launch(1500) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in r.stderr
