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


def _fake_tree(tmp_path, sha, per_pass="268563935"):
    """A tree holding the kernel sources and a traffic profile that records
    the kernel-source hash `sha`."""
    fake = tmp_path / "persistent_fusion_amd" / "csrc"
    fake.mkdir(parents=True)
    for name in bench.KERNEL_SOURCES:
        shutil.copy(os.path.join(ROOT, "persistent_fusion_amd", "csrc", name), fake / name)
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "gpuos_resident_fused_chain_16M_traffic.md").write_text(
        f"# traffic\n\n- kernel_sources_sha256: `{sha}`\n- hbm_bytes_per_pass: `{per_pass}`\n")
    return fake


def _sources_sha():
    import hashlib

    h = hashlib.sha256()
    for name in bench.KERNEL_SOURCES:
        with open(os.path.join(ROOT, "persistent_fusion_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def test_traffic_is_reported_for_the_profiled_kernel_only(tmp_path, monkeypatch):
    fake = _fake_tree(tmp_path, _sources_sha())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_per_launch(1500) == 1500 * 268_563_935
    # the same profile against edited kernel sources: no traffic
    (fake / bench.KERNEL_SOURCES[0]).write_text((fake / bench.KERNEL_SOURCES[0]).read_text() + "\n// edited\n")
    assert bench.traffic_per_launch(1500) is None


def test_committed_profile_is_read_when_current():
    """The committed counter summary is used exactly when it records the
    hash of the kernel sources in the tree."""
    path = os.path.join(ROOT, "profiles", "gpuos_resident_fused_chain_16M_traffic.md")
    text = open(path).read()
    per_launch = bench.traffic_per_launch(1500)
    if _sources_sha() in text:
        assert isinstance(per_launch, int) and per_launch > 1500 * 268_435_456
    else:
        assert per_launch is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in r.stderr
