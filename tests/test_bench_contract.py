"""Host-side checks of bench.py's contract: the multi-GPU refusal and the rule that the recorded
HBM traffic is reported only while the counted kernel sources are unchanged."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

WORKLOAD = "llama8b-32k-block-router"
COUNTED = ("attn_bf16.hip", "elastic_internal.hpp", "plan.hip")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "not supported" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line is printed


def _copy_tree(tmp_path):
    csrc = tmp_path / "hybrid_sparse_full_elastic_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name in COUNTED:
        shutil.copy(os.path.join(ROOT, "hybrid_sparse_full_elastic_amd", "csrc", name), csrc / name)
    prof = tmp_path / "profiles"
    prof.mkdir()
    src = os.path.join(ROOT, "profiles", f"attn_bf16_kernel-{WORKLOAD}.pmc.txt")
    shutil.copy(src, prof / os.path.basename(src))
    return csrc


def _committed_bytes():
    path = os.path.join(ROOT, "profiles", f"attn_bf16_kernel-{WORKLOAD}.pmc.txt")
    for line in open(path):
        if line.startswith("traffic_bytes_per_launch: "):
            return int(float(line.split(": ", 1)[1]))
    raise AssertionError("no traffic line in the counter summary")


def test_traffic_follows_the_source_hash(tmp_path, monkeypatch):
    csrc = _copy_tree(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    got = bench.recorded_traffic(WORKLOAD)
    if got is None:
        pytest.skip("the counted sources changed since the counters were taken")
    assert got == _committed_bytes()
    # any edit of a counted source voids the figure
    with open(csrc / "plan.hip", "a") as f:
        f.write("\n")
    assert bench.recorded_traffic(WORKLOAD) is None


def test_missing_counter_summary_gives_none(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.recorded_traffic("no-such-workload") is None
