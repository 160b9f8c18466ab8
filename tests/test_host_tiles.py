"""Exhaustive host-side check of the key-tile schedule (compiled from the library's own
header with hipcc's host compiler; no GPU code runs)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_key_tile_schedule_covers_exactly(tmp_path):
    cc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cc):
        pytest.skip("hipcc not available")
    exe = tmp_path / "tiles_check"
    subprocess.run([cc, "-O2", "-std=c++17", "-x", "hip", "--offload-arch=gfx950",
                    os.path.join(HERE, "tiles_check.cpp"), "-o", str(exe)], check=True,
                   capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
