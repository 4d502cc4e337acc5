"""Host logic: the binade search grid of the encode kernel (built by csrc/tables.cpp), checked
exhaustively over every fp32 value of the grid's domain [2, 4) by a small C++ program linked
against the library's own table code (no GPU)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "kv_cache_transform_amd", "csrc")
CXX = "/opt/rocm/llvm/bin/clang++"   # the host compiler with _Float16 support


@pytest.mark.skipif(not os.path.exists(CXX) and shutil.which("clang++") is None, reason="no clang++")
def test_binade_grid_exhaustive(tmp_path):
    cxx = CXX if os.path.exists(CXX) else shutil.which("clang++")
    exe = str(tmp_path / "host_grid_check")
    subprocess.run([cxx, "-O2", "-std=c++17", "-I", CSRC, os.path.join(HERE, "host_grid_check.cpp"),
                    os.path.join(CSRC, "tables.cpp"), "-o", exe], check=True, capture_output=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
    # the benchmark's codebooks (d = 128 with b = 3, 4) must take the binade grid
    assert "d=128 b=4: index mismatches 0, centroid-row mismatches 0" in r.stdout
    assert "d=128 b=3: index mismatches 0, centroid-row mismatches 0" in r.stdout
