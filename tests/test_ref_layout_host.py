"""The tiled layout of the searches' fp32 reference output, checked on the
host: tests/host/ref_layout_check.cpp includes the library's internal header
and verifies that the layout is a bijection onto its padded buffer and that
each lane's 16 accumulator values of a sub-tile are contiguous. Built with
hipcc as host code (nothing runs on a GPU)."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_reference_layout_is_a_bijection(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = tmp_path / "ref_layout_check"
    src = os.path.join(HERE, "host", "ref_layout_check.cpp")
    r = subprocess.run([hipcc, "-x", "hip", "--offload-arch=gfx950", "-O2", "-std=c++17", src, "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout + out.stderr
