"""The C ABI's argument checks under AddressSanitizer and
UndefinedBehaviorSanitizer, on the host: a copy of the library is built with
both sanitizers on its host code only (device code unchanged), and
tests/host/abi_sanitize.cpp, built with the same sanitizers, calls every
entry point with arguments its checks must refuse before any GPU work. A
sanitizer report aborts the program; a wrong status code fails it. Nothing
runs on a GPU."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.timeout(600)
def test_abi_checks_under_host_sanitizers(tmp_path):
    from weight_only_int4_quantize_amd import build as b

    clang = "/opt/rocm/llvm/bin/clang++"
    if not os.path.exists(clang) or shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("ROCm toolchain not available")
    lib = b.build(extra_flags=SAN, out_path=str(tmp_path / "libawq_san.so"), obj_dir=str(tmp_path / "obj"))
    exe = tmp_path / "abi_sanitize"
    src = os.path.join(HERE, "host", "abi_sanitize.cpp")
    r = subprocess.run([clang, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                        "-fno-omit-frame-pointer", src, lib, f"-Wl,-rpath,{tmp_path}", "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert out.returncode == 0 and out.stdout.strip().endswith("ok"), (out.stdout + out.stderr)[-4000:]
