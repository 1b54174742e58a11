"""Builds libawq_mi355x.so (all HIP sources, gfx950) in the package folder.

    python -m weight_only_int4_quantize_amd.build
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_NAME = "libawq_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-function",
    # Packed fp32 VALU ops stay disabled (the compiler would otherwise emit
    # them from ordinary float code); packed fp16 is unaffected.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# Per-source flags. The decode kernels (GEMV, column tiles, skinny) are
# short and launched back to back, so a wave's first kernel-argument load
# sits on the critical path of every launch; the hardware preloads the
# arguments into SGPRs instead, as many as fit beside the argument pointer
# (14 dwords; the rest are loaded as usual). Measured on the GEMV (us, M = 1):
# 4096 x 4096 4.09 -> 3.83, 11008 x 4096 6.71 -> 6.30, 4096 x 11008
# 7.55 -> 7.18.
_PRELOAD = ["-mllvm", "-amdgpu-kernarg-preload-count=16"]
SOURCE_FLAGS = {"gemv.hip": _PRELOAD, "coltile.hip": _PRELOAD, "skinny.hip": _PRELOAD}


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build the library")
    return path


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)


def _finish(proc, verbose) -> None:
    out, err = proc.communicate()
    if proc.returncode != 0:
        sys.stderr.write(out + err)
        raise RuntimeError(f"hipcc failed with exit code {proc.returncode}")
    if verbose and err.strip():
        sys.stderr.write(err)


def build(verbose: bool = False, extra_flags=None, out_path: str = LIB_PATH, obj_dir: str = None) -> str:
    """Compile every HIP source (one hipcc process per translation unit, in
    parallel) and link them into one shared library; returns its path.
    extra_flags go to every compile and to the link (e.g. host-only
    sanitizers, each -fsanitize= after -Xarch_host); out_path and obj_dir
    place a variant build elsewhere."""
    obj_dir = obj_dir or os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"] + list(extra_flags or [])
    objs, procs = [], []
    jobs = max(1, min(len(sources()), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    for src in sources():
        obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
        objs.append(obj)
        flags = compile_flags + SOURCE_FLAGS.get(os.path.basename(src), [])
        procs.append(_run([hipcc(), *flags, "-c", src, "-o", obj], verbose))
        if len(procs) >= jobs:
            _finish(procs.pop(0), verbose)
    for p in procs:
        _finish(p, verbose)
    tmp = out_path + ".tmp"
    link = _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *list(extra_flags or []), *objs, "-o", tmp],
                verbose)
    _finish(link, verbose)
    os.replace(tmp, out_path)
    return out_path


if __name__ == "__main__":
    print(build(verbose=True))
