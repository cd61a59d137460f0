"""Build the HIP kernels and the C ABI into ``libkvevict.so`` (gfx950 only).

Every ``csrc/*.hip`` file is compiled with hipcc for ``--offload-arch=gfx950``
into ``_build/kvevict/`` at the repository root and linked into a shared
library placed next to this file, where the Python binding loads it.
Packed-fp32 instruction selection is disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build", "kvevict")
LIB_NAME = "libkvevict.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

COMPILE_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _hipcc() -> str:
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found; ROCm is required to build the kernels")
    return h


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, jobs: int = 8, out: str = LIB_PATH, defines=(), host_flags=(),
          tag: str = "", device_flags=()) -> str:
    """Compile every kernel source and link ``libkvevict.so`` (or ``out``); returns its path.

    ``defines`` are extra ``NAME=VALUE`` preprocessor definitions (tuning knobs such as
    KV_SCORE_BATCHES_PER_WAVE); the default build uses none. ``host_flags`` apply to the host
    compilation and the link only (each is passed as ``-Xarch_host <flag>``), for
    instance a sanitizer for the host-side argument checks; ``tag`` names their object folder.
    ``device_flags`` likewise apply to the device compilation only (``-Xarch_device <flag>``);
    ``("-O0",)`` gives a quick build for host-side checks that launch no kernel.
    """
    hipcc = _hipcc()
    sub = "_".join([d.replace("=", "") for d in defines] + ([tag] if tag else []))
    bdir = BUILD_DIR if not sub else os.path.join(BUILD_DIR, sub)
    os.makedirs(bdir, exist_ok=True)
    srcs = sources()
    dflags = [f"-D{d}" for d in defines]
    hflags = [x for f in host_flags for x in ("-Xarch_host", f)]
    xflags = [x for f in device_flags for x in ("-Xarch_device", f)]

    def compile_one(src):
        obj = os.path.join(bdir, os.path.basename(src)[:-4] + ".o")
        cmd = [hipcc, *COMPILE_FLAGS, *dflags, *hflags, *xflags, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        if verbose and r.stderr.strip():
            sys.stderr.write(r.stderr)
        return obj

    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = out + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *hflags, "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
