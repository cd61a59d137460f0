"""Build the HIP kernels and the C ABI into ``libkvevict.so`` (gfx950 only).

Every ``csrc/*.hip`` file is compiled with hipcc for ``--offload-arch=gfx950``
into ``_build/kvevict/`` at the repository root and linked into a shared
library placed next to this file, where the Python binding loads it.
Packed-fp32 instruction selection is disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import hashlib
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
DEBUG_LIB_PATH = os.path.join(PKG, "libkvevict_debug.so")
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


def _headers():
    return sorted(glob.glob(os.path.join(CSRC, "*.hpp")) + glob.glob(os.path.join(INCLUDE, "*.h")))


def build(verbose: bool = False, jobs: int = 8, out: str = LIB_PATH, defines=(), host_flags=(),
          tag: str = "", device_flags=(), force: bool = True) -> str:
    """Compile every kernel source and link ``libkvevict.so`` (or ``out``); returns its path.

    ``defines`` are extra ``NAME=VALUE`` preprocessor definitions (tuning knobs such as
    KV_SCORE_BATCHES_PER_WAVE); the default build uses none. ``host_flags`` apply to the host
    compilation and the link only (each is passed as ``-Xarch_host <flag>``), for
    instance a sanitizer for the host-side argument checks; ``tag`` names their object folder.
    ``device_flags`` likewise apply to the device compilation only (``-Xarch_device <flag>``);
    ``("-O0",)`` gives a quick build for host-side checks that launch no kernel.
    ``force=False`` reuses an object whose source, headers and flags are unchanged since it was
    compiled (a stamp beside it records their hash); the default recompiles everything.
    """
    hipcc = _hipcc()
    sub = "_".join([d.replace("=", "") for d in defines] + ([tag] if tag else []))
    bdir = BUILD_DIR if not sub else os.path.join(BUILD_DIR, sub)
    os.makedirs(bdir, exist_ok=True)
    srcs = sources()
    dflags = [f"-D{d}" for d in defines]
    hflags = [x for f in host_flags for x in ("-Xarch_host", f)]
    xflags = [x for f in device_flags for x in ("-Xarch_device", f)]

    hdr = hashlib.sha256()
    for f in _headers():
        hdr.update(open(f, "rb").read())

    def compile_one(src):
        obj = os.path.join(bdir, os.path.basename(src)[:-4] + ".o")
        cmd = [hipcc, *COMPILE_FLAGS, *dflags, *hflags, *xflags, "-c", src, "-o", obj]
        h = hdr.copy()
        h.update(open(src, "rb").read())
        h.update(" ".join(cmd).encode())
        stamp = obj + ".sha256"
        if not force and os.path.exists(obj) and os.path.exists(stamp) and open(stamp).read() == h.hexdigest():
            return obj
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        if verbose and r.stderr.strip():
            sys.stderr.write(r.stderr)
        with open(stamp, "w") as f:
            f.write(h.hexdigest())
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


def build_debug(verbose: bool = False) -> str:
    """``libkvevict_debug.so``: the release objects with ``api.hip`` rebuilt with KV_DEVICE_CHECKS=1,
    so every call first checks its device-side preconditions into the workspace status word.
    Run after ``build()`` (it links the release objects from the same folder)."""
    hipcc = _hipcc()
    srcs = sources()
    objs = [os.path.join(BUILD_DIR, os.path.basename(src)[:-4] + ".o") for src in srcs]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"release objects missing ({missing}): run build() first")
    ddir = os.path.join(BUILD_DIR, "device_checks")
    os.makedirs(ddir, exist_ok=True)
    api_src = os.path.join(CSRC, "api.hip")
    api_obj = os.path.join(ddir, "api.o")
    cmd = [hipcc, *COMPILE_FLAGS, "-DKV_DEVICE_CHECKS=1", "-c", api_src, "-o", api_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {api_src}:\n{r.stderr}")
    if verbose and r.stderr.strip():
        sys.stderr.write(r.stderr)
    objs = [api_obj if o.endswith(os.sep + "api.o") else o for o in objs]
    tmp = DEBUG_LIB_PATH + ".tmp"
    r = subprocess.run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, DEBUG_LIB_PATH)
    return DEBUG_LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True, force="--incremental" not in sys.argv))
    print(build_debug(verbose=True))
