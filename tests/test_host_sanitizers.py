"""Host-side argument validation of the C ABI under AddressSanitizer and UBSan (CPU only).

The library is rebuilt with the sanitizers on its host code (device code unoptimised: no kernel
is launched) and ``abi_host_check.cpp`` calls every entry point with arguments the validation
must reject. A sanitizer report or an unexpected status fails the test.
"""
import os
import re
import shutil
import subprocess

import pytest

from eviction_long_reasoning_amd import build as kvbuild

HERE = os.path.dirname(os.path.abspath(__file__))
HARNESS = os.path.join(HERE, "abi_host_check.cpp")
CLANG = "/opt/rocm/llvm/bin/clang++"
SANITIZE = ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all")


def _declared_entry_points():
    text = open(os.path.join(kvbuild.INCLUDE, "kvevict.h")).read()
    return sorted(set(re.findall(r"^\S.*?\b([a-z_]+)\(", text, re.M)) - {"typedef"})


def test_harness_calls_every_entry_point():
    harness = open(HARNESS).read()
    missing = [n for n in _declared_entry_points() if not re.search(rf"\b{n}\(", harness)]
    assert not missing, f"host check does not call {missing}"


@pytest.mark.skipif(not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc"))
                    or not os.path.exists(CLANG), reason="ROCm compilers not installed")
def test_argument_validation_is_clean_under_sanitizers(tmp_path):
    out_dir = os.path.join(kvbuild.BUILD_DIR, "sanitize")
    os.makedirs(out_dir, exist_ok=True)
    lib = kvbuild.build(out=os.path.join(out_dir, "libkvevict_sanitize.so"), host_flags=SANITIZE,
                        tag="sanitize", device_flags=("-O0",))
    exe = str(tmp_path / "abi_host_check")
    r = subprocess.run([CLANG, "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer", *SANITIZE,
                        "-I", kvbuild.INCLUDE, HARNESS, "-o", exe, lib, f"-Wl,-rpath,{out_dir}"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and "host checks ok" in r.stdout, r.stdout + r.stderr
    assert "Sanitizer" not in r.stderr, r.stderr
