"""Pins for the oracle's Philox4x32-10 (CPU only).

The oracle's generator is compared with rocRAND's Philox4x32-10, an
independent library implementation of the same published generator, compiled
as a host program from rocRAND's header (it is host-callable). Counter words
the oracle uses map onto rocRAND's (subsequence, offset) arguments as
ctr = (offset/4 low, offset/4 high, subsequence low, subsequence high).
"""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

from oracle import philox4x32_10, philox4x32_10_np
from workloads import rng

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_ref():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand/rocrand_kernel.h"):
        pytest.skip("hipcc / rocRAND headers not available")
    d = tempfile.mkdtemp(prefix="philox_ref_")
    exe = os.path.join(d, "ref")
    subprocess.run([hipcc, "-O1", "-o", exe, os.path.join(HERE, "rocrand_philox_ref.cpp")],
                   check=True, capture_output=True)
    yield exe
    shutil.rmtree(d, ignore_errors=True)


def _ref(exe, triples):
    inp = "\n".join(f"{s} {b} {o}" for s, b, o in triples) + "\n"
    out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
    return [tuple(int(x) for x in line.split()) for line in out.strip().splitlines()]


def test_philox_matches_rocrand(rocrand_ref):
    r = rng(300)
    triples = [(0, 0, 0), (2 ** 64 - 1, 2 ** 64 - 1, 0), (0x299F31D0A4093822, 0, 0)]
    for _ in range(60):
        seed = int(r.integers(0, 2 ** 63)) * 2 + int(r.integers(0, 2))
        sub = int(r.integers(0, 2 ** 63)) * 2 + int(r.integers(0, 2))
        off = int(r.integers(0, 2 ** 40)) * 4            # whole blocks: first word starts a block
        triples.append((seed, sub, off))
    got = _ref(rocrand_ref, triples)
    for (seed, sub, off), ref in zip(triples, got):
        blk = off // 4
        ctr = (blk & 0xFFFFFFFF, blk >> 32, sub & 0xFFFFFFFF, sub >> 32)
        key = (seed & 0xFFFFFFFF, seed >> 32)
        assert philox4x32_10(ctr, key) == ref, (seed, sub, off)


def test_numpy_and_integer_forms_agree():
    r = rng(301)
    n = 500
    c = [r.integers(0, 2 ** 32, n, dtype=np.uint64) for _ in range(4)]
    k = [r.integers(0, 2 ** 32, n, dtype=np.uint64) for _ in range(2)]
    vec = philox4x32_10_np(*c, *k)
    for i in range(0, n, 7):
        assert tuple(int(w[i]) for w in vec) == philox4x32_10([int(x[i]) for x in c], [int(x[i]) for x in k])


def test_output_bits_balanced():
    # weak statistical sanity: over a counter sweep every output bit is set about half the time
    n = 1 << 14
    w = philox4x32_10_np(np.arange(n, dtype=np.uint64), 0, 0, 0, 12345, 678)
    for word in w:
        bits = ((word[:, None] >> np.arange(32, dtype=np.uint64)) & np.uint64(1)).mean(0)
        assert np.all(np.abs(bits - 0.5) < 0.02)
