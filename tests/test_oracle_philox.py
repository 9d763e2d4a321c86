"""Pins for the oracle's Philox4x32-10 (CPU only).

The oracle's pure-Python Philox is checked against rocRAND's Philox4x32-10
engine, a library routine compiled here for the host from rocRAND's public
header (tests/pins/rocrand_philox_host.cpp), plus the properties the stream
addressing relies on.
"""
import ctypes
import os
import random
import shutil
import subprocess

import numpy as np
import pytest

from oracle import philox

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="session")
def rocrand_lib(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand/rocrand_kernel.h"):
        pytest.skip("rocRAND headers / hipcc not available")
    out = tmp_path_factory.mktemp("rr") / "librr.so"
    src = os.path.join(HERE, "pins", "rocrand_philox_host.cpp")
    subprocess.run([hipcc, "-O2", "-shared", "-fPIC", "--offload-host-only", "-x", "hip",
                    src, "-o", str(out)], check=True, capture_output=True)
    return ctypes.CDLL(str(out))


def _rocrand_block(lib, c, k):
    out = (ctypes.c_uint * 4)()
    lib.rocrand_philox4x32_10_block(*[ctypes.c_uint(x) for x in list(c) + list(k)], out)
    return tuple(out)


def test_matches_rocrand_engine(rocrand_lib):
    rng = random.Random(20240115)
    cases = [((0, 0, 0, 0), (0, 0)),
             ((0xFFFFFFFF, 0x3FFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF), (0xFFFFFFFF, 0xFFFFFFFF)),
             ((1, 0, 0, 0), (0, 0)), ((0, 0, 1, 0), (0, 0)), ((0, 0, 0, 0), (1, 0))]
    for _ in range(3000):
        # rocRAND's skip-ahead takes word1:word0 as a block count times four,
        # so word 1 stays below 2**30 (the counters used here pack node and
        # batch index into it, far below that bound).
        c = (rng.getrandbits(32), rng.getrandbits(30), rng.getrandbits(32), rng.getrandbits(32))
        k = (rng.getrandbits(32), rng.getrandbits(32))
        cases.append((c, k))
    for c, k in cases:
        assert philox.philox4x32_10(c, k) == _rocrand_block(rocrand_lib, c, k), (c, k)


def test_verification_addressing_matches_rocrand(rocrand_lib):
    for seed in (0, 0x5EED0002, (1 << 40) + 7):
        for off in (0, 1, 12345, (1 << 33) + 5):
            for b in (0, 3, 1000):
                for node in (0, 5, 63):
                    for slot in (0, 1, 9, philox.SAMPLE_SLOT):
                        c = philox.counter_for(b, node, slot, off)
                        k = philox.key_for(seed)
                        x0 = _rocrand_block(rocrand_lib, c, k)[0]
                        assert philox.uniform(seed, off, b, node, slot) == (x0 >> 8) / 2.0 ** 24


def test_counter_fields_are_distinct():
    seen = set()
    for b in range(3):
        for node in range(64):
            for slot in list(range(4)) + [philox.SAMPLE_SLOT]:
                for off in (0, 1):
                    seen.add(philox.counter_for(b, node, slot, off))
    assert len(seen) == 3 * 64 * 5 * 2


def test_uniform_grid_and_uniformity():
    n = 20000
    us = np.array([philox.uniform(7, 0, 0, i % 64, i // 64) for i in range(n)])
    assert us.min() >= 0.0 and us.max() < 1.0
    assert np.all(us * 2 ** 24 == np.floor(us * 2 ** 24))          # 24-bit grid
    hist = np.bincount((us * 32).astype(int), minlength=32)
    chi2 = ((hist - n / 32) ** 2 / (n / 32)).sum()
    assert chi2 < 70.0   # dof 31; 99.99th percentile ~ 66.6 .. keep a deterministic margin
    assert abs(us.mean() - 0.5) < 0.01


def test_counter_layout_is_the_documented_one():
    # (slot, node | batch << 8, offset low word, offset high word); key = seed words
    assert philox.counter_for(3, 5, 9, (7 << 32) | 11) == (9, 5 | (3 << 8), 11, 7)
    assert philox.counter_for(0, 63, philox.SAMPLE_SLOT, 0) == (0xFFFFFFFF, 63, 0, 0)
    assert philox.key_for((0xAB << 32) | 0xCD) == (0xCD, 0xAB)
