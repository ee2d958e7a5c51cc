"""Pins for the oracle's counter-based generator.

The Philox4x32-10 definition is Salmon, Moraes, Dror and Shaw, "Parallel
random numbers: as easy as 1, 2, 3" (SC'11).  The oracle's implementation is
checked against an independent one: rocRAND's header-only Philox4x32-10
engine, compiled for the host.  rocRAND's engine at seed s, subsequence S and
skip 4c produces the block at counter (c low, c high, S low, S high) and key
(s low, s high); the oracle's stream for (request, position, step) uses
counter (position, request, step, 0), i.e. c = position + 2^32 request and
S = step.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
DUMP_SRC = os.path.join(HERE, "philox_ref", "rocrand_philox_dump.cpp")


@pytest.fixture(scope="module")
def rocrand_dump(tmp_path_factory):
    if shutil.which("g++") is None or not os.path.exists("/opt/rocm/include/rocrand"):
        pytest.skip("needs g++ and the rocRAND headers")
    exe = str(tmp_path_factory.mktemp("rr") / "rr_dump")
    subprocess.check_call(["g++", "-O1", "-std=c++17", "-D__HIP_PLATFORM_AMD__",
                           "-I/opt/rocm/include", "-o", exe, DUMP_SRC])

    def run(seed, subseq, c0, n):
        out = subprocess.check_output([exe, str(seed), str(subseq), str(c0), str(n)], text=True)
        rows = np.array([[int(t) for t in line.split()] for line in out.strip().splitlines()],
                        dtype=np.uint64)
        return rows
    return run


CASES = [
    (0, 0, 0),
    (0, 0, (5 << 32) + 0),          # request 5, positions 0..
    (0, 3, (63 << 32) + 0),         # step 3, request 63
    (0x0123456789ABCDEF, 7, (17 << 32) + 2**31),
    (0xFFFFFFFFFFFFFFFF, 0xFFFFFFFF, (0xFFFFFFFF << 32) + 0xFFFFFF00),
    (42, 1, 123456),
]


@pytest.mark.parametrize("seed,step,c0", CASES)
def test_philox_matches_rocrand(svo, rocrand_dump, seed, step, c0):
    n = 300
    ref = rocrand_dump(seed, step, c0, n)
    key = [seed & 0xFFFFFFFF, seed >> 32]
    for row in ref:
        c = int(row[0])
        ctr = [c & 0xFFFFFFFF, c >> 32, step & 0xFFFFFFFF, step >> 32]
        got = svo.philox(ctr, key)
        assert [int(x) for x in got] == [int(x) for x in row[1:]], (seed, step, c)


def test_uniform_stream_layout_matches_rocrand(svo, rocrand_dump):
    # uniforms(seed, request, step, position) must be words 0 and 1 of the
    # rocRAND block at skip 4 * (position + 2^32 request), subsequence step.
    seed, step = 0xDEADBEEF12345678, 9
    for request in (0, 1, 31, 4000):
        ref = rocrand_dump(seed, step, request << 32, 17)
        for row in ref:
            pos = int(row[0]) & 0xFFFFFFFF
            ua, us = svo.uniforms(seed, request, step, pos)
            assert ua == (int(row[1]) >> 8) / 2.0**24
            assert us == (int(row[2]) >> 8) / 2.0**24


def test_u24_grid(svo):
    assert svo.u24(0) == 0.0
    assert svo.u24(0xFFFFFFFF) == 1.0 - 2.0**-24
    assert svo.u24(0x100) == 2.0**-24
    assert svo.u24(0xFF) == 0.0
    assert svo.u24(0x80000000) == 0.5


def test_uniforms_are_uniform(svo):
    # Chi-square over 64 bins of 64000 accept uniforms, and of the sample
    # uniforms: a broken round or key schedule shows as gross non-uniformity
    # or as correlation between the two words.
    n = 64000
    ua = np.empty(n)
    us = np.empty(n)
    for i in range(n):
        ua[i], us[i] = svo.uniforms(0, i % 64, 0, i // 64)
    for u in (ua, us):
        counts, _ = np.histogram(u, bins=64, range=(0.0, 1.0))
        expected = n / 64
        chi2 = ((counts - expected) ** 2 / expected).sum()
        # 63 degrees of freedom: mean 63, sd ~11.2; 6 sd bound.
        assert chi2 < 63 + 6 * 11.2
    corr = np.corrcoef(ua, us)[0, 1]
    assert abs(corr) < 5.0 / np.sqrt(n)
