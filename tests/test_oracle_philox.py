"""Pins for the oracle's Philox4x32-10 and the stochastic-rounding word mapping (CPU)."""

import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

from oracle.philox import philox4x32_10, sr_word

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_published_known_answers():
    """tests/golden/philox4x32_10_kat.txt: the Random123 known-answer vectors."""
    n = 0
    for line in open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")):
        if line.startswith("#") or not line.strip():
            continue
        v = [int(s, 16) for s in line.split()]
        out = philox4x32_10(*v[:6])
        assert [int(o) for o in out] == v[6:], line
        n += 1
    assert n == 3


def test_stream_mode_is_word_stream():
    seed = 0x1234_5678_9ABC
    n = np.arange(64, dtype=np.uint64)
    s = sr_word(n, seed, "stream")
    for j in range(16):
        blk = philox4x32_10(j, 0, 0, 0, seed & 0xFFFFFFFF, seed >> 32)
        for w in range(4):
            assert int(s[4 * j + w]) == int(blk[w])
    e = sr_word(n, seed, "element")
    for j in range(8):
        assert int(e[j]) == int(philox4x32_10(j, 0, 0, 0, seed & 0xFFFFFFFF, seed >> 32)[0])


_RR_SRC = r"""
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
#include <cstdlib>
int main(int argc, char** argv) {
  for (int i = 1; i + 1 < argc; i += 2) {
    unsigned long long seed = strtoull(argv[i], 0, 10), off = strtoull(argv[i + 1], 0, 10);
    rocrand_state_philox4x32_10 st;
    rocrand_init(seed, 0, off, &st);
    printf("%u\n", rocrand(&st));
  }
  return 0;
}
"""


def test_matches_rocrand_host_engine():
    """Library pin: rocRAND's Philox4x32-10 engine, run on the host.  Its offset
    counts 32-bit outputs, so offset 4n yields word 0 of counter n (element mode)
    and offset n yields the stream word n (stream mode)."""
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
        pytest.skip("rocRAND headers / hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "rr.cpp")
        exe = os.path.join(d, "rr")
        open(src, "w").write(_RR_SRC)
        subprocess.run([hipcc, "-x", "hip", "--offload-arch=gfx950", src, "-o", exe], check=True,
                       capture_output=True, timeout=300)
        cases = [(1234, 0), (1234, 1), (1234, 4095), (1234, 32768 * 4096 - 1), (0, 7),
                 (2 ** 40 + 17, 123456789), (1234, 2 ** 33 + 5)]
        args = []
        for seed, n in cases:
            args += [str(seed), str(4 * n), str(seed), str(n)]
        out = subprocess.run([exe] + args, check=True, capture_output=True, text=True, timeout=60).stdout.split()
        got = [int(v) for v in out]
        for i, (seed, n) in enumerate(cases):
            assert got[2 * i] == int(sr_word(n, seed, "element")), (seed, n)
            assert got[2 * i + 1] == int(sr_word(n, seed, "stream")), (seed, n)
