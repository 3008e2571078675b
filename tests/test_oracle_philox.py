"""Pins of the oracle's Philox4x32-10 uniform stream.

The raw 4x32 block function is checked word for word against ATen's
header-only Philox engine (an independent implementation of the same
published generator, Salmon et al. SC'11), called from a tiny C++ program
compiled here.  The uniform mapping is checked for range, grid and
distribution.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest
from scipy import stats

_HELPER_SRC = r"""
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdio>
#include <cstdint>
int main() {
  unsigned c0, c1, c2, c3, k0, k1;
  while (std::scanf("%x %x %x %x %x %x", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    uint64_t seed = (uint64_t)k0 | ((uint64_t)k1 << 32);
    uint64_t sub = (uint64_t)c2 | ((uint64_t)c3 << 32);
    uint64_t off = (uint64_t)c0 | ((uint64_t)c1 << 32);
    at::Philox4_32 eng(seed, sub, off);
    unsigned a = eng(), b = eng(), c = eng(), d = eng();
    std::printf("%08x %08x %08x %08x\n", a, b, c, d);
  }
  return 0;
}
"""


def _torch_include():
    try:
        import torch
    except Exception:
        return None
    inc = os.path.join(os.path.dirname(torch.__file__), "include")
    return inc if os.path.exists(os.path.join(inc, "ATen/core/PhiloxRNGEngine.h")) else None


def test_raw_words_match_aten_engine(orc, tmp_path):
    inc = _torch_include()
    if inc is None or shutil.which("g++") is None:
        pytest.skip("ATen Philox header or g++ not available")
    src = tmp_path / "aten_philox.cpp"
    exe = tmp_path / "aten_philox"
    src.write_text(_HELPER_SRC)
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", inc, str(src), "-o", str(exe)], check=True)
    rng = np.random.default_rng(7)
    cases = [[0] * 6, [0xFFFFFFFF] * 6, [1, 2, 3, 4, 5, 6]]
    cases += rng.integers(0, 2**32, size=(300, 6), dtype=np.uint64).tolist()
    # counters shaped like the ones the method uses: (b, k, stream, offset)
    cases += [[b, k, s, 0, 0, 0] for b in range(3) for k in range(3) for s in range(3)]
    text = "\n".join(" ".join("%x" % int(v) for v in c) for c in cases) + "\n"
    res = subprocess.run([str(exe)], input=text, capture_output=True, text=True, check=True)
    lines = res.stdout.strip().split("\n")
    assert len(lines) == len(cases)
    for c, line in zip(cases, lines):
        want = [int(w, 16) for w in line.split()]
        got = orc.philox4x32_10(c[:4], c[4:]).tolist()
        assert got == want, (c, got, want)


def test_uniform_is_24bit_grid_in_unit_interval(orc):
    for b in range(20):
        for k in range(20):
            u = orc.uniform(1234567890123, 5, b, k, b % 3)
            assert 0.0 <= u < 1.0
            assert (u * 2**24) == int(u * 2**24)


def test_uniform_counter_layout(orc):
    # counter = (request, position, stream, call offset); key = seed halves;
    # the uniform keeps the top 24 bits of word 0.
    seed = (7 << 32) | 11
    for (b, k, s, off) in [(0, 0, 0, 0), (3, 5, 1, 9), (127, 15, 2, 1)]:
        w = orc.philox4x32_10([b, k, s, off], [11, 7])
        assert orc.uniform(seed, off, b, k, s) == (int(w[0]) >> 8) / 2.0**24


def test_uniform_statistics(orc):
    n = 1 << 15
    u = np.array([orc.uniform(42, 0, i & 1023, i >> 10, 0) for i in range(n)])
    assert abs(u.mean() - 0.5) < 4 * np.sqrt(1 / 12 / n)
    assert abs(u.var() - 1 / 12) < 0.01
    counts = np.bincount((u * 256).astype(int), minlength=256)
    assert stats.chisquare(counts).pvalue > 1e-4
    # streams and offsets give different values
    assert orc.uniform(42, 0, 0, 0, 0) != orc.uniform(42, 0, 0, 0, 1)
    assert orc.uniform(42, 0, 0, 0, 0) != orc.uniform(42, 1, 0, 0, 0)
