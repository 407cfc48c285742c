"""Pins for the oracle's Philox4x32-10 block function and uniform mapping.

The block function is checked against published known-answer vectors and,
where the rocRAND headers and g++ are present, against rocRAND's own
philox4x32_10 engine on many random counters and keys.
"""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def _kat_rows():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            w = [int(t, 16) for t in line.split()]
            rows.append((w[0:4], w[4:6], w[6:10]))
    return rows


def test_known_answer_vectors():
    rows = _kat_rows()
    assert len(rows) == 3
    for ctr, key, want in rows:
        got = oracle.philox4x32_10(ctr, key)
        assert [int(g) for g in got] == want


_ROCRAND_PROBE = r"""
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
struct Eng : rocrand_device::philox4x32_10_engine {
  uint4 block(uint4 c, uint2 k) { return ten_rounds(c, k); }
};
int main() {
  Eng e; unsigned c0, c1, c2, c3, k0, k1;
  while (std::scanf("%x %x %x %x %x %x", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    uint4 r = e.block(uint4{c0, c1, c2, c3}, uint2{k0, k1});
    std::printf("%08x %08x %08x %08x\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
"""


def test_block_function_matches_rocrand():
    hdr = "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"
    if not (os.path.exists(hdr) and shutil.which("g++")):
        pytest.skip("rocRAND headers or g++ not available")
    rng = np.random.default_rng(1234)
    vals = rng.integers(0, 2**32, size=(500, 6), dtype=np.uint64)
    vals[:8, :4] = 0  # include small counters
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "p.cpp")
        exe = os.path.join(d, "p")
        with open(src, "w") as f:
            f.write(_ROCRAND_PROBE)
        subprocess.run(["g++", "-O1", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", src, "-o", exe],
                       check=True, capture_output=True)
        inp = "\n".join(" ".join(f"{int(x):08x}" for x in row) for row in vals) + "\n"
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout.split("\n")
    for row, line in zip(vals, out):
        want = [int(t, 16) for t in line.split()]
        got = oracle.philox4x32_10(row[:4].astype(np.uint32), row[4:].astype(np.uint32))
        assert [int(g) for g in got] == want


def test_uniform_mapping_bounds():
    # u = ((w >> 8) + 0.5) * 2^-24 never reaches 0 or 1 and is a dyadic rational
    assert oracle.u01(0) == 2.0 ** -25
    assert oracle.u01(0xFFFFFFFF) == 1.0 - 2.0 ** -25
    assert oracle.u01(0x000000FF) == 2.0 ** -25
    assert oracle.u01(0x00000100) == 1.5 * 2.0 ** -24
    assert oracle.u01(0x80000000) == 0.5 + 2.0 ** -25


def test_counter_layout_streams_are_distinct():
    # the draft stream uses word (v & 3) of the block at counter word1 = v >> 2
    seed, rnd = 0x0123456789ABCDEF, 7
    for stream in (0, 2):  # per-vocabulary streams: word (v & 3) of block v >> 2
        for v in range(8):
            blk = oracle.philox4x32_10([(stream << 24) | 3, v >> 2, 5, rnd], [seed & 0xFFFFFFFF, seed >> 32])
            assert oracle.random_word(seed, rnd, stream, 3, 5, v) == blk[v & 3]
    blk = oracle.philox4x32_10([(1 << 24) | 3, 0, 5, rnd], [seed & 0xFFFFFFFF, seed >> 32])
    assert oracle.random_word(seed, rnd, 1, 3, 5, 0) == blk[0]
    assert oracle.random_word(seed, rnd, 1, 3, 5, 77) == blk[0]  # accept stream ignores v
    words = {oracle.random_word(seed, rnd, s, 3, 5, 0) for s in range(3)}
    assert len(words) == 3


def test_draft_stream_uniformity_and_serial_correlation():
    # 16 equiprobable bins over 64k consecutive vocabulary entries, and the
    # lag-1 correlation of the uniforms along v
    n = 1 << 16
    u = np.array([oracle.u01(oracle.random_word(5, 0, 0, 1, 0, v)) for v in range(n)])
    counts = np.bincount((u * 16).astype(int), minlength=16)
    chi2 = ((counts - n / 16) ** 2 / (n / 16)).sum()
    assert chi2 < 37.7  # chi-square, 15 dof, alpha = 1e-3
    x = u - 0.5
    rho = (x[:-1] * x[1:]).mean() / (x * x).mean()
    assert abs(rho) < 4.0 / np.sqrt(n)
