"""Host check of the 64-bit half split and join (csrc/halves.h) that the
attention kernels use to pass a wave-uniform address or index through the
32-bit wave broadcast. The header is plain C++; it is compiled here with g++
into a small program that prints the results for fixed and random values.

The case that matters is a low half with bit 31 set: widened as a signed int
it would fill the high word with ones and send the address far out of its
buffer."""

import os
import shutil
import subprocess

import numpy as np
import pytest

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "sequence_sharded_paged_amd", "csrc")

PROGRAM = r"""
#include <cstdio>
#include <cinttypes>
#include "halves.h"
static_assert(dcp::join_halves(-1, 0x12) == 0x00000012FFFFFFFFull, "low half widened with its sign");
static_assert(dcp::join_halves(0, -1) == 0xFFFFFFFF00000000ull, "high half");
static_assert(dcp::low_half(0x7FFF0000ABCD1234ull) == 0xABCD1234 - 0x100000000ll, "low half as a signed int");
int main() {
  uint64_t v;
  while (std::scanf("%" SCNu64, &v) == 1) {
    const int lo = dcp::low_half(v), hi = dcp::high_half(v);
    std::printf("%d %d %" PRIu64 "\n", lo, hi, dcp::join_halves(lo, hi));
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def halves_exe(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    d = tmp_path_factory.mktemp("halves")
    src, exe = d / "halves.cpp", d / "halves"
    src.write_text(PROGRAM)
    subprocess.run([gxx, "-std=c++17", "-O2", "-Wall", "-Werror", "-I", CSRC, str(src), "-o", str(exe)], check=True)
    return str(exe)


def run(exe, values):
    out = subprocess.run([exe], input="".join(f"{v}\n" for v in values), capture_output=True, text=True, check=True)
    return [tuple(int(x) for x in line.split()) for line in out.stdout.splitlines()]


def signed32(x):
    return x - (1 << 32) if x >= (1 << 31) else x


def test_split_and_join_round_trip(halves_exe):
    rng = np.random.default_rng(11)
    fixed = [0, 1, (1 << 31) - 1, 1 << 31, (1 << 32) - 1, 1 << 32, 0x00007F12_80000000, 0x00007FFF_FFFFFFF0,
             0xFFFFFFFF_FFFFFFFF, 0x80000000_00000000]
    # device addresses live high in a 48-bit space; the random draws cover all 64 bits too
    rand = [int(x) for x in rng.integers(0, 1 << 62, size=200, dtype=np.int64)] + \
           [int(x) | (1 << 63) for x in rng.integers(0, 1 << 62, size=50, dtype=np.int64)] + \
           [(int(x) << 4) | 0x0000_7000_0000_0000 | (1 << 31) for x in rng.integers(0, 1 << 40, size=50)]
    values = fixed + rand
    got = run(halves_exe, values)
    assert len(got) == len(values)
    for v, (lo, hi, back) in zip(values, got):
        assert lo == signed32(v & 0xFFFFFFFF)
        assert hi == signed32(v >> 32)
        assert back == v


def test_low_half_with_sign_bit_keeps_high_word(halves_exe):
    # the sign-extension mistake would give 0xFFFFFFFF in the high word
    (lo, hi, back), = run(halves_exe, [0x00000012_FFFFFFFF])
    assert (lo, hi) == (-1, 0x12) and back == 0x00000012_FFFFFFFF
