"""The implicit-GEMM address generator splits a K index into (filter tap,
channel) and a tap into (r, s) with fastdiv (csrc/fastdiv.hpp): a precomputed
rounded-up reciprocal, one high multiply and one correction.  Compiled here for
the host with g++ and checked against integer division on every divisor up to
3000 with all small numerators and random ones up to 2^31 - 1, and on random
divisors of every magnitude."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
HEADER = os.path.join(os.path.dirname(HERE), "implicit_gemm_conv_amd", "csrc", "fastdiv.hpp")

PROGRAM = r"""
#include "fastdiv.hpp"
#include <cstdio>
#include <random>
int main() {
    std::mt19937_64 g(7);
    long bad = 0;
    for (uint32_t d = 1; d <= 3000; ++d) {
        const uint32_t m = igc::fastdiv_magic(d);
        for (uint32_t n = 0; n < 4096; ++n) bad += igc::fastdiv(n, d, m) != n / d;
        for (int i = 0; i < 512; ++i) {
            const uint32_t n = (uint32_t)(g() & 0x7fffffff);
            bad += igc::fastdiv(n, d, m) != n / d;
        }
        bad += igc::fastdiv(0x7fffffffu, d, m) != 0x7fffffffu / d;
        bad += igc::fastdiv(0x7fffffffu - (0x7fffffffu % d), d, m) != 0x7fffffffu / d;
    }
    for (int i = 0; i < 2000000; ++i) {
        uint32_t d = (uint32_t)(g() & 0x7fffffff) >> (g() % 31);
        if (d == 0) d = 1;
        const uint32_t n = (uint32_t)(g() & 0x7fffffff);
        bad += igc::fastdiv(n, d, igc::fastdiv_magic(d)) != n / d;
    }
    std::printf("%ld\n", bad);
    return 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_fastdiv_matches_integer_division(tmp_path):
    src = tmp_path / "fd.cpp"
    src.write_text(PROGRAM)
    exe = tmp_path / "fd"
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    assert int(out.strip()) == 0

