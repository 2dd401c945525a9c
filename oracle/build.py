"""Builds the CPU oracle (plain C, gcc) into oracle/liboracle.so.

Test infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline leg load the result.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "igc_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(extra_flags=(), out=LIB, src=SRC):
    """Compiles igc_oracle.c (or a copy of it) with gcc.  No fast-math: fp64 sums stay IEEE."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
           "-ffp-contract=off", "-Wall", "-Wextra", *extra_flags, src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build(sys.argv[1:]))
