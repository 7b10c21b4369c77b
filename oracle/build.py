"""Builds oracle/liboracle.so with gcc (plain C11, OpenMP, no HIP).

Test infrastructure: only the test suite, the smoke check and the bench's
CPU-baseline leg load the result.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "sp24_oracle.c")
OUT = os.path.join(HERE, "liboracle.so")


def build(extra_flags=()) -> str:
    tmp = OUT + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           *extra_flags, SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(sys.argv[1:]))
