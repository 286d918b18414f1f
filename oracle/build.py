"""Compile the float64 oracle (plain C, OpenMP) into oracle/libtt_oracle.so.

Test infrastructure: the oracle checks the HIP library and is never part of it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "tt_oracle.c")
LIB = os.path.join(HERE, "libtt_oracle.so")


def build(src: str = SRC, out: str = LIB, extra=()) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
           *extra, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(), file=sys.stderr)
