"""Compile the CPU oracle (norm_oracle.c) into oracle/liboracle.so with gcc.

Test infrastructure: the oracle is the reference the HIP library is checked against. Only the
tests, the smoke check and the benchmark's CPU-baseline leg load it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "norm_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# IEEE double arithmetic exactly as written: no fast-math, no FMA contraction.
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
          "-shared", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Build liboracle.so. With force=False an existing library is kept."""
    if not force and os.path.exists(LIB):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
