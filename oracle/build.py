"""Build the CPU oracle (plain C) into oracle/liboracle.so.

Test infrastructure only: the tests, the smoke check and the bench's
cpu_baseline leg load the result; the product library never does.
"""

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# No contraction and no fast math: every a*b+c stays two rounded operations
# unless the source writes fmaf().
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(extra_flags=()):
    cmd = ["gcc", *CFLAGS, *extra_flags, SRC, "-o", LIB + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build())
