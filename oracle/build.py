"""Compile the CPU oracle (plain C, gcc) into oracle/liboracle.so.

Test infrastructure: the library built here is loaded only by the test suite,
the smoke check and the benchmark's CPU-baseline leg.
"""
import os
import subprocess
from pathlib import Path

HERE = Path(__file__).resolve().parent
SOURCE = HERE / "specv_oracle.c"
LIBRARY = HERE / "liboracle.so"


def build(verbose: bool = False) -> Path:
    # -O2 without -ffast-math: gcc keeps the written order of every float64
    # sum, so the oracle sums exactly in index order.
    tmp = LIBRARY.with_suffix(".so.tmp%d" % os.getpid())
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-pthread", "-Wall", "-Wextra",
           "-fno-fast-math", "-ffp-contract=off", str(SOURCE), "-o", str(tmp), "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
