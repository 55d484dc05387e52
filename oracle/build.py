"""Compile the fp64 CPU oracle (``oracle.c``) into ``liboracle.so``.

Test infrastructure only: the oracle checks the HIP path and is never part of
it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
# The row-parallel drivers (OpenMP) around oracle.c's serial functions, for
# the benchmark's all-cores CPU baseline.
SRC_ROWS = os.path.join(HERE, "oracle_rows.c")
LIB = os.path.join(HERE, "liboracle.so")


def stale() -> bool:
    return not os.path.exists(LIB) or any(os.path.getmtime(LIB) < os.path.getmtime(s)
                                          for s in (SRC, SRC_ROWS))


def build_oracle(force: bool = True) -> str:
    """Build ``liboracle.so`` next to this file with plain gcc (no fast-math)."""
    if not force and not stale():
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC", "-fopenmp",
           SRC, SRC_ROWS, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_oracle())
