"""Build the fp64 CPU oracle (test infrastructure only) into oracle/liborc.so.

gcc, -O2, OpenMP, and -ffp-contract=off so that no multiply-add is fused:
the routing keys must come out of exactly the binary64 operations written in
orc.c.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "orc.c")
OUT = os.path.join(HERE, "liborc.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           "-Wno-unused-parameter", SRC, "-o", OUT + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
