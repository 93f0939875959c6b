"""Compile the scalar fp64 oracle (oracle.c) into oracle/liboracle.so.

Test infrastructure: the oracle is only loaded by the test-suite, the smoke
check and the CPU-baseline leg of the benchmark.  Built with plain gcc at -O2
and without fast-math so that the fp64 arithmetic is the one written in the
source.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
OUT = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math",
           "-Wall", "-Wextra", "-o", OUT + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
