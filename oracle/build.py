"""Builds the fp64 CPU oracle (test infrastructure) with the host C compiler.

The oracle is plain C compiled by gcc, never by hipcc, and includes no HIP
header: it shares nothing with the GPU library.  Run as a script or call
``build()``; the shared object lands next to the source.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gn_oracle.c")
LIB = os.path.join(HERE, "libgnoracle.so")


def build(verbose: bool = False) -> str:
    # -ffp-contract=off keeps every multiply and add a separate IEEE rounding,
    # in the order the source writes them.
    cmd = [
        os.environ.get("CC", "gcc"), "-O2", "-std=c11", "-fPIC", "-shared",
        "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
        "-o", LIB + ".tmp", SRC, "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
