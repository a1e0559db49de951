"""Build the CPU oracle (test infrastructure) into oracle/libqpn_oracle.so.

Plain gcc, C11, FP64 arithmetic with contraction off so every FP32 pack step
is a single IEEE round-to-nearest operation, OpenMP over output rows only.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qpn_oracle.c")
LIB = os.path.join(HERE, "libqpn_oracle.so")

CFLAGS = [
    "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp",
    "-ffp-contract=off", "-fno-fast-math", "-fexcess-precision=standard",
    "-Wall", "-Wextra", "-Wno-unused-parameter",
]


def build(verbose: bool = False) -> str:
    """Compile the oracle unconditionally; return the library path."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
