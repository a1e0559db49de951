"""Build the CPU oracle (test infrastructure) into oracle/libqpn_oracle.so.

Plain gcc, C11, FP64 arithmetic with contraction off so every FP32 pack step
is a single IEEE round-to-nearest operation, OpenMP over output rows only.

build(sanitize=True) builds it with AddressSanitizer and
UndefinedBehaviorSanitizer into _build/sanitize/libqpn_oracle.so for the CPU
test suite (tests/run_sanitized.py); it never replaces the normal library.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qpn_oracle.c")
LIB = os.path.join(HERE, "libqpn_oracle.so")
SANITIZED_LIB = os.path.join(os.path.dirname(HERE), "_build", "sanitize", "libqpn_oracle.so")
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
            "-fno-omit-frame-pointer", "-g"]

CFLAGS = [
    "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp",
    "-ffp-contract=off", "-fno-fast-math", "-fexcess-precision=standard",
    "-Wall", "-Wextra", "-Wno-unused-parameter",
]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile the oracle unconditionally; return the library path."""
    lib = SANITIZED_LIB if sanitize else LIB
    os.makedirs(os.path.dirname(lib), exist_ok=True)
    tmp = lib + ".tmp"
    cmd = ["gcc", *CFLAGS, *(SANITIZE if sanitize else []), SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    build(verbose=True, sanitize="--sanitize" in sys.argv)
    sys.exit(0)
