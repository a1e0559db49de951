"""Compile the HIP sources under csrc/ into fp8_quantized_skinny_qpn_amd/libqpn.so.

hipcc cross-compiles for gfx950 without a GPU.  Flags:
  -ffp-contract=off and correctly rounded FP32 division keep every FP32 step
  of the pack kernels a single IEEE operation; denormals are preserved; packed
  FP32 instructions are disabled (the compiler would otherwise form them from
  scalar float code).

build(sanitize=True) builds the same library with AddressSanitizer and
UndefinedBehaviorSanitizer on the HOST code only (argument checks, plan
choice, launch set-up; the GPU code is unchanged) into _build/sanitize/, for
the CPU test suite (tests/run_sanitized.py); it never replaces libqpn.so.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libqpn.so")
SANITIZE_DIR = os.path.join(BUILD, "sanitize")
SANITIZED_LIB = os.path.join(SANITIZE_DIR, "libqpn.so")

SOURCES = ["qpn_api.cpp", "qpn_gemm.hip", "qpn_pack.hip", "qpn_prefill.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-result",
    "-I" + INCLUDE, "-I" + CSRC,
]


# host-only sanitizers: each -fsanitize applies to the host pass alone
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def _compile(src: str, verbose: bool, sanitize: bool = False) -> str:
    out_dir = SANITIZE_DIR if sanitize else BUILD
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"]
    extra = HOST_SANITIZE if sanitize else []
    cmd = [HIPCC, *FLAGS, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile every source and link libqpn.so (always rebuilds); with
    sanitize, the host-sanitized copy in _build/sanitize/ instead."""
    out_dir = SANITIZE_DIR if sanitize else BUILD
    lib = SANITIZED_LIB if sanitize else LIB
    os.makedirs(out_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, sanitize), SOURCES))
    tmp = lib + ".tmp"
    # every symbol resolved at link time: a kernel whose host-side launch
    # stub the compiler did not emit fails here, not when the library loads
    link_extra = ["-shared-libsan", *HOST_SANITIZE] if sanitize else ["-Wl,--no-undefined"]
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *link_extra, *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link of libqpn.so failed")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
