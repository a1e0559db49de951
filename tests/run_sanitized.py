"""Run the CPU test suite against AddressSanitizer + UndefinedBehaviorSanitizer
builds of the host code: the oracle (gcc) and the library's host side (its
argument checks, plan choice and launch set-up; clang through hipcc).

The two compilers' sanitizer runtimes cannot share one process, so there are
two pytest runs, each with its own runtime preloaded:
  1. the oracle's pins (tests/test_oracle_*.py) against the sanitized oracle;
  2. the C ABI tests (tests/test_abi.py) against the sanitized library.
Any sanitizer report aborts the run (halt_on_error, no recovery from UB).
Leak detection is off: the Python interpreter keeps allocations until exit.

    python tests/run_sanitized.py
"""
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def _clang_asan():
    hits = sorted(glob.glob("/opt/rocm*/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise SystemExit("clang's ASan runtime was not found under /opt/rocm")
    return hits[-1]


def _gcc_asan():
    out = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = out.stdout.strip()
    if not os.path.isabs(path):
        raise SystemExit("gcc's ASan runtime was not found")
    return path


def main():
    from fp8_quantized_skinny_qpn_amd import build as hip_build
    from oracle import build as oracle_build
    oracle_build.build(sanitize=True)
    hip_build.build(sanitize=True)
    env = dict(os.environ, QPN_SANITIZED_BUILD="1",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    runs = [(_gcc_asan(), sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))),
            (_clang_asan(), [os.path.join(ROOT, "tests", "test_abi.py")])]
    for runtime, files in runs:
        print(f"== sanitized run: {os.path.basename(runtime)} on {len(files)} file(s)", flush=True)
        rc = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                             *files], cwd=ROOT, env=dict(env, LD_PRELOAD=runtime)).returncode
        if rc != 0:
            sys.exit(rc)
    print("sanitized runs passed", flush=True)


if __name__ == "__main__":
    main()
