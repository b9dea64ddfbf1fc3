"""The CPU test suite under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU needed).

Two runs, one sanitizer runtime each (gcc's and clang's cannot share a process):
  1. the oracle and the host input generator built by gcc with -fsanitize=address,undefined,
     gcc's runtime preloaded, every `-m "not gpu"` test;
  2. the host half of libmpstep.so (argument checks, chunk tables, gradset slots) built by
     hipcc with the same sanitizers on the host side only, clang's runtime preloaded, the
     tests that drive the library on the host.
Findings abort the run (-fno-sanitize-recover=all).  The normal libraries are rebuilt at the
end, whatever happened.

    python tests/run_sanitized.py
"""
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def pytest(preload, args):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", LD_PRELOAD=preload)
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
           *args]
    print("+", "LD_PRELOAD=" + preload, " ".join(cmd), flush=True)
    return subprocess.run(cmd, cwd=ROOT, env=env).returncode


def main():
    from oracle import build as oracle_build
    from inputs import build as gen_build
    from optimizer_step_tensor_amd import build as lib_build
    rc = 0
    try:
        lib_build.build()
        oracle_build.build(sanitize=True)
        gen_build.build_host(sanitize=True)
        gcc_asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                                  text=True, check=True).stdout.strip()
        # the mutation tests rebuild oracle copies without sanitizers: skipped here
        rc = pytest(gcc_asan, ["tests", "--deselect", "tests/test_oracle_mutants.py",
                               "--ignore", "tests/test_kernel_resources.py"])
        oracle_build.build()
        gen_build.build_host()
        if rc == 0:
            lib_build.build(sanitize=True)
            clang_asan = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/"
                                          "libclang_rt.asan-x86_64.so"))[-1]
            rc = pytest(clang_asan, ["tests/test_host_abi.py", "tests/test_bench_host.py"])
    finally:
        oracle_build.build()
        gen_build.build_host()
        lib_build.build()
    print("sanitized CPU runs:", "clean" if rc == 0 else "FAILED (rc %d)" % rc, flush=True)
    return rc


if __name__ == "__main__":
    sys.exit(main())
