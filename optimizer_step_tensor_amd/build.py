"""Build libmpstep.so (the HIP kernels and the C ABI of include/mpstep.h) for gfx950."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmpstep.so")
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("api.hip", "kernels.hip")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# -ffp-contract=off: no fusing of a*b+c, every operation rounds as written.
# -fhip-fp32-correctly-rounded-divide-sqrt: IEEE division and square root.
# -packed-fp32-ops off: no v_pk_* fp32 instructions are generated.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
         "-fno-gpu-flush-denormals-to-zero",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wextra", "-Wno-unused-parameter",
         "-I", os.path.join(ROOT, "include")]


# The host half (argument checks, chunk tables, gradset slots) under AddressSanitizer
# and UndefinedBehaviorSanitizer, findings fatal; the device code is built as usual.
# For CPU test runs with clang's sanitizer runtime preloaded (tests/run_sanitized.py).
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def build(out=LIB, extra=(), sanitize=False):
    """Compile the library (always recompiles); returns its path."""
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *(SANITIZE_HOST if sanitize else ()), *extra, "-o", tmp, *SOURCES]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


CEILING_SRC = os.path.join(HERE, "csrc", "ceiling.hip")
CEILING_LIB = os.path.join(HERE, "libmpceiling.so")


def build_ceiling(out=CEILING_LIB):
    """The benchmark's bandwidth probes (csrc/ceiling.hip): not part of the library's API."""
    tmp = out + ".tmp"
    subprocess.run([HIPCC, *FLAGS, "-o", tmp, CEILING_SRC], check=True)
    os.replace(tmp, out)
    return out


EXAMPLE_SRC = os.path.join(HERE, "examples", "c_api_step.cpp")
EXAMPLE = os.path.join(HERE, "examples", "c_api_step")


def build_example():
    """The C example that drives the library with plain HIP allocations (host code only)."""
    cmd = [HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall", "-Wextra",
           "-I", os.path.join(ROOT, "include"), "-o", EXAMPLE + ".tmp", EXAMPLE_SRC,
           "-L", HERE, "-lmpstep", "-Wl,-rpath,$ORIGIN/.."]
    subprocess.run(cmd, check=True)
    os.replace(EXAMPLE + ".tmp", EXAMPLE)
    return EXAMPLE


if __name__ == "__main__":
    print(build())
    print(build_ceiling())
    print(build_example())
