"""Build the seeded input generator: a host library (gcc + OpenMP) and its HIP twin."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(HERE, "libmpgen_host.so")
DEV_LIB = os.path.join(HERE, "libmpgen_dev.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
             "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd, out):
    tmp = out + ".tmp"
    subprocess.run([c if c != "@OUT" else tmp for c in cmd], check=True)
    os.replace(tmp, out)
    return out


def build_host(sanitize=False):
    """sanitize: AddressSanitizer + UndefinedBehaviorSanitizer, findings fatal (CPU test runs)."""
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-g"] if sanitize else []
    return _run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                 "-fno-fast-math", "-Wall", *san, "-o", "@OUT", os.path.join(HERE, "gen_host.c")],
                HOST_LIB)


def build_dev():
    return _run([HIPCC, *HIP_FLAGS, "-o", "@OUT", os.path.join(HERE, "gen_dev.hip")], DEV_LIB)


def build():
    return build_host(), build_dev()


if __name__ == "__main__":
    print(build())
