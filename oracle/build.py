"""Build the oracle's shared library with gcc.

Test infrastructure only: the oracle checks the HIP library and is never part
of it.  Flags: binary32/binary64 IEEE arithmetic with no contraction into FMA
and no fast-math, so each C operation is exactly one correctly rounded step.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mpstep_oracle.c")
LIB = os.path.join(HERE, "libmporacle.so")

CFLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-fexcess-precision=standard", "-Wall", "-Wextra"]


# AddressSanitizer + UndefinedBehaviorSanitizer build, for a CPU test run with the
# sanitizer runtime preloaded (tests/run_sanitized.py); every finding is fatal.
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
            "-g"]


def build(out=LIB, src=SRC, extra=(), sanitize=False):
    """Compile `src` into `out` (always recompiles); returns the library path."""
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, *(SANITIZE if sanitize else ()), *extra, "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
