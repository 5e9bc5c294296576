"""Build the CPU oracle shared library (test infrastructure only).

The oracle is plain C compiled with gcc: no intrinsics, no -march flags,
OpenMP only to spread independent (sequence, head) pairs over host threads.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "pa_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(src=SRC, out=LIB, extra_flags=(), quiet=False):
    """Compile `src` into the shared library `out`; returns `out`."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           *extra_flags, "-o", out + ".tmp", src, "-lm"]
    if not quiet:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


# AddressSanitizer + UndefinedBehaviorSanitizer build of the same source: any
# out-of-bounds access, use after free or undefined operation aborts.
SANITIZE_FLAGS = ("-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                  "-fno-omit-frame-pointer", "-g")


def build_sanitized(out, src=SRC, quiet=True):
    """The oracle with ASan/UBSan (host code only; gcc, no GPU code)."""
    return build(src, out, extra_flags=SANITIZE_FLAGS, quiet=quiet)


def sanitizer_preload():
    """The runtime a non-instrumented python must preload to load an ASan
    library (ASan has to come first in the process)."""
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                       check=True)
    return r.stdout.strip()


if __name__ == "__main__":
    build(quiet="-q" in sys.argv)
