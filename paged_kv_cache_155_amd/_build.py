"""Build the HIP library libpa.so for gfx950 (in-tree, next to this file).

    python -m paged_kv_cache_155_amd._build

hipcc cross-compiles without a GPU.  Packed-fp32 instruction selection is
switched off for all device code.
"""
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -amdgpu-mfma-vgpr-form: matrix-core accumulators in VGPRs.  The multi-query
# kernel keeps its softmax state and rescales O with VALU ops, and the AGPR form
# made the compiler copy S and O between the register files on every chunk.
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form=1",
         "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(out=LIB, extra=(), quiet=False):
    cmd = [HIPCC, *FLAGS, *extra, "-o", out + ".tmp", *sources()]
    if not quiet:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


PROBE_SRC = os.path.join(ROOT, "read_probe.hip")
PROBE = os.path.join(ROOT, "_build", "read_probe")


def build_probe(quiet=False):
    """The streaming-read probe that bench.py --probe read runs (not part of
    the library)."""
    os.makedirs(os.path.dirname(PROBE), exist_ok=True)
    cmd = [HIPCC, "-O3", "-std=c++17", f"--offload-arch={ARCH}",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-o", PROBE + ".tmp", PROBE_SRC]
    if not quiet:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(PROBE + ".tmp", PROBE)
    return PROBE


if __name__ == "__main__":
    build(quiet="-q" in sys.argv)
    build_probe(quiet="-q" in sys.argv)
