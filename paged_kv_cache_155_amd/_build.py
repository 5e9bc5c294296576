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


if __name__ == "__main__":
    build(quiet="-q" in sys.argv)
