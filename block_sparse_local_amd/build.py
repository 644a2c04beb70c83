"""Build libbsl.so in-tree with hipcc for gfx950.

    python -m block_sparse_local_amd.build          # or build() from Python

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection disabled (ordinary float code stays scalar VALU).  The host ABI layer
is compiled by hipcc as well and everything is linked into one shared library
next to this file.
"""
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbsl.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["fwd_bf16.hip", "fwd_f32.hip", "bsl_api.cpp"]
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Werror", f"--offload-arch={ARCH}",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]
# no packed-fp32 instruction selection; MFMA accumulators in ordinary VGPRs
# (the AGPR form makes the compiler copy every accumulator each step)
DEVICE_ONLY = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-mllvm", "-amdgpu-mfma-vgpr-form"]


def _compile(src, obj, extra=()):
    is_hip = src.endswith(".hip")
    cmd = [HIPCC, *COMMON]
    if is_hip:
        cmd += [*DEVICE_ONLY, "-x", "hip"]
    else:
        cmd += ["-x", "hip"]  # host-only file, but compiled by the same driver
    cmd += [*extra, "-c", src, "-o", obj]
    subprocess.run(cmd, check=True)


def build(out=LIB, extra=(), verbose=False):
    with tempfile.TemporaryDirectory(prefix="bsl_build_") as tmp:
        objs = []
        for s in SOURCES:
            obj = os.path.join(tmp, os.path.basename(s) + ".o")
            _compile(os.path.join(CSRC, s), obj, extra)
            objs.append(obj)
        link = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out + ".tmp"]
        subprocess.run(link, check=True)
    os.replace(out + ".tmp", out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
