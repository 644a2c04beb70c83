"""Build libbsl.so in-tree with hipcc for gfx950.

    python -m block_sparse_local_amd.build          # or build() from Python

A design variant (one design choice of the bf16 kernel reverted, for timing and
counter comparisons against the shipped kernel) is built elsewhere and loaded
through the BSL_LIBRARY environment variable:

    python -m block_sparse_local_amd.build --variant no-swizzle --out /tmp/v.so
    BSL_LIBRARY=/tmp/v.so python bench.py

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection disabled (ordinary float code stays scalar VALU).  The host ABI layer
is compiled by hipcc as well and everything is linked into one shared library
next to this file.
"""
import argparse
import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbsl.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["fwd_bf16.hip", "fwd_f32.hip", "bwd_bf16.hip", "bwd_valu.hip", "kmer.hip", "check.hip",
           "scratch.hip", "bsl_api.cpp"]
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Werror", f"--offload-arch={ARCH}",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]
# no packed-fp32 instruction selection
DEVICE_ONLY = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# MFMA accumulators in ordinary VGPRs (the AGPR form makes the compiler copy
# every accumulator each step)
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]

# name -> (extra compiler flags, MFMA accumulators in VGPRs); the switches are
# described at the top of csrc/fwd_bf16.hip
VARIANTS = {
    "shipped": ([], True),
    "no-swizzle": (["-DBSL_SWIZZLE=0"], True),
    "no-xcd-remap": (["-DBSL_XCD_REMAP=0"], True),
    "no-rotation": (["-DBSL_ROTATE=0"], True),
    "hardware-order": (["-DBSL_XCD_REMAP=0", "-DBSL_ROTATE=0"], True),
    "eager-rescale": (["-DBSL_RESCALE_SLACK=0.0f"], True),
    "eager-exchange": (["-DBSL_LAZY_EXCHANGE=0"], True),
    "agpr-accumulators": ([], False),
    "global-ring-loads": (["-DBSL_RING_BUFFER_LOADS=0"], True),
    "narrow-stores": (["-DBSL_WIDE_STORES=0"], True),
}


def _compile(src, obj, extra=(), vgpr_form=True):
    is_hip = src.endswith(".hip")
    cmd = [HIPCC, *COMMON]
    if is_hip:
        cmd += [*DEVICE_ONLY, *(VGPR_FORM if vgpr_form else []), "-x", "hip"]
    else:
        cmd += ["-x", "hip"]  # host-only file, compiled by hipcc like the kernels
    cmd += [*extra, "-c", src, "-o", obj]
    subprocess.run(cmd, check=True)


def build(out=LIB, extra=(), verbose=False, variant="shipped"):
    if variant not in VARIANTS:
        raise ValueError(f"unknown variant {variant!r}; one of {sorted(VARIANTS)}")
    vflags, vgpr_form = VARIANTS[variant]
    with tempfile.TemporaryDirectory(prefix="bsl_build_") as tmp:
        objs = []
        for s in SOURCES:
            obj = os.path.join(tmp, os.path.basename(s) + ".o")
            _compile(os.path.join(CSRC, s), obj, [*vflags, *extra], vgpr_form)
            objs.append(obj)
        link = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out + ".tmp"]
        subprocess.run(link, check=True)
    os.replace(out + ".tmp", out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    ap = argparse.ArgumentParser(description="build libbsl.so for gfx950")
    ap.add_argument("--variant", default="shipped", choices=sorted(VARIANTS))
    ap.add_argument("--out", default=None, help="output path (default: the in-tree library; "
                    "a variant other than 'shipped' needs an explicit --out)")
    args, extra = ap.parse_known_args()
    if args.variant != "shipped" and args.out is None:
        ap.error("a design variant is built next to, never over, the in-tree library: give --out")
    build(out=args.out or LIB, extra=extra, verbose=True, variant=args.variant)
