"""Compile the HIP/C++ sources under csrc/ into one shared library for gfx950.

The library is built in-tree (next to this file) so that it travels with the
repository snapshot to a GPU machine; nothing is JIT-compiled at import time.
"""
import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libmoe_route_topk.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # IEEE fp32: correctly rounded divide, denormals kept, no FMA contraction
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-ffp-contract=off",
    # packed fp32 VALU ops stay off on this target family
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")) +
                  glob.glob(os.path.join(PKG, "csrc", "*.cpp")))


def build(verbose: bool = False) -> str:
    srcs = sources()
    if not srcs:
        return ""
    cmd = [HIPCC] + FLAGS + ["-I", os.path.join(ROOT, "include"), "-o", LIB + ".tmp"] + srcs
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    # the GEMMs' untracked weight and LDS loads: check the generated assembly
    # before the library is installed; a failing build leaves no library
    from .isa_check import check
    asm_flags = [f for f in FLAGS if f not in ("-shared", "-fPIC")]
    try:
        for src in ("ffn_q8.hip", "router.hip"):
            check(HIPCC, asm_flags, os.path.join(PKG, "csrc", src),
                  [os.path.join(ROOT, "include"), os.path.join(PKG, "csrc")])
    except Exception:
        for f in (LIB + ".tmp", LIB):
            if os.path.exists(f):
                os.remove(f)
        raise
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
