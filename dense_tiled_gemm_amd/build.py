"""Build libgemm_bt.so (hand-written HIP for gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SO = os.path.join(HERE, "libgemm_bt.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # keep the compiler from forming packed-fp32 VALU ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMAs read and write their accumulators in VGPRs.  For a 256-thread
    # workgroup the compiler otherwise assumes a wave may need more than 256
    # registers, picks the AGPR form and then rotates the accumulator blocks
    # through copies inside the K loop (1024x4096x4096: 48 -> 40 us).  Every
    # kernel here keeps its accumulators within 256 registers.
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall",
    "-Wno-unused-function",
]


def sources():
    return [os.path.join(CSRC, "gemm_bt.hip")]


def build(extra=None, out=SO, verbose=False) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + ["-I", os.path.join(ROOT, "include"), "-I", CSRC] + list(extra or []) \
        + sources() + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


C_CHECK_SRC = os.path.join(ROOT, "tests", "c_abi_check.cpp")
C_CHECK = os.path.join(ROOT, "tests", "c_abi_check")


def build_c_check(verbose=False) -> str:
    """The C++ program that calls the library through include/gemm_bt.h alone (host code, linked to the in-tree
    libgemm_bt.so by an rpath relative to itself)."""
    tmp = C_CHECK + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), C_CHECK_SRC, "-L", HERE, "-lgemm_bt",
           "-Wl,-rpath,$ORIGIN/../dense_tiled_gemm_amd", "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, C_CHECK)
    return C_CHECK


SWZ_DUMP_SRC = os.path.join(ROOT, "tests", "swizzle_dump.cpp")
SWZ_DUMP = os.path.join(ROOT, "tests", "swizzle_dump")


def build_swizzle_dump(verbose=False) -> str:
    """The host program that prints the kernels' LDS swizzle maps (from the kernel headers) for the CPU tests."""
    tmp = SWZ_DUMP + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, SWZ_DUMP_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, SWZ_DUMP)
    return SWZ_DUMP


if __name__ == "__main__":
    print(build(extra=sys.argv[1:], verbose=True))
