"""Checks on the gfx950 code object inside the built library (no GPU needed): every kernel keeps its data in
registers and LDS.  A kernel with scratch memory (a private segment, or spilled registers) pays for it on every
launch; an indexed array in device code once put 48 bytes per lane of scratch into every whole-row epilogue."""
import os
import re
import subprocess

import pytest

import dense_tiled_gemm_amd as gb

LLVM = "/opt/rocm/llvm/bin"
TOOLS = [os.path.join(LLVM, t) for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-readelf")]


def kernel_metadata(tmp_path):
    lib = gb.LIB_PATH
    if not os.path.exists(lib):
        pytest.skip("library not built")
    if not all(os.path.exists(t) for t in TOOLS):
        pytest.skip("LLVM tools of the ROCm install not found")
    fat = str(tmp_path / "fat.bin")
    co = str(tmp_path / "gfx950.co")
    subprocess.run([TOOLS[0], "--dump-section=.hip_fatbin=" + fat, lib, os.devnull], check=True)
    subprocess.run([TOOLS[1], "--unbundle", "--type=o", "--input=" + fat,
                    "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", "--output=" + co], check=True)
    notes = subprocess.run([TOOLS[2], "--notes", co], check=True, capture_output=True, text=True).stdout
    kernels = []
    for block in notes.split("  - .agpr_count")[1:]:
        field = lambda key: int(re.search(r"\." + key + r":\s+(\d+)", block).group(1))
        name = re.search(r"\.name:\s+(\S+)", block).group(1)
        kernels.append((name, field("private_segment_fixed_size"), field("vgpr_spill_count"),
                        field("sgpr_spill_count"), field("vgpr_count")))
    return kernels


def test_no_kernel_uses_scratch(tmp_path):
    kernels = kernel_metadata(tmp_path)
    assert len(kernels) > 100, len(kernels)
    for name, private, vspill, sspill, vgprs in kernels:
        assert private == 0 and vspill == 0 and sspill == 0, (name, private, vspill, sspill)
        assert vgprs <= 256, (name, vgprs)
