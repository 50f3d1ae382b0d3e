"""Register budgets of the kernels, from the compiler's own report (no GPU).

The GEMM pipeline counts its outstanding memory operations exactly (vmcnt
waits of a fixed depth, one wave per SIMD): a register spill would add
scratch loads and stores to those counts and let a wait release before its
data has landed.  Every instantiation must therefore compile with no VGPR or
SGPR spills, within one wave's 512 registers.  The other kernels keep their
rows and weight windows in registers by design, so none of them may spill
either.  The sources are compiled here for gfx950 with the library's own
flags and the AMDGPU kernel metadata of the assembly is read back.
"""

import os
import re
import subprocess

import pytest

from transformer_ffn_block_residual_amd import build


def kernel_metadata(asm):
    """[(name, {field: value})] for every kernel in the amdhsa.kernels list."""
    out = []
    cur = None
    for line in asm.splitlines():
        m = re.match(r"^\s+- \.(\w+):\s+(\S+)", line)
        if m and cur is not None and m.group(1) == "agpr_count":
            out.append(cur)
            cur = None
        if m and m.group(1) == "agpr_count":
            cur = {"agpr_count": m.group(2)}
            continue
        if cur is not None:
            f = re.match(r"^\s+\.(\w+):\s+(\S+)", line)
            if f:
                cur.setdefault(f.group(1), f.group(2))
    if cur is not None:
        out.append(cur)
    return [(k.get("name", "?"), k) for k in out]


def device_asm(tmp_path, src):
    if not os.path.exists(build.HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path / (src + ".s")
    flags = [f for f in build.FLAGS if f != "-fPIC"]
    r = subprocess.run([build.HIPCC, *flags, "--cuda-device-only", "-S", "-o", str(out),
                        os.path.join(build.CSRC, src)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def test_every_gemm_instantiation_compiles_without_spills(tmp_path):
    kernels = [(n, k) for n, k in kernel_metadata(device_asm(tmp_path, "gemm.hip")) if "gemm_kernel" in n]
    # the forward, backward and quantising epilogues in both dtypes
    assert len(kernels) >= 10, [n for n, _ in kernels]
    for name, k in kernels:
        assert int(k["vgpr_spill_count"]) == 0, (name, k["vgpr_spill_count"])
        assert int(k["sgpr_spill_count"]) == 0, (name, k["sgpr_spill_count"])
        assert int(k["agpr_count"]) == 256, (name, k["agpr_count"])    # the 128 x 128 accumulator tile
        assert int(k["vgpr_count"]) <= 512, (name, k["vgpr_count"])    # one wave per SIMD
        assert int(k.get("private_segment_fixed_size", "0")) == 0, name  # no scratch at all


@pytest.mark.parametrize("src", [s for s in build.SOURCES if s not in ("gemm.hip", "abi.hip")])
def test_no_kernel_of_the_library_spills(tmp_path, src):
    kernels = kernel_metadata(device_asm(tmp_path, src))
    assert kernels, src
    for name, k in kernels:
        assert int(k["vgpr_spill_count"]) == 0 and int(k["sgpr_spill_count"]) == 0, (name, k["vgpr_spill_count"])
        assert int(k.get("private_segment_fixed_size", "0")) == 0, name
