"""Resource use of every kernel in the built library, read from the library's
own gfx950 code objects (their AMDGPU metadata notes): no kernel uses scratch
memory or spills vector registers, every workgroup's LDS fits a CU, and the
one-launch prefill keeps the register and LDS budget of two resident
workgroups per CU.

CPU only: the code object is unbundled from the built libtreewy.so with the
ROCm LLVM tools (llvm-objcopy, clang-offload-bundler, llvm-readelf).  Skipped
when the library has not been built or the tools are absent."""
import os
import shutil
import subprocess
import sys

import pytest
import yaml

sys.path.insert(0, os.path.join(os.path.dirname(__file__), ".."))
from gated_deltanet_tree_03_amd import abi  # noqa: E402

LLVM = "/opt/rocm/llvm/bin"
TOOLS = ("llvm-objcopy", "clang-offload-bundler", "llvm-readelf")
LDS_PER_CU = 160 * 1024
VGPRS_PER_SIMD_LANE = 512


def _kernels(tmp_path):
    lib = abi.LIB_PATH
    if not os.path.exists(lib):
        pytest.skip("libtreewy.so is not built")
    if not all(os.path.exists(os.path.join(LLVM, t)) for t in TOOLS):
        pytest.skip("ROCm LLVM tools not found")
    fat = tmp_path / "fat.bin"
    subprocess.run([os.path.join(LLVM, "llvm-objcopy"), f"--dump-section=.hip_fatbin={fat}", lib,
                    str(tmp_path / "copy.so")], check=True, capture_output=True)
    # one offload bundle per source file, concatenated
    data = fat.read_bytes()
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    starts = []
    i = data.find(magic)
    while i >= 0:
        starts.append(i)
        i = data.find(magic, i + 1)
    assert starts, "no offload bundle in the library"
    out = {}
    for n, a in enumerate(starts):
        b = starts[n + 1] if n + 1 < len(starts) else len(data)
        part = tmp_path / f"bundle{n}.bin"
        part.write_bytes(data[a:b])
        co = tmp_path / f"gfx950_{n}.co"
        subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--unbundle", "--type=o",
                        "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--input={part}", f"--output={co}"],
                       check=True, capture_output=True)
        if co.stat().st_size == 0:
            continue
        notes = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "--notes", str(co)], check=True,
                               capture_output=True, text=True).stdout
        if "amdhsa.kernels" not in notes:
            continue
        start = notes.index("---")
        end = notes.index("\n...", start)
        meta = yaml.safe_load(notes[start:end])
        out.update({k[".name"]: k for k in meta["amdhsa.kernels"]})
    return out


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    return _kernels(tmp_path_factory.mktemp("codeobj"))


def test_every_kernel_is_present(kernels):
    names = " ".join(kernels)
    for family in ("verify_kernel", "commit_kernel", "store_all_kernel", "select_kernel", "prefill_kernel"):
        assert family in names, f"no {family} in the code object"


def test_no_kernel_uses_scratch_or_spills_vector_registers(kernels):
    # (scalar registers spilled into vector-register lanes touch no memory
    # and are allowed: the deep-tree table classes and the prefill have some)
    bad = []
    for name, k in kernels.items():
        if (k[".private_segment_fixed_size"] != 0 or k.get(".vgpr_spill_count", 0) != 0
                or k.get(".uses_dynamic_stack", False)):
            bad.append((name, k[".private_segment_fixed_size"], k.get(".vgpr_spill_count")))
    assert not bad, f"kernels with scratch or vector-register spills: {bad}"


def test_lds_fits_a_cu(kernels):
    for name, k in kernels.items():
        assert k[".group_segment_fixed_size"] <= LDS_PER_CU, name


def test_prefill_keeps_two_workgroups_per_cu(kernels):
    # 16-bit inputs: 8 waves per workgroup, two workgroups per CU = 4 waves
    # per SIMD, so at most 128 registers per lane; and two workgroups' LDS
    pf = [k for n, k in kernels.items() if "prefill_kernel" in n and "ILb0E" in n]
    assert len(pf) == 1
    k = pf[0]
    assert k[".vgpr_count"] + k[".agpr_count"] <= VGPRS_PER_SIMD_LANE // 4
    assert 2 * k[".group_segment_fixed_size"] <= LDS_PER_CU
