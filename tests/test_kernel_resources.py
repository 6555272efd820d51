"""Resources of the built gfx950 kernels, read without a GPU from the
library's own device code objects (the AMDGPU metadata notes that
llvm-readelf prints): the decode kernels keep their arrays in registers (no
scratch memory), and the bf16 exact kernel keeps the register and LDS budget
of two blocks per compute unit.  A loop the compiler fails to unroll can put
a kernel's arrays in scratch memory with no other sign: a residual batch of
16 clusters per wave did so at G = 2..5 (528 bytes per lane, about a third
slower at 1M) until its early exit was removed."""

import os
import re
import subprocess

import pytest

from long_context_sparse_mog_amd import build_lib, capi

LLVM = "/opt/rocm/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"
BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def _tool(name):
    path = os.path.join(LLVM, name)
    if not os.path.exists(path):
        pytest.skip(f"{path} is not installed")
    return path


def _kernel_metadata(lib_path, tmp):
    """Kernel name -> metadata fields, from every gfx950 code object bundled
    in the library's device-code section (one bundle per source file)."""
    fatbin = os.path.join(tmp, "fatbin")
    subprocess.run([_tool("llvm-objcopy"), f"--dump-section=.hip_fatbin={fatbin}", lib_path, os.path.join(tmp, "x")],
                   check=True, capture_output=True)
    data = open(fatbin, "rb").read()
    starts = [m.start() for m in re.finditer(re.escape(BUNDLE_MAGIC), data)]
    assert starts, "no offload bundle in the library"
    kernels = {}
    for i, s in enumerate(starts):
        e = starts[i + 1] if i + 1 < len(starts) else len(data)
        bundle, co = os.path.join(tmp, f"b{i}"), os.path.join(tmp, f"co{i}")
        open(bundle, "wb").write(data[s:e])
        subprocess.run([_tool("clang-offload-bundler"), "--unbundle", "--type=o", f"--targets={TARGET}",
                        f"--input={bundle}", f"--output={co}"], check=True, capture_output=True)
        notes = subprocess.run([_tool("llvm-readelf"), "--notes", co], check=True, capture_output=True,
                               text=True).stdout
        # one YAML map per kernel, its keys in alphabetical order
        for entry in re.split(r"\n  - (?=\.)", notes)[1:]:
            fields = dict(re.findall(r"^\s*\.?(\w+):\s+(\S+)\s*$", entry, flags=re.M))
            if "name" in fields:
                kernels[fields["name"]] = fields
    return kernels


@pytest.fixture(scope="module")
def meta(tmp_path_factory):
    if not os.path.exists(capi.LIB_PATH):
        build_lib.build(force=False)
    return _kernel_metadata(capi.LIB_PATH, str(tmp_path_factory.mktemp("co")))


DECODE_KERNELS = ("k_score_clusters", "k_select_topc", "k_select_sub1", "k_sub_wave", "k_subclusters", "k_exact",
                  "k_merge", "k_dense")


def test_metadata_lists_the_decode_kernels(meta):
    for k in DECODE_KERNELS:
        assert any(k in n for n in meta), k
    # every (head dim, group size) instance of the bf16 exact kernel
    exact = [n for n in meta if "k_exact" in n and "MfmaTile" in n]
    assert len(exact) == 16, exact


def test_decode_kernels_use_no_scratch(meta):
    # the float32 engine at G = 8 is exempt: its register tile of 8 heads
    # spills at either head dimension (a configuration no workload here uses)
    hot = {n: m for n, m in meta.items()
           if any(k in n for k in DECODE_KERNELS) and not ("RowAcc" in n and "Li8E" in n)}
    assert len(hot) > 50
    bad = {n: m["private_segment_fixed_size"] for n, m in hot.items() if int(m["private_segment_fixed_size"]) != 0}
    assert not bad, bad


def test_exact_kernel_fits_two_blocks_per_compute_unit(meta):
    # 4 waves a block, 2 blocks a compute unit: at most 256 vector registers
    # (VGPRs + AGPRs) a lane and 80 KB of LDS a block
    for n, m in meta.items():
        if "k_exact" in n and "MfmaTile" in n:
            regs = int(m["vgpr_count"]) + int(m.get("agpr_count", 0))
            assert regs <= 256, (n, regs)
            assert int(m["group_segment_fixed_size"]) <= 80 * 1024, (n, m["group_segment_fixed_size"])
