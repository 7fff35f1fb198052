"""CPU checks of the compiled gfx950 kernels' resources (hipcc cross-compiles
without a GPU): register budgets that set the occupancy the kernels are
designed for, no register spills, and no scratch memory traffic on the hot
paths (a by-reference argument once spilled a struct to scratch for every
row and added 43% to the select kernel's writes)."""
from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "streaming_indexer_top_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC) and not shutil.which("hipcc"),
                                reason="hipcc not available")


def device_asm(src, tmp_path):
    out = tmp_path / (os.path.basename(src) + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-mcode-object-version=5",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I" + os.path.join(ROOT, "include"), "-S", "--cuda-device-only",
           os.path.join(CSRC, src), "-o", str(out)]
    # hipcc leaves intermediate files in its working directory.
    subprocess.run(cmd, check=True, capture_output=True, text=True, cwd=str(tmp_path))
    return out.read_text()


def kernel_meta(asm):
    """{symbol: {field: int}} from the code object metadata."""
    meta = {}
    for block in asm.split("  - .agpr_count:")[1:]:
        name = re.search(r"\.name:\s+(\S+)", block).group(1)
        fields = dict((k, int(v)) for k, v in re.findall(
            r"\.(vgpr_count|vgpr_spill_count|sgpr_spill_count|private_segment_fixed_size):\s+(\d+)",
            block))
        meta[name] = fields
    return meta


def body(asm, symbol):
    i = asm.index(symbol + ":")
    return asm[i:asm.index(".Lfunc_end", i)]


@pytest.fixture(scope="module")
def score_asm(tmp_path_factory):
    return device_asm("score_kernels.hip", tmp_path_factory.mktemp("asm"))


@pytest.fixture(scope="module")
def select_asm(tmp_path_factory):
    return device_asm("select_kernels.hip", tmp_path_factory.mktemp("asm"))


def test_score_kernels_no_scratch_and_two_waves_per_simd(score_asm):
    meta = kernel_meta(score_asm)
    bf16 = {n: m for n, m in meta.items() if "score_bf16_kernel" in n}
    assert bf16
    for name, m in bf16.items():
        assert m["vgpr_spill_count"] == 0, name
        assert m["private_segment_fixed_size"] == 0, name
    # D_I=128 with 64 heads and double-buffered 128- or 192-key tiles (the
    # latter is the automatic choice): two waves per SIMD, i.e. at most 256
    # registers.
    for tile in (128, 192):
        main = ("_ZN3csa12_GLOBAL__N_117score_bf16_kernelILi128ELi2ELi%dELb1ELi8EEEvNS_9ScoreArgsE"
                % tile)
        assert bf16[main]["vgpr_count"] <= 256, main
    # The fp32 path keeps q for up to 64 heads resident (128 registers at
    # D_I=128) in 8-wave workgroups: no spills, at most 256 registers, and
    # its tiles plus the 8 row histograms within the CU's 160 KiB of LDS.
    f32 = {n: m for n, m in meta.items() if "score_f32_kernel" in n}
    assert len(f32) == 6
    for name, m in f32.items():
        assert m["vgpr_spill_count"] == 0 and m["private_segment_fixed_size"] == 0, name
        assert m["vgpr_count"] <= 256, name
    for block in score_asm.split("  - .agpr_count:")[1:]:
        name = re.search(r"\.name:\s+(\S+)", block).group(1)
        if "score_f32_kernel" in name:
            assert int(re.search(r"\.group_segment_fixed_size:\s+(\d+)", block).group(1)) <= 160 * 1024, name


def test_select_kernels_no_scratch_on_the_hot_path(select_asm):
    meta = kernel_meta(select_asm)
    for k in (2048, 4096):
        name = "_ZN3csa12_GLOBAL__N_113select_kernelILi%dEEEvNS_10SelectArgsE" % k
        assert meta[name]["vgpr_spill_count"] == 0
        # Only the out-of-line fallback (massive ties, fp32 scores) may touch
        # scratch, for its own saved registers; the kernel body never does.
        assert "scratch_" not in body(select_asm, name), name
    # Four rows per CU for k <= 2048: at most 128 registers.
    assert meta["_ZN3csa12_GLOBAL__N_113select_kernelILi2048EEEvNS_10SelectArgsE"]["vgpr_count"] <= 128
    for name, m in meta.items():
        if "merge" in name:
            assert m["private_segment_fixed_size"] == 0 and m["vgpr_spill_count"] == 0, name


@pytest.fixture(scope="module")
def attention_asm(tmp_path_factory):
    return device_asm("attention_kernels.hip", tmp_path_factory.mktemp("asm"))


def test_attention_kernels_fit_one_row_per_cu(attention_asm):
    """Every attention instance (two head counts x two dim pairs): no
    spills, no scratch, LDS within the CU's 160 KiB, and 8 waves, two per
    SIMD, so at most 256 registers."""
    meta = kernel_meta(attention_asm)
    att = {n: m for n, m in meta.items() if "attention_" in n and "kernel" in n}
    assert len(att) == 4
    assert all("attention_split_kernel" in n for n in att)
    for name, m in att.items():
        assert m["vgpr_spill_count"] == 0 and m["sgpr_spill_count"] == 0, name
        assert m["private_segment_fixed_size"] == 0, name
        assert "scratch_" not in body(attention_asm, name), name
        assert m["vgpr_count"] <= 256, name
    for block in attention_asm.split("  - .agpr_count:")[1:]:
        name = re.search(r"\.name:\s+(\S+)", block).group(1)
        if "attention_" in name and "kernel" in name:
            assert int(re.search(r"\.group_segment_fixed_size:\s+(\d+)", block).group(1)) <= 160 * 1024, name
