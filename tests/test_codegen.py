"""Checks on the generated gfx950 code (no GPU needed: hipcc cross-compiles)."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "stream_paged_attention_amd", "csrc")


_ASM = {}


def _asm(src, tmp_path):
    """gfx950 assembly of one source file (compiled once per session)."""
    if src not in _ASM:
        hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
        if not os.path.exists(hipcc):
            pytest.skip("hipcc not available")
        out = tmp_path / (src + ".s")
        subprocess.run([hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
                        "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                        "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", str(out)],
                       check=True, capture_output=True)
        _ASM[src] = out.read_text().splitlines()
    return _ASM[src]


def test_m0_is_only_written_for_the_tile_dma(tmp_path):
    # rows_mfma issues its global->LDS loads from asm that sets M0; nothing
    # else in the file may read or write M0
    lines = [ln.strip() for ln in _asm("rows_mfma.hip", tmp_path)]
    code = [ln for ln in lines if ln and not ln.startswith((";", ".", "//")) and not ln.endswith(":")]
    n = 0
    for i, ln in enumerate(code):
        if re.search(r"\bm0\b", ln):
            assert re.fullmatch(r"s_mov_b32 m0, s\d+", ln), ln
            assert code[i + 1] == "s_nop 0", code[i + 1]
            assert code[i + 2].startswith("global_load_lds_dwordx4"), code[i + 2]
            n += 1
    assert n > 0


def test_no_packed_fp32_arithmetic(tmp_path):
    for src in sorted(f for f in os.listdir(CSRC) if f.endswith(".hip")):
        for ln in _asm(src, tmp_path):
            assert not re.search(r"\bv_pk_(add|mul|fma)_f32\b", ln), (src, ln)


def _descriptors(lines):
    """kernel name -> {field: int} from the .amdhsa_kernel blocks."""
    out, name = {}, None
    for ln in lines:
        ln = ln.strip()
        if ln.startswith(".amdhsa_kernel "):
            name = ln.split()[1]
            out[name] = {}
        elif ln.startswith(".end_amdhsa_kernel"):
            name = None
        elif name and ln.startswith(".amdhsa_"):
            parts = ln.split()
            if len(parts) == 2 and parts[1].lstrip("-").isdigit():
                out[name][parts[0]] = int(parts[1])
    return out


def test_rows_kernels_use_no_scratch_and_the_small_shape_fits_two_a_cu(tmp_path):
    # no rows kernel spills to scratch; the head-dim-256 shape for small
    # query tiles keeps registers within two waves a SIMD (<= 256) and its
    # LDS within half a CU's 160 KB, so two of its 4-wave workgroups share a CU
    small = 0
    for src in ("rows_mfma.hip", "rows_valu.hip"):
        desc = _descriptors(_asm(src, tmp_path))
        assert desc, src
        for name, d in desc.items():
            assert d[".amdhsa_private_segment_fixed_size"] == 0, name
            if "rows_mfma_kernelILi256" in name and name.endswith("ELb1EEEvNS_10RowsParamsE"):
                small += 1
                assert d[".amdhsa_next_free_vgpr"] <= 256, name
                assert d[".amdhsa_group_segment_fixed_size"] <= 80 * 1024, name
    assert small == 9   # 3 storage kinds x 3 masks


def test_d128_matrix_core_kernel_runs_two_workgroups_a_cu(tmp_path):
    # three workgroups a CU ran the ring drafter 15 % slower than two: the
    # D 128 kernel allocates more than a third of a CU's 160 KB of LDS
    desc = _descriptors(_asm("rows_mfma.hip", tmp_path))
    n = 0
    for name, d in desc.items():
        if "rows_mfma_kernelILi128" in name:
            n += 1
            assert d[".amdhsa_group_segment_fixed_size"] > 160 * 1024 // 3, name
            assert d[".amdhsa_group_segment_fixed_size"] <= 160 * 1024 // 2, name
    assert n == 9
