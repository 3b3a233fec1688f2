"""Checks on the generated gfx950 code (no GPU needed: hipcc cross-compiles)."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "stream_paged_attention_amd", "csrc")


def _asm(src, tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = tmp_path / "k.s"
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
                    "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                    "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", str(out)],
                   check=True, capture_output=True)
    return out.read_text().splitlines()


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
