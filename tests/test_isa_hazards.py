"""The d = 128 attention kernel's asm MFMAs keep their wait states (CPU only: compiles to assembly)."""
import os
import shutil
import subprocess
import sys

import pytest

sys.path.insert(0, os.path.dirname(__file__))
from isa_hazards import functions, scan  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "long_context_sparse_patsearch_amd", "csrc", "attn.hip")


def test_scan_finds_planted_hazards():
    listing = [
        "v_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]",
        "v_accvgpr_read_b32 v8, a3",                      # A: 0 wait states after the MFMA
        "s_nop 7", "s_nop 3",
        "v_accvgpr_read_b32 v9, a4",                      # 1 + 8 + 4 = 13 after: fine
        "v_mov_b32 v5, v9",
        "v_mfma_f32_32x32x16_bf16 v[16:31], v[4:7], a[20:23], 0",   # B: v5 written just before
        "v_add_f32 v17, v17, v9",                         # A: MFMA result read at once
    ]
    kinds = sorted(m[0] for m in scan(listing))
    assert kinds == ["A", "A", "B"], kinds


def test_scan_accepts_compiler_spacing():
    listing = [
        "v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], 0",
        "s_nop 11",
        "v_add_f32 v24, v0, v1",
        "v_mov_b32 v20, v24",
        "s_nop 1",
        "v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]",
    ]
    assert scan(listing) == []


@pytest.mark.skipif(shutil.which("/opt/rocm/bin/hipcc") is None, reason="hipcc not installed")
def test_q64_kernel_has_no_mfma_hazards(tmp_path):
    out = tmp_path / "attn.s"
    cmd = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-w",
           "-I" + os.path.join(ROOT, "include"), "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "--cuda-device-only", "-S", SRC, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    fns = functions(out.read_text(), "attn_q64_kernel")
    assert len(fns) == 4, sorted(fns)
    for name, lines in fns.items():
        assert sum("v_mfma" in ln for ln in lines) >= 160, name
        problems = scan(lines)
        assert not problems, (name, problems[:5])
