"""The 16 x 16 x 32 GEMM kernel writes its [k][n] products as inline asm (accumulator tied in place),
so the compiler does not pad the wait states around them.  These tests compile the kernel source
for gfx950 with the library's flags and scan the listing for data hazards on those products
(tests/asm_hazards.py), and check that the scan catches planted hazards."""

import os
import subprocess

import pytest

from tensor_transformer_linear_amd import build as B
from tests.asm_hazards import scan

SRC = os.path.join(B.CSRC, "gemm_bigwave16.hip")


def test_scanner_catches_planted_hazards():
    listing = "\n".join([
        "_Zplanted:",
        "\tv_accvgpr_write_b32 a0, 0",          # written right before the product reads it
        "\t;;#ASMSTART",
        "\tv_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], a[0:3]",
        "\t;;#ASMEND",
        "\ts_nop 3",
        "\tv_accvgpr_read_b32 v8, a1",           # read 4 wait states after it
        "\tv_mov_b32 v4, 0",                     # source rewritten ...
        "\ts_nop 0",
        "\t;;#ASMSTART",
        "\tv_mfma_f32_16x16x32_bf16 a[4:7], v[0:3], v[4:7], a[4:7]",  # ... 1 wait state before
        "\t;;#ASMEND",
        "\ts_nop 15",
        "\ts_nop 15",
        "\tv_accvgpr_read_b32 v9, a5",           # 32 wait states after: fine
        "\tv_mfma_f32_16x16x32_bf16 a[8:11], v[0:3], v[4:7], a[8:11]",  # compiler's own: not checked
        "\tv_accvgpr_read_b32 v10, a9",
        ".Lfunc_end0:",
    ])
    report, products = scan(listing)
    assert products == 2
    assert len(report) == 3, report


@pytest.mark.skipif(not os.path.exists(B.hipcc()) and B.hipcc() == "hipcc", reason="needs hipcc")
def test_gemm16_asm_products_have_no_hazards(tmp_path):
    out = tmp_path / "gemm_bigwave16.s"
    cmd = [B.hipcc(), *B.COMMON, "--cuda-device-only", "-S", SRC, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    listing = out.read_text()
    report, products = scan(listing)
    # every [k][n] and blocked instance writes its products as asm: 128 or 96 per k-tile, in the
    # loop and the peeled k-tiles
    assert products > 1000, products
    assert not report, "\n".join(report[:20])
    assert "scratch_" not in listing, "a GEMM kernel uses scratch memory"
