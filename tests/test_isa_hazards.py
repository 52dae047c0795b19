"""Wait-state checks on the generated gfx950 assembly of the MFMA-bound kernel
(weight_only_fp4_amd.isa_check holds the rules and the walk).

Each build of the kernel's translation unit is compiled to assembly on the
host (no GPU involved) and every inline-asm MFMA, accumulator read and
global -> LDS copy is checked; the walk itself is checked on planted cases.
"""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from weight_only_fp4_amd import build as B
from weight_only_fp4_amd.isa_check import hazards, inline_ops

HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def _asm(extra):
    out = subprocess.run(
        [HIPCC, *B.COMMON, *extra, "--cuda-device-only", "-S", "-o", "-", os.path.join(B.CSRC, "gemm_mfma.hip")],
        capture_output=True, text=True)
    assert out.returncode == 0, out.stderr[-2000:]
    return out.stdout


MFMA_BUILDS = [extra for src, extra, _ in B.SOURCES if src == "gemm_mfma.hip"]


def test_mfma_unit_builds_are_listed():
    assert len(MFMA_BUILDS) == 8


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_inline_mfma_wait_states():
    with ThreadPoolExecutor(len(MFMA_BUILDS)) as ex:
        texts = list(ex.map(_asm, MFMA_BUILDS))
    for extra, text in zip(MFMA_BUILDS, texts):
        ops = inline_ops(text)
        assert any(o.startswith("v_mfma") for o in ops), extra
        assert any(o.startswith("global_load_lds") for o in ops), extra
        assert hazards(text) == [], (extra, hazards(text)[:10])


def test_checker_flags_planted_hazards():
    """An operand written right before an inline MFMA, an accumulator read
    right after one, and an SGPR base written by a VALU right before a copy
    are reported; the padded forms are not."""
    bad = "\n".join([
        "_ZN5nvfp411k_gemm_mfmaILi4EEEv:",
        "\tv_perm_b32 v13, v13, v105, s49",
        "\t;;#ASMSTART",
        "\tv_mfma_f32_16x16x32_bf16 a[12:15], v[10:13], v[50:53], a[12:15]",
        "\t;;#ASMEND",
        "\tv_accvgpr_read_b32 v0, a13",
        ".Lfunc_end0:",
    ])
    good = bad.replace("\t;;#ASMSTART\n", "\t;;#ASMSTART\n\ts_nop 1\n").replace(
        "\tv_accvgpr_read_b32", "\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\tv_accvgpr_read_b32")
    assert len(hazards(bad)) == 2
    assert hazards(good) == []
    # an operand written one wait state before, and a branch target in between
    assert len(hazards(bad.replace("\t;;#ASMSTART\n", "\t;;#ASMSTART\n\ts_nop 0\n"))) == 2
    assert len(hazards(bad.replace("\t;;#ASMSTART\n", ".LBB0_3:\n\t;;#ASMSTART\n"))) == 2
    copy = "\n".join([
        "_ZN5nvfp411k_gemm_mfmaILi4EEEv:",
        "\tv_readfirstlane_b32 s45, v7",
        "\t;;#ASMSTART",
        "\ts_mov_b32 m0, s34",
        "\ts_nop 0",
        "\tglobal_load_lds_dwordx4 v69, s[44:45]",
        "\t;;#ASMEND",
        ".Lfunc_end0:",
    ])
    assert len(hazards(copy)) == 1
    assert hazards(copy.replace("\ts_mov_b32 m0", "\ts_nop 2\n\ts_mov_b32 m0")) == []
    # a scalar move rewriting the base in between: the copy reads the moved value (the form the copies use)
    moved = copy.replace("\ts_nop 0\n\tglobal_load_lds_dwordx4 v69, s[44:45]",
                         "\ts_mov_b64 s[44:45], s[0:1]\n\tglobal_load_lds_dwordx4 v69, s[44:45]")
    assert hazards(moved) == []
    # a compare reads its first operand: it does not hide the write
    cmp = copy.replace("\t;;#ASMSTART", "\ts_cmp_eq_u32 s45, 0\n\t;;#ASMSTART")
    assert len(hazards(cmp)) == 1
