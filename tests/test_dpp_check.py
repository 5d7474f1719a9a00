"""The DPP hazard check of the built device code
(dense_linear_solvers_amd/dpp_check.py): first on hand-written disassembly
(a VALU write then a DPP read of the same VGPR with zero, one and two wait
states between them, on the fall-through path and through a branch), then
on the library as built, which must have none."""
from __future__ import annotations

import os

import pytest

from dense_linear_solvers_amd import dpp_check

HEAD = "0000000000001000 <k>:\n"


def _lines(body):
    out, addr = [], 0x1000
    for ins in body:
        out.append(f"\t{ins} // {addr:012X}: 00000000")
        addr += 8
    return HEAD + "\n".join(out) + "\n"


def test_fall_through():
    w = "v_mul_f32_e32 v7, v1, v2"
    d = "v_fmac_f32_dpp v9, -v7, v3 row_newbcast:0 row_mask:0xf bank_mask:0xf"
    assert len(dpp_check.scan_disassembly(_lines([w, d]))) == 1
    assert len(dpp_check.scan_disassembly(_lines([w, "v_add_u32_e32 v5, v5, v6", d]))) == 1
    assert dpp_check.scan_disassembly(_lines([w, "s_nop 1", d])) == []
    assert dpp_check.scan_disassembly(_lines([w, "s_nop 0", "v_add_u32_e32 v5, v5, v6", d])) == []
    # a 64-bit write overlapping the source pair
    w64 = "v_fma_f64 v[6:7], v[0:1], v[2:3], v[4:5]"
    d64 = "v_fmac_f64_dpp v[10:11], -v[6:7], v[8:9] row_newbcast:3 row_mask:0xf bank_mask:0xf"
    assert len(dpp_check.scan_disassembly(_lines([w64, d64]))) == 1
    # the accumulator and the other source are not DPP sources
    assert dpp_check.scan_disassembly(_lines(["v_mov_b32_e32 v9, 0", d])) == []
    # writes to SGPRs (compares, readlane) are not VGPR writes
    assert dpp_check.scan_disassembly(_lines(["v_cmp_eq_u32_e32 vcc, v7, v1", d])) == []


def test_branch_into_the_read():
    # s_branch at 0x1000 jumps over the nop to the DPP read at 0x1018; the
    # write just before the branch reaches it with one wait state
    text = (HEAD +
            "\tv_mul_f32_e32 v7, v1, v2 // 000000000FF8: 0\n"
            "\ts_branch 2 // 000000001000: 0 <k+0x20>\n"
            "\tv_add_u32_e32 v5, v5, v6 // 000000001008: 0\n"
            "\ts_nop 1 // 000000001010: 0\n"
            "\tv_fmac_f32_dpp v9, -v7, v3 row_newbcast:0 row_mask:0xf bank_mask:0xf"
            " // 000000001018: 0\n")
    text = text.replace(HEAD, "0000000000000ff8 <k>:\n")
    found = dpp_check.scan_disassembly(text)
    assert len(found) == 1 and found[0][4] == hex(0xFF8)


def test_built_library_has_no_dpp_hazard():
    from dense_linear_solvers_amd.build import library_path
    lib = library_path()
    if not os.path.exists(lib) or not os.path.exists(dpp_check.OBJDUMP):
        pytest.skip("library not built here")
    n, bad = dpp_check.check_library(lib)
    assert n > 10000
    assert bad == [], bad[:5]
