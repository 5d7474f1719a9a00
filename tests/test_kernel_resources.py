"""Register budget of the built device code, read from the code objects'
metadata (llvm-readelf --notes of the gfx950 images the library carries):
no kernel spills to scratch, AGPRs appear only where documented, and every
LU solve that takes panels of two columns for one more wave per SIMD
(lu_min_waves) fits the registers of that wave count, so the occupancy its
launch bound declares is the one the hardware gives it."""
from __future__ import annotations

import os
import re
import subprocess
import tempfile

import pytest

from dense_linear_solvers_amd import dpp_check

READELF = "/opt/rocm/llvm/bin/llvm-readelf"

# (dtype, N, NRHS, T) of the gesv kernels with panels of two, and the waves
# per SIMD each declares (lu_min_waves in csrc/tdls_internal.h)
EXTRA_WAVE = {
    ("d", 32, 1, 16): 3,
    ("d", 24, 1, 16): 3,
    ("d", 24, 2, 16): 3,
    ("d", 24, 4, 16): 3,
    ("d", 48, 4, 64): 3,
    ("d", 48, 8, 64): 3,
    ("f", 32, 8, 16): 4,
}

_LU = re.compile(r"gesv_panel_kernelI([fd])Li(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELb([01])E")


def parse_notes(text: str) -> list:
    """Kernel records (name, vgpr_count, agpr_count, private_segment_fixed_size)
    of llvm-readelf --notes output."""
    kernels, cur = [], None
    for line in text.splitlines():
        m = re.match(r"^  - \.agpr_count:\s+(\d+)", line)
        if m:
            cur = {"agpr_count": int(m.group(1))}
            kernels.append(cur)
            continue
        m = re.match(r"^    \.(name|vgpr_count|private_segment_fixed_size):\s+(\S+)", line)
        if m and cur is not None:
            key, val = m.group(1), m.group(2)
            cur[key] = val if key == "name" else int(val)
    return [k for k in kernels if "name" in k]


def vgpr_budget(waves: int) -> int:
    """VGPRs per lane that leave room for `waves` waves per SIMD (512 per
    SIMD lane, allocated in blocks of 8)."""
    return 512 // waves // 8 * 8


def test_parse_notes_and_budget():
    text = ("  - .agpr_count:     0\n"
            "    .args:\n"
            "      - .name:           col\n"
            "    .name:           _ZN4tdls17gesv_panel_kernelIdLi32ELi1ELi16ELi2ELb0EEEv\n"
            "    .private_segment_fixed_size: 20\n"
            "    .vgpr_count:     168\n"
            "  - .agpr_count:     4\n"
            "    .name:           k2\n"
            "    .private_segment_fixed_size: 0\n"
            "    .vgpr_count:     64\n")
    ks = parse_notes(text)
    assert [k["name"][:14] for k in ks] == ["_ZN4tdls17gesv", "k2"]
    assert ks[0]["vgpr_count"] == 168 and ks[0]["private_segment_fixed_size"] == 20
    assert ks[1]["agpr_count"] == 4
    assert (vgpr_budget(2), vgpr_budget(3), vgpr_budget(4), vgpr_budget(5)) == (256, 168, 128, 96)


def _library_kernels() -> list:
    from dense_linear_solvers_amd.build import library_path
    lib = library_path()
    if not os.path.exists(lib) or not os.path.exists(READELF) \
            or not os.path.exists(dpp_check.OBJDUMP):
        pytest.skip("library not built here")
    with tempfile.TemporaryDirectory() as wd:
        kernels = []
        for img in dpp_check.device_images(lib, wd):
            out = subprocess.run([READELF, "--notes", img], check=True, capture_output=True,
                                 text=True).stdout
            kernels += parse_notes(out)
    return kernels


def test_built_kernels_fit_their_declared_occupancy():
    kernels = _library_kernels()
    assert len(kernels) > 100
    spilling = [k["name"] for k in kernels if k["private_segment_fixed_size"] != 0]
    assert spilling == [], spilling[:5]
    # AGPRs only in the float64 n = 16 quad-group LU kernels, which the
    # planner never picks (16-lane groups there; the group-size override
    # reaches them): their registers exceed 256 and AGPRs hold the rest
    agpr = [k["name"] for k in kernels if k["agpr_count"] != 0]
    assert all(re.search(r"gesv_panel_kernelIdLi16ELi\d+ELi4E", a) for a in agpr), agpr
    narrow = {}
    for k in kernels:
        m = _LU.search(k["name"])
        if not m:
            continue
        dt, n, nrhs, t, b, fact = m.group(1), *map(int, m.group(2, 3, 4, 5, 6))
        if b == 2 and n > 2:
            assert not fact, k["name"]                    # the factorization keeps four
            shape = (dt, n, nrhs, t)
            assert shape in EXTRA_WAVE, shape
            assert k["vgpr_count"] <= vgpr_budget(EXTRA_WAVE[shape]), (shape, k["vgpr_count"])
            narrow[shape] = k["vgpr_count"]
    assert set(narrow) == set(EXTRA_WAVE)
    # n = 32 float64, one right-hand side, 16-lane groups: three waves per SIMD
    assert narrow[("d", 32, 1, 16)] <= 168
