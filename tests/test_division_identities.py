"""Arithmetic identities the quantizer's kernels rely on, checked exhaustively.

- The scale division s_B = RN(M / q_max) (UFP4 hyper.ai summary: block scale
  as the absmax over the largest codebook level) is computed as a product
  with RN(1/q_max) corrected once by its fma remainder; for q_max = 1.75
  (E1M2), 7 (INT4) and 6 (E2M1) it must equal the IEEE quotient for every
  float in [1, 4) (host check, compiled with gcc; fmaf is correctly rounded).
- The reciprocal r = RN(1/s) the element quotients use comes from gfx950's
  reciprocal with one fma correction; that one is checked on the GPU (every
  mantissa in seven binades) through a test library that includes the
  kernels' own helper."""
import ctypes
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_scale_division_equals_ieee(tmp_path):
    exe = str(tmp_path / "div_identity")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", os.path.join(HERE, "div_identity.c"), "-o", exe,
                    "-lm"], check=True)
    out = subprocess.run([exe, "1.75", "7", "6"], capture_output=True, text=True, check=True).stdout
    assert [int(v) for v in out.split()] == [0, 0, 0]


@pytest.mark.gpu
def test_reciprocal_equals_ieee():
    lib_path = os.path.join(HERE, "libufp4_hwcheck.so")
    assert os.path.exists(lib_path), "tests/libufp4_hwcheck.so is built by __graft_entry__.build()"
    lib = ctypes.CDLL(lib_path)
    lib.ufp4_test_rcp_mismatches.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_uint)]
    lib.ufp4_test_rcp_mismatches.restype = ctypes.c_int
    for e in (-60, -30, -1, 0, 1, 30, 59):
        bad = ctypes.c_uint(0)
        assert lib.ufp4_test_rcp_mismatches(e, ctypes.byref(bad)) == 0
        assert bad.value == 0, (e, bad.value)
