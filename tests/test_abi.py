"""The C-ABI library on the CPU: it loads without a GPU, exports every symbol
include/ufp4.h declares, its structs match the header's layout, and every
argument error is rejected before any HIP call (so these run anywhere)."""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

import rht_bit_block_amd as U

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ufp4.h")

pytestmark = pytest.mark.skipif(not os.path.exists(U.LIB_PATH), reason="library not built")

FAKE = 0x10000  # aligned, never dereferenced: validation rejects first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ufp4_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = U.lib_handle()
    names = declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(U.EXPORTED) == names


def test_struct_layout_matches_header():
    src = r"""
#include <stdio.h>
#include <stddef.h>
#include "ufp4.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu %zu\n", sizeof(ufp4_quant_cfg), offsetof(ufp4_quant_cfg, sign_seed),
         offsetof(ufp4_quant_cfg, sr_stream), offsetof(ufp4_quant_cfg, tensor_scale),
         sizeof(ufp4_qtensor), offsetof(ufp4_qtensor, P), offsetof(ufp4_qtensor, cfg));
  return 0;
}
"""
    d = tempfile.mkdtemp()
    c = os.path.join(d, "layout.c")
    open(c, "w").write(src)
    exe = os.path.join(d, "layout")
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
    got = [int(v) for v in subprocess.run([exe], capture_output=True, text=True).stdout.split()]
    want = [ctypes.sizeof(U.QuantCfg), U.QuantCfg.sign_seed.offset, U.QuantCfg.sr_stream.offset,
            U.QuantCfg.tensor_scale.offset, ctypes.sizeof(U.QTensorC), U.QTensorC.P.offset,
            U.QTensorC.cfg.offset]
    assert got == want


def test_status_strings():
    for st in (0, -1, -2, -3, -4, -5):
        assert U.ufp4_status_string(st) != "unknown status"
    assert U.ufp4_status_string(-99) == "unknown status"


def _quant(lib, rows=64, cols=64, ld=64, along=0, cfg=None, x=FAKE, codes=FAKE, scales=FAKE):
    cfg = cfg or U.make_cfg()
    return lib.ufp4_rht_quant(ctypes.c_void_p(x), rows, cols, ld, along, ctypes.byref(cfg),
                              ctypes.c_void_p(codes), ctypes.c_void_p(scales), None, None)


def test_quant_argument_errors():
    lib = U.lib_handle()
    E = U
    assert _quant(lib, x=0) == E.UFP4_ERR_INVALID_ARG
    assert _quant(lib, codes=0) == E.UFP4_ERR_INVALID_ARG
    assert _quant(lib, rows=-1) == E.UFP4_ERR_INVALID_ARG
    assert _quant(lib, ld=32) == E.UFP4_ERR_INVALID_ARG            # ld < cols
    assert _quant(lib, along=2) == E.UFP4_ERR_INVALID_ARG
    assert _quant(lib, x=FAKE + 2) == E.UFP4_ERR_INVALID_ARG       # misaligned
    assert _quant(lib, cfg=U.make_cfg(grid=4)) == E.UFP4_ERR_INVALID_ARG
    assert _quant(lib, cfg=U.make_cfg(rht_n=24)) == E.UFP4_ERR_SHAPE
    assert _quant(lib, cfg=U.make_cfg(rht_n=256)) == E.UFP4_ERR_SHAPE
    assert _quant(lib, cols=48, ld=48, cfg=U.make_cfg(rht_n=32, block_cols=16)) == E.UFP4_ERR_SHAPE
    assert _quant(lib, cols=40, ld=48) == E.UFP4_ERR_SHAPE          # K % 16
    assert _quant(lib, cfg=U.make_cfg(block_cols=8)) == E.UFP4_ERR_UNSUPPORTED
    assert _quant(lib, cfg=U.make_cfg(sr_stream=0xFFFFFFFF)) == E.UFP4_ERR_UNSUPPORTED
    two_d = U.make_cfg(grid=U.UFP4_E2M1, scale_mode=U.UFP4_SCALE_POW2, block_rows=32,
                       block_cols=32, rht_n=1)
    assert _quant(lib, along=1, cfg=two_d) == E.UFP4_ERR_UNSUPPORTED
    assert _quant(lib, rows=48, cfg=two_d) == E.UFP4_ERR_SHAPE      # P % 32
    bad = two_d.copy(scale_mode=U.UFP4_SCALE_F32)
    assert _quant(lib, cfg=bad) == E.UFP4_ERR_UNSUPPORTED
    sq16 = two_d.copy(block_rows=16, block_cols=16)
    assert _quant(lib, rows=40, cfg=sq16) == E.UFP4_ERR_SHAPE      # P % 16
    assert _quant(lib, along=1, cfg=sq16) == E.UFP4_ERR_UNSUPPORTED
    assert _quant(lib, cfg=sq16.copy(rht_n=32)) == E.UFP4_ERR_UNSUPPORTED
    assert _quant(lib, cfg=sq16.copy(scale_mode=U.UFP4_SCALE_F32)) == E.UFP4_ERR_UNSUPPORTED
    assert _quant(lib, cfg=two_d.copy(block_rows=16)) == E.UFP4_ERR_UNSUPPORTED   # 16 x 32
    # 1D power-of-two scales only with the 1 x 32 MX block
    assert _quant(lib, cfg=U.make_cfg(scale_mode=U.UFP4_SCALE_POW2, block_cols=16)) == E.UFP4_ERR_UNSUPPORTED
    # two-level scaling: a positive, finite, normal factor, power-of-two scales only
    pow2 = U.make_cfg(scale_mode=U.UFP4_SCALE_POW2, block_cols=32, rht_n=32)
    for ts in (-1.0, float("nan"), float("inf"), 1e-40):
        assert _quant(lib, cfg=pow2.copy(tensor_scale=ts)) == E.UFP4_ERR_INVALID_ARG, ts
    assert _quant(lib, cfg=U.make_cfg(tensor_scale=0.5)) == E.UFP4_ERR_UNSUPPORTED   # fp32 scales
    assert _quant(lib, rows=0, cfg=pow2.copy(tensor_scale=0.5)) == E.UFP4_OK
    # empty inputs are a successful no-op (no HIP call is made)
    assert _quant(lib, rows=0) == E.UFP4_OK
    assert _quant(lib, cols=0, ld=0) == E.UFP4_OK


def _qt(P, K, cfg=None, codes=FAKE, scales=FAKE):
    return U.QTensorC(codes, scales, P, K, cfg or U.make_cfg())


def test_gemm_argument_errors():
    lib = U.lib_handle()
    a, b = _qt(64, 64), _qt(32, 64)
    f = lib.ufp4_gemm_fprop
    assert f(None, ctypes.byref(b), ctypes.c_void_p(FAKE), 32, None) == U.UFP4_ERR_INVALID_ARG
    assert f(ctypes.byref(a), ctypes.byref(b), None, 32, None) == U.UFP4_ERR_INVALID_ARG
    assert f(ctypes.byref(a), ctypes.byref(b), ctypes.c_void_p(FAKE), 16, None) == U.UFP4_ERR_INVALID_ARG
    bk = _qt(32, 128)
    assert f(ctypes.byref(a), ctypes.byref(bk), ctypes.c_void_p(FAKE), 32, None) == U.UFP4_ERR_MISMATCH
    for kw in ({"grid": U.UFP4_INT4}, {"rht_n": 32}, {"sign_seed": 5}):
        bm = _qt(32, 64, U.make_cfg(**kw))
        assert f(ctypes.byref(a), ctypes.byref(bm), ctypes.c_void_p(FAKE), 32, None) == U.UFP4_ERR_MISMATCH
    # sign seeds may differ when there is no rotation
    a1, b1 = _qt(0, 64, U.make_cfg(rht_n=1, sign_seed=1)), _qt(32, 64, U.make_cfg(rht_n=1, sign_seed=2))
    assert f(ctypes.byref(a1), ctypes.byref(b1), ctypes.c_void_p(FAKE), 32, None) == U.UFP4_OK
    # grouped: offsets must start at 0, end at P, ascend, G in [1, 64]
    g = lib.ufp4_gemm_fprop_grouped
    wb = _qt(4 * 32, 64)
    ok_off = (ctypes.c_int64 * 5)(0, 16, 16, 48, 64)
    bad_off = (ctypes.c_int64 * 5)(0, 32, 16, 48, 64)
    assert g(ctypes.byref(a), ctypes.byref(wb), 4, bad_off, ctypes.c_void_p(FAKE), 32, None) == U.UFP4_ERR_INVALID_ARG
    assert g(ctypes.byref(a), ctypes.byref(wb), 65, ok_off, ctypes.c_void_p(FAKE), 32, None) == U.UFP4_ERR_INVALID_ARG
    assert g(ctypes.byref(a), ctypes.byref(_qt(3 * 32 + 1, 64)), 4, ok_off, ctypes.c_void_p(FAKE), 32, None) == U.UFP4_ERR_SHAPE


def test_gemm_workspace_errors():
    """ufp4_gemm_ws / ufp4_gemm_workspace_bytes: sizes come from metadata
    alone; a bad op, a null workspace with a size, a workspace smaller than
    asked for or not 256-byte aligned are rejected before any HIP call."""
    lib = U.lib_handle()
    pow2 = U.make_cfg(U.UFP4_E1M2, U.UFP4_RTNE, U.UFP4_SCALE_POW2, 1, 32, 1)
    a, b = _qt(300, 256, pow2), _qt(64, 256, pow2)
    wb = lib.ufp4_gemm_workspace_bytes
    need = (300 * 256 + 255) // 256 * 256 + 64 * 256      # FP6: one byte per element
    for op in (U.UFP4_GEMM_FPROP, U.UFP4_GEMM_DGRAD, U.UFP4_GEMM_WGRAD):
        assert wb(op, ctypes.byref(a), ctypes.byref(b), 0) == need
    assert wb(3, ctypes.byref(a), ctypes.byref(b), 0) == 0
    e2m1 = pow2.copy(grid=U.UFP4_E2M1)
    assert wb(0, ctypes.byref(_qt(300, 256, e2m1)), ctypes.byref(_qt(64, 256, e2m1)), 0) == 0
    assert wb(0, ctypes.byref(_qt(300, 160, pow2)), ctypes.byref(_qt(64, 160, pow2)), 0) == 0
    assert wb(0, ctypes.byref(_qt(300, 256)), ctypes.byref(_qt(64, 256)), 0) == 0   # fp32 scales
    assert wb(0, None, ctypes.byref(b), 0) == 0
    f = lib.ufp4_gemm_ws
    C = ctypes.c_void_p(FAKE)
    ab = (ctypes.byref(a), ctypes.byref(b))
    assert f(3, *ab, 0, None, C, 64, ctypes.c_void_p(FAKE), need, None) == U.UFP4_ERR_INVALID_ARG
    assert f(0, *ab, -1, None, C, 64, ctypes.c_void_p(FAKE), need, None) == U.UFP4_ERR_INVALID_ARG
    assert f(0, *ab, 0, None, C, 64, None, need, None) == U.UFP4_ERR_INVALID_ARG
    assert f(0, *ab, 0, None, C, 64, ctypes.c_void_p(FAKE), need - 1, None) == U.UFP4_ERR_INVALID_ARG
    assert f(0, *ab, 0, None, C, 64, ctypes.c_void_p(FAKE + 16), need, None) == U.UFP4_ERR_INVALID_ARG
    assert f(0, *ab, 0, None, None, 64, ctypes.c_void_p(FAKE), need, None) == U.UFP4_ERR_INVALID_ARG
    assert f(0, *ab, 0, None, C, 63, ctypes.c_void_p(FAKE), need, None) == U.UFP4_ERR_INVALID_ARG
    assert f(0, ctypes.byref(a), ctypes.byref(_qt(64, 128, pow2)), 0, None, C, 64,
             ctypes.c_void_p(FAKE), need, None) == U.UFP4_ERR_MISMATCH
    # grouped WGRAD with E8M0 blocks: segments must be multiples of 128
    seg = (ctypes.c_int64 * 3)(0, 96, 256)
    g = lib.ufp4_gemm_wgrad_grouped
    assert g(*ab, 2, seg, C, 256, None) == U.UFP4_ERR_UNSUPPORTED
    assert f(2, *ab, 2, seg, C, 256, ctypes.c_void_p(FAKE), need, None) == U.UFP4_ERR_UNSUPPORTED
    assert wb(2, ctypes.byref(a), ctypes.byref(b), 2) == need
    sq = U.make_cfg(U.UFP4_E1M2, U.UFP4_RTNE, U.UFP4_SCALE_POW2, 32, 32, 1)   # 32 x 32 blocks
    assert wb(0, ctypes.byref(_qt(320, 256, sq)), ctypes.byref(_qt(96, 256, sq)), 4) == 0   # 24-row groups
    assert wb(0, ctypes.byref(_qt(320, 256, sq)), ctypes.byref(_qt(128, 256, sq)), 4) > 0
    assert wb(0, ctypes.byref(a), ctypes.byref(_qt(128, 256, pow2)), 4) == need - 64 * 256 + 128 * 256
    # empty operands: nothing to do, the workspace is not touched
    assert f(0, ctypes.byref(_qt(0, 256, pow2)), ctypes.byref(b), 0, None, C, 64,
             ctypes.c_void_p(FAKE), 1, None) == U.UFP4_OK


def test_segmented_and_misc_errors():
    lib = U.lib_handle()
    cfg = U.make_cfg(rht_n=32, block_cols=32)
    off = (ctypes.c_int64 * 3)(0, 48, 96)                      # 48 % 32 != 0
    st = lib.ufp4_rht_quant_segmented(ctypes.c_void_p(FAKE), 96, 64, 64, off, 2, ctypes.byref(cfg),
                                      ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), None)
    assert st == U.UFP4_ERR_SHAPE
    off2 = (ctypes.c_int64 * 3)(0, 32, 64)                     # does not end at rows
    st = lib.ufp4_rht_quant_segmented(ctypes.c_void_p(FAKE), 96, 64, 64, off2, 2, ctypes.byref(cfg),
                                      ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), None)
    assert st == U.UFP4_ERR_INVALID_ARG
    assert lib.ufp4_philox_fill(1, 0xFFFFFFFF, 0, 8, ctypes.c_void_p(FAKE), None) == U.UFP4_ERR_UNSUPPORTED
    assert lib.ufp4_philox_fill(1, 0, 0, -1, ctypes.c_void_p(FAKE), None) == U.UFP4_ERR_INVALID_ARG
    q = _qt(64, 64)                                            # 1D blocks cannot be transposed
    assert lib.ufp4_transpose_qtensor(ctypes.byref(q), ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), None) == U.UFP4_ERR_UNSUPPORTED
    assert lib.ufp4_dequant(ctypes.byref(q), None, 64, None) == U.UFP4_ERR_INVALID_ARG


def test_stream_copy_errors():
    lib = U.lib_handle()
    vp = ctypes.c_void_p
    assert lib.ufp4_stream_copy(None, None, 0, None) == U.UFP4_OK              # nothing to do
    assert lib.ufp4_stream_copy(vp(FAKE), vp(FAKE + 4096), -1, None) == U.UFP4_ERR_INVALID_ARG
    assert lib.ufp4_stream_copy(None, vp(FAKE), 16, None) == U.UFP4_ERR_INVALID_ARG
    assert lib.ufp4_stream_copy(vp(FAKE), None, 16, None) == U.UFP4_ERR_INVALID_ARG
    assert lib.ufp4_stream_copy(vp(FAKE + 8), vp(FAKE + 4096), 16, None) == U.UFP4_ERR_INVALID_ARG
    assert lib.ufp4_stream_copy(vp(FAKE), vp(FAKE + 4104), 16, None) == U.UFP4_ERR_INVALID_ARG
    # overlapping ranges, either order
    assert lib.ufp4_stream_copy(vp(FAKE), vp(FAKE + 64), 128, None) == U.UFP4_ERR_INVALID_ARG
    assert lib.ufp4_stream_copy(vp(FAKE + 64), vp(FAKE), 128, None) == U.UFP4_ERR_INVALID_ARG


def test_size_helpers():
    cfg = U.make_cfg()
    assert U.ufp4_codes_bytes(8192, 2048) == 8192 * 1024
    assert U.ufp4_scales_bytes(8192, 2048, cfg) == 8192 * 128 * 4
    c2 = U.make_cfg(scale_mode=U.UFP4_SCALE_POW2, block_rows=32, block_cols=32, rht_n=1)
    assert U.ufp4_scales_bytes(4096, 4096, c2) == 128 * 128


def _dual(lib, rows=64, cols=64, ld=64, offs=None, cfg_r=None, cfg_c=None, x=FAKE, ptr=FAKE):
    cr, cc = cfg_r or U.make_cfg(sign_seed=1), cfg_c or U.make_cfg(sign_seed=2)
    off = (ctypes.c_int64 * len(offs))(*offs) if offs is not None else None
    n = len(offs) - 1 if offs is not None else 1
    p = ctypes.c_void_p(ptr)
    return lib.ufp4_rht_quant_dual(ctypes.c_void_p(x), rows, cols, ld, off, n, ctypes.byref(cr),
                                   ctypes.byref(cc), p, p, p, p, None)


def test_dual_quant_argument_errors():
    lib = U.lib_handle()
    E = U
    assert _dual(lib, x=0) == E.UFP4_ERR_INVALID_ARG
    assert _dual(lib, ptr=0) == E.UFP4_ERR_INVALID_ARG
    assert _dual(lib, ld=32) == E.UFP4_ERR_INVALID_ARG
    # the two sides may differ only in signs and draws
    assert _dual(lib, cfg_c=U.make_cfg(grid=U.UFP4_INT4)) == E.UFP4_ERR_UNSUPPORTED
    assert _dual(lib, cfg_c=U.make_cfg(rounding=U.UFP4_SR)) == E.UFP4_ERR_UNSUPPORTED
    assert _dual(lib, cfg_c=U.make_cfg(rht_n=32)) == E.UFP4_ERR_UNSUPPORTED
    big = U.make_cfg(rht_n=128)   # n = 128: both axes in multiples of 128
    assert _dual(lib, rows=64, cols=128, ld=128, cfg_r=big, cfg_c=big) == E.UFP4_ERR_SHAPE
    assert _dual(lib, rows=128, cols=64, ld=64, cfg_r=big, cfg_c=big) == E.UFP4_ERR_SHAPE
    assert _dual(lib, rows=40) == E.UFP4_ERR_SHAPE                  # rows % 16
    assert _dual(lib, cols=40, ld=48) == E.UFP4_ERR_SHAPE           # cols % 16
    assert _dual(lib, offs=[0, 24, 64]) == E.UFP4_ERR_SHAPE         # segment % 16
    assert _dual(lib, offs=[0, 32, 48]) == E.UFP4_ERR_INVALID_ARG   # must end at rows
    assert _dual(lib, offs=[8, 64]) == E.UFP4_ERR_INVALID_ARG       # must start at 0
    two_d = U.make_cfg(grid=U.UFP4_E2M1, scale_mode=U.UFP4_SCALE_POW2, block_rows=32,
                       block_cols=32, rht_n=1)
    assert _dual(lib, cfg_r=two_d, cfg_c=two_d) == E.UFP4_ERR_UNSUPPORTED
    assert _dual(lib, rows=0) == E.UFP4_OK


def _diag(lib, x=FAKE, rows=64, cols=64, ld=64, cfg=None, stats=FAKE, ws=FAKE):
    c = cfg or U.make_cfg()
    return lib.ufp4_quant_diag(ctypes.c_void_p(x), rows, cols, ld, ctypes.byref(c),
                               ctypes.c_void_p(stats), ctypes.c_void_p(ws), None)


def test_diag_argument_errors():
    """Every call here fails validation (a valid call launches a kernel even
    for an empty operand, since it zeroes stats)."""
    lib = U.lib_handle()
    E = U
    assert _diag(lib, stats=0) == E.UFP4_ERR_INVALID_ARG
    assert _diag(lib, ws=0) == E.UFP4_ERR_INVALID_ARG               # workspace required
    assert _diag(lib, ws=FAKE + 4) == E.UFP4_ERR_INVALID_ARG        # 8-byte alignment
    assert _diag(lib, rows=0, ws=0) == E.UFP4_ERR_INVALID_ARG
    assert _diag(lib, stats=FAKE + 4) == E.UFP4_ERR_INVALID_ARG     # 8-byte alignment
    assert _diag(lib, rows=0, stats=0) == E.UFP4_ERR_INVALID_ARG
    assert _diag(lib, x=0) == E.UFP4_ERR_INVALID_ARG
    assert _diag(lib, x=FAKE + 2) == E.UFP4_ERR_INVALID_ARG
    assert _diag(lib, rows=-1) == E.UFP4_ERR_INVALID_ARG
    assert _diag(lib, ld=32) == E.UFP4_ERR_INVALID_ARG
    assert _diag(lib, ld=68) == E.UFP4_ERR_INVALID_ARG              # ld % 8
    assert _diag(lib, cols=40, ld=48) == E.UFP4_ERR_SHAPE            # K % 16
    assert _diag(lib, cfg=U.make_cfg(rht_n=24)) == E.UFP4_ERR_SHAPE
    two_d = U.make_cfg(grid=U.UFP4_E2M1, scale_mode=U.UFP4_SCALE_POW2, block_rows=32,
                       block_cols=32, rht_n=1)
    assert _diag(lib, cfg=two_d) == E.UFP4_ERR_UNSUPPORTED
    assert _diag(lib, cfg=U.make_cfg(scale_mode=U.UFP4_SCALE_POW2, block_cols=16)) == E.UFP4_ERR_UNSUPPORTED


def test_mxfp8_argument_errors():
    """MXFP8 (E4M3) only with 1 x 32 power-of-two blocks and RTNE, only on
    the row/column quantizer, dequant and the dense GEMMs."""
    lib = U.lib_handle()
    E = U
    mx = U.make_cfg(grid=U.UFP4_E4M3, scale_mode=U.UFP4_SCALE_POW2, block_cols=32, rht_n=16)
    assert _quant(lib, cfg=mx.copy(rounding=U.UFP4_SR)) == E.UFP4_ERR_UNSUPPORTED
    assert _quant(lib, cfg=mx.copy(scale_mode=U.UFP4_SCALE_F32)) == E.UFP4_ERR_UNSUPPORTED
    assert _quant(lib, cfg=mx.copy(block_cols=16)) == E.UFP4_ERR_UNSUPPORTED
    assert _quant(lib, cfg=mx.copy(block_rows=32, rht_n=1)) == E.UFP4_ERR_UNSUPPORTED
    assert _quant(lib, cfg=U.make_cfg(grid=4)) == E.UFP4_ERR_INVALID_ARG
    assert _diag(lib, cfg=mx) == E.UFP4_ERR_UNSUPPORTED
    assert _dual(lib, cfg_r=mx, cfg_c=mx) == E.UFP4_ERR_UNSUPPORTED
    a = _qt(64, 160, mx.copy(rht_n=1))
    b = _qt(64, 160, mx.copy(rht_n=1))
    assert lib.ufp4_gemm_fprop(ctypes.byref(a), ctypes.byref(b), ctypes.c_void_p(FAKE), 64, None) == E.UFP4_ERR_UNSUPPORTED
    a = _qt(64, 256, mx)
    b = _qt(64, 256, mx)
    offs = (ctypes.c_int64 * 3)(0, 32, 64)
    assert lib.ufp4_gemm_fprop_grouped(ctypes.byref(a), ctypes.byref(b), 2, offs, ctypes.c_void_p(FAKE), 32, None) == E.UFP4_ERR_UNSUPPORTED
    assert lib.ufp4_gemm_wgrad_grouped(ctypes.byref(a), ctypes.byref(b), 2, offs, ctypes.c_void_p(FAKE), 64, None) == E.UFP4_ERR_UNSUPPORTED
