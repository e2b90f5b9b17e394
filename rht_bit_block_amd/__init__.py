"""Python binding of the UFP4 hot-path library (librht_ufp4.so, C ABI in
include/ufp4.h).

Argument marshalling only: torch supplies device memory and the current HIP
stream; every step of the path runs in the library's HIP kernels.  There is
no CPU fallback -- if the library is missing, every call raises.

Functions carry the C names (ufp4_rht_quant, ufp4_gemm_fprop, ...).  Outputs
that the caller does not pass are allocated with torch on the input's device.
"""
import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# UFP4_LIBRARY names another build of the same library (the sanitizer build
# of rht_bit_block_amd.build for CPU runs of the ABI tests).
LIB_PATH = os.environ.get("UFP4_LIBRARY") or os.path.join(_HERE, "librht_ufp4.so")

UFP4_E1M2, UFP4_INT4, UFP4_E2M1, UFP4_E4M3 = 0, 1, 2, 3
UFP4_RTNE, UFP4_SR = 0, 1
UFP4_SCALE_F32, UFP4_SCALE_POW2 = 0, 1
UFP4_OK, UFP4_ERR_INVALID_ARG, UFP4_ERR_SHAPE = 0, -1, -2
UFP4_ERR_MISMATCH, UFP4_ERR_UNSUPPORTED, UFP4_ERR_HIP = -3, -4, -5
UFP4_GEMM_FPROP, UFP4_GEMM_DGRAD, UFP4_GEMM_WGRAD = 0, 1, 2

EXPORTED = [
    "ufp4_rht_quant", "ufp4_rht_quant_segmented", "ufp4_rht_quant_dual", "ufp4_quant_diag",
    "ufp4_quant_diag_noalloc",
    "ufp4_dequant",
    "ufp4_gemm_fprop", "ufp4_gemm_dgrad", "ufp4_gemm_wgrad",
    "ufp4_gemm_fprop_grouped", "ufp4_gemm_dgrad_grouped", "ufp4_gemm_wgrad_grouped",
    "ufp4_gemm_workspace_bytes", "ufp4_gemm_ws",
    "ufp4_transpose_qtensor", "ufp4_codes_bytes", "ufp4_scales_bytes",
    "ufp4_philox_fill", "ufp4_stream_copy", "ufp4_status_string",
]


class UFP4Error(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        msg = _lib().ufp4_status_string(status).decode()
        super().__init__(f"{fn} failed: {msg} ({status})")


class QuantCfg(ctypes.Structure):
    _fields_ = [("grid", ctypes.c_int32), ("rounding", ctypes.c_int32),
                ("scale_mode", ctypes.c_int32), ("block_rows", ctypes.c_int32),
                ("block_cols", ctypes.c_int32), ("rht_n", ctypes.c_int32),
                ("sign_seed", ctypes.c_uint64), ("sr_seed", ctypes.c_uint64),
                ("sr_stream", ctypes.c_uint32), ("tensor_scale", ctypes.c_float)]

    def copy(self, **kw):
        c = QuantCfg()
        ctypes.memmove(ctypes.byref(c), ctypes.byref(self), ctypes.sizeof(QuantCfg))
        for k, v in kw.items():
            setattr(c, k, v)
        return c


def make_cfg(grid=UFP4_E1M2, rounding=UFP4_RTNE, scale_mode=UFP4_SCALE_F32, block_rows=1,
             block_cols=16, rht_n=16, sign_seed=0, sr_seed=0, sr_stream=0, tensor_scale=0.0):
    """tensor_scale: 0 (single-level) or the per-tensor fp32 factor of
    two-level scaling over power-of-two block scales."""
    return QuantCfg(int(grid), int(rounding), int(scale_mode), int(block_rows), int(block_cols),
                    int(rht_n), int(sign_seed), int(sr_seed), int(sr_stream), float(tensor_scale))


class QTensorC(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("P", ctypes.c_int64), ("K", ctypes.c_int64), ("cfg", QuantCfg)]


@dataclass
class QTensor:
    """A quantized logical operand: codes uint8 [P, K/2], scales (fp32 or
    E8M0 uint8) per block, both on the GPU."""
    codes: torch.Tensor
    scales: torch.Tensor
    P: int
    K: int
    cfg: QuantCfg

    def c(self):
        dev = self.codes.device if isinstance(self.codes, torch.Tensor) else None
        _check_buffer("codes", self.codes, torch.uint8, _codes_elems(self.P, self.K, self.cfg), dev)
        _check_buffer("scales", self.scales, scales_dtype(self.cfg),
                      _scales_elems(self.P, self.K, self.cfg), dev)
        if self.P and self.K:
            _on_gpu(self.codes, "codes")
        return QTensorC(self.codes.data_ptr(), self.scales.data_ptr(), self.P, self.K, self.cfg)


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() or "
                               "python -m rht_bit_block_amd.build")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, u64, u32 = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                  ctypes.c_uint64, ctypes.c_uint32)
        cfgp, qtp = ctypes.POINTER(QuantCfg), ctypes.POINTER(QTensorC)
        i64p = ctypes.POINTER(ctypes.c_int64)
        sig = {
            "ufp4_rht_quant": [vp, i64, i64, i64, i32, cfgp, vp, vp, vp, vp],
            "ufp4_rht_quant_segmented": [vp, i64, i64, i64, i64p, i32, cfgp, vp, vp, vp],
            "ufp4_rht_quant_dual": [vp, i64, i64, i64, i64p, i32, cfgp, cfgp, vp, vp, vp, vp, vp],
            "ufp4_quant_diag": [vp, i64, i64, i64, cfgp, vp, vp, vp],
            "ufp4_quant_diag_noalloc": [vp, i64, i64, i64, cfgp, vp, vp],
            "ufp4_dequant": [qtp, vp, i64, vp],
            "ufp4_gemm_fprop": [qtp, qtp, vp, i64, vp],
            "ufp4_gemm_dgrad": [qtp, qtp, vp, i64, vp],
            "ufp4_gemm_wgrad": [qtp, qtp, vp, i64, vp],
            "ufp4_gemm_fprop_grouped": [qtp, qtp, i32, i64p, vp, i64, vp],
            "ufp4_gemm_dgrad_grouped": [qtp, qtp, i32, i64p, vp, i64, vp],
            "ufp4_gemm_wgrad_grouped": [qtp, qtp, i32, i64p, vp, i64, vp],
            "ufp4_gemm_ws": [i32, qtp, qtp, i32, i64p, vp, i64, vp, ctypes.c_size_t, vp],
            "ufp4_transpose_qtensor": [qtp, vp, vp, vp],
            "ufp4_philox_fill": [u64, u32, u64, i64, vp, vp],
            "ufp4_stream_copy": [vp, vp, i64, vp],
        }
        for name, args in sig.items():
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        lib.ufp4_gemm_workspace_bytes.argtypes = [i32, qtp, qtp, i32]
        lib.ufp4_gemm_workspace_bytes.restype = ctypes.c_size_t
        lib.ufp4_codes_bytes.argtypes = [i64, i64]
        lib.ufp4_codes_bytes.restype = ctypes.c_size_t
        lib.ufp4_scales_bytes.argtypes = [i64, i64, cfgp]
        lib.ufp4_scales_bytes.restype = ctypes.c_size_t
        lib.ufp4_status_string.argtypes = [ctypes.c_int]
        lib.ufp4_status_string.restype = ctypes.c_char_p
        _LIB = lib
    return _LIB


def lib_handle():
    """The loaded ctypes library (raises if it is not built)."""
    return _lib()


def _check(fn, st):
    if st != UFP4_OK:
        raise UFP4Error(fn, st)


def _stream(t: Optional[torch.Tensor] = None):
    if t is not None and t.is_cuda:
        return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _i64arr(vals: Sequence[int]):
    arr = (ctypes.c_int64 * len(vals))(*[int(v) for v in vals])
    return arr


# ---------------------------------------------------------------------------
# Buffer checks.  The C ABI takes raw device pointers and cannot know buffer
# sizes, so the binding checks every tensor it hands over (dtype, device,
# unit inner stride, size) and raises ValueError before the call.
# ---------------------------------------------------------------------------
def _codes_elems(P, K, cfg):
    return P * K if cfg.grid == UFP4_E4M3 else P * ((K + 1) // 2)


def _scales_elems(P, K, cfg):
    br, bc = max(1, cfg.block_rows), max(1, cfg.block_cols)
    return ((P + br - 1) // br) * ((K + bc - 1) // bc)


def _check_buffer(name, t, dtype, min_elems, device=None):
    """A flat buffer of at least min_elems elements: dtype, device, and
    contiguous storage (the library writes it densely)."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if min_elems == 0:
        return
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < min_elems:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {min_elems}")
    if (device is None and not t.is_cuda) or (device is not None and t.device != device):
        raise ValueError(f"{name} must be on {device if device is not None else 'a GPU'}")


def _check_matrix(name, t, rows, cols, device):
    """An fp32 output matrix of at least rows x cols, unit column stride
    (the row pitch is passed to the library as its leading dimension)."""
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.dim() != 2:
        raise ValueError(f"{name} must be a 2-D float32 tensor")
    if rows == 0 or cols == 0:
        return
    if t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride")
    if t.shape[0] < rows or t.shape[1] < cols:
        raise ValueError(f"{name} has shape {tuple(t.shape)}, needs at least ({rows}, {cols})")
    if t.stride(0) < cols:
        raise ValueError(f"{name} row pitch {t.stride(0)} is below its {cols} columns")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}")


def _check_x(x):
    if not isinstance(x, torch.Tensor) or x.dtype != torch.bfloat16 or x.dim() != 2:
        raise ValueError("x must be a 2-D bfloat16 tensor")
    if x.stride(1) != 1:
        raise ValueError("x must be row-major (unit column stride)")


def _on_gpu(x, name="x"):
    """Checked last, after the outputs (which must sit on x's device)."""
    if x.numel() and not x.is_cuda:
        raise ValueError(f"{name} must be on a GPU")


def codes_shape(P, K, cfg):
    """4-bit codes two per byte; E4M3 (MXFP8) codes one per byte."""
    return (P, K) if cfg.grid == UFP4_E4M3 else (P, K // 2)


def scales_shape(P, K, cfg):
    return (P // cfg.block_rows, K // cfg.block_cols)


def scales_dtype(cfg):
    return torch.float32 if cfg.scale_mode == UFP4_SCALE_F32 else torch.uint8


# ---------------------------------------------------------------------------
# Entry points (same names as the C ABI)
# ---------------------------------------------------------------------------
def ufp4_rht_quant(x: torch.Tensor, along: int, cfg: QuantCfg, codes=None, scales=None,
                   rotated=False, ld: Optional[int] = None):
    """Quantize bf16 x [rows, cols] (row-major, row pitch ld).  Returns
    (QTensor, rotated fp32 [P, K] or None)."""
    _check_x(x)
    rows, cols = x.shape
    ld = x.stride(0) if ld is None else ld
    P, K = (cols, rows) if along else (rows, cols)
    dev = x.device
    if codes is None:
        codes = torch.empty(codes_shape(P, K, cfg), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty(scales_shape(P, K, cfg), dtype=scales_dtype(cfg), device=dev)
    _check_buffer("codes", codes, torch.uint8, _codes_elems(P, K, cfg), dev)
    _check_buffer("scales", scales, scales_dtype(cfg), _scales_elems(P, K, cfg), dev)
    rot = torch.empty((P, K), dtype=torch.float32, device=dev) if rotated is True else (
        rotated if isinstance(rotated, torch.Tensor) else None)
    if rot is not None:
        _check_matrix("rotated", rot, P, K, dev)
        if rot.stride(0) != K:
            raise ValueError("rotated must be a dense [P, K] tensor")
    _on_gpu(x)
    st = _lib().ufp4_rht_quant(_ptr(x), rows, cols, ld, int(along), ctypes.byref(cfg),
                               _ptr(codes), _ptr(scales), _ptr(rot), _stream(x))
    _check("ufp4_rht_quant", st)
    return QTensor(codes, scales, P, K, cfg), rot


DIAG_WORKSPACE_BYTES = 8192   # UFP4_DIAG_WORKSPACE_BYTES


def ufp4_quant_diag(x: torch.Tensor, cfg: QuantCfg, stats=None, ld: Optional[int] = None,
                    workspace=None):
    """Level statistics of the row-wise quantization of bf16 x [rows, cols]:
    int64 [16] on x's device -- [0:8] element counts per magnitude level index,
    [8:16] sums of rint((L_k - |t|) * 2^28) (see the C header).  workspace:
    uint8 device buffer of DIAG_WORKSPACE_BYTES (allocated when not given)."""
    _check_x(x)
    rows, cols = x.shape
    ld = x.stride(0) if ld is None else ld
    if stats is None:
        stats = torch.empty(16, dtype=torch.int64, device=x.device)
    if workspace is None:
        workspace = torch.empty(DIAG_WORKSPACE_BYTES, dtype=torch.uint8, device=x.device)
    _check_buffer("stats", stats, torch.int64, 16, x.device)
    _check_buffer("workspace", workspace, torch.uint8, DIAG_WORKSPACE_BYTES, x.device)
    _on_gpu(x)
    st = _lib().ufp4_quant_diag(_ptr(x), rows, cols, ld, ctypes.byref(cfg), _ptr(stats),
                                _ptr(workspace), _stream(x))
    _check("ufp4_quant_diag", st)
    return stats


def ufp4_quant_diag_noalloc(x: torch.Tensor, cfg: QuantCfg, stats=None, ld: Optional[int] = None):
    """ufp4_quant_diag on the library's per-GPU scratch array instead of a
    workspace (for callers that cannot allocate; calls that overlap on one
    GPU race).  Returns the int64 [16] statistics."""
    _check_x(x)
    rows, cols = x.shape
    ld = x.stride(0) if ld is None else ld
    if stats is None:
        stats = torch.empty(16, dtype=torch.int64, device=x.device)
    _check_buffer("stats", stats, torch.int64, 16, x.device)
    _on_gpu(x)
    st = _lib().ufp4_quant_diag_noalloc(_ptr(x), rows, cols, ld, ctypes.byref(cfg), _ptr(stats),
                                        _stream(x))
    _check("ufp4_quant_diag_noalloc", st)
    return stats


def ufp4_rht_quant_segmented(x: torch.Tensor, row_offsets: Sequence[int], cfg: QuantCfg,
                             codes=None, scales=None):
    """Column-wise quantization of row segments of x (per-expert transposed
    operands).  Returns a QTensor with P = cols and K = rows whose storage is
    segment-major (segment g: [cols, L_g] at element offset cols*offset_g)."""
    _check_x(x)
    rows, cols = x.shape
    dev = x.device
    if codes is None:
        codes = torch.empty(cols * rows // 2, dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty(cols * rows // cfg.block_cols, dtype=scales_dtype(cfg), device=dev)
    _check_buffer("codes", codes, torch.uint8, _codes_elems(cols, rows, cfg), dev)
    _check_buffer("scales", scales, scales_dtype(cfg), _scales_elems(cols, rows, cfg), dev)
    _on_gpu(x)
    off = _i64arr(row_offsets)
    st = _lib().ufp4_rht_quant_segmented(_ptr(x), rows, cols, x.stride(0), off,
                                         len(row_offsets) - 1, ctypes.byref(cfg), _ptr(codes),
                                         _ptr(scales), _stream(x))
    _check("ufp4_rht_quant_segmented", st)
    return QTensor(codes, scales, cols, rows, cfg)


def ufp4_rht_quant_dual(x: torch.Tensor, cfg_row: QuantCfg, cfg_col: QuantCfg,
                        row_offsets: Optional[Sequence[int]] = None, out_row=None, out_col=None):
    """Row-wise (A = x, K = cols) and column-wise (A = x^T, K = rows, or per
    row segment when row_offsets is given) quantization from one read of x.
    Returns (QTensor row, QTensor col); out_row / out_col: optional
    (codes, scales) pairs to write into."""
    _check_x(x)
    rows, cols = x.shape
    dev = x.device
    cr, sr = out_row if out_row is not None else (
        torch.empty(rows * cols // 2, dtype=torch.uint8, device=dev),
        torch.empty(rows * cols // cfg_row.block_cols, dtype=scales_dtype(cfg_row), device=dev))
    cc, sc = out_col if out_col is not None else (
        torch.empty(rows * cols // 2, dtype=torch.uint8, device=dev),
        torch.empty(rows * cols // cfg_col.block_cols, dtype=scales_dtype(cfg_col), device=dev))
    _check_buffer("codes_row", cr, torch.uint8, _codes_elems(rows, cols, cfg_row), dev)
    _check_buffer("scales_row", sr, scales_dtype(cfg_row), _scales_elems(rows, cols, cfg_row), dev)
    _check_buffer("codes_col", cc, torch.uint8, _codes_elems(cols, rows, cfg_col), dev)
    _check_buffer("scales_col", sc, scales_dtype(cfg_col), _scales_elems(cols, rows, cfg_col), dev)
    _on_gpu(x)
    off = _i64arr(row_offsets) if row_offsets is not None else None
    nseg = len(row_offsets) - 1 if row_offsets is not None else 1
    st = _lib().ufp4_rht_quant_dual(_ptr(x), rows, cols, x.stride(0), off, nseg,
                                    ctypes.byref(cfg_row), ctypes.byref(cfg_col), _ptr(cr),
                                    _ptr(sr), _ptr(cc), _ptr(sc), _stream(x))
    _check("ufp4_rht_quant_dual", st)
    return QTensor(cr, sr, rows, cols, cfg_row), QTensor(cc, sc, cols, rows, cfg_col)


def stacked(q: QTensor, groups: int) -> QTensor:
    """View a segmented column-wise quantization with equal segments (e.g.
    W^T of every expert) as one operand stacked along P: [G*cols, L]."""
    return QTensor(q.codes, q.scales, q.P * groups, q.K // groups, q.cfg)


def ufp4_dequant(q: QTensor, out=None):
    if out is None:
        out = torch.empty((q.P, q.K), dtype=torch.float32, device=q.codes.device)
    qc = q.c()
    _check_matrix("out", out, q.P, q.K, q.codes.device)
    st = _lib().ufp4_dequant(ctypes.byref(qc), _ptr(out), out.stride(0), _stream(out))
    _check("ufp4_dequant", st)
    return out


def _gemm(name, A: QTensor, B: QTensor, out=None):
    if out is None:
        out = torch.empty((A.P, B.P), dtype=torch.float32, device=A.codes.device)
    a, b = A.c(), B.c()
    _check_matrix("out", out, A.P, B.P, A.codes.device)
    st = getattr(_lib(), name)(ctypes.byref(a), ctypes.byref(b), _ptr(out), out.stride(0),
                               _stream(out))
    _check(name, st)
    return out


def ufp4_gemm_fprop(X: QTensor, W: QTensor, out=None):
    """Y = X W^T on the quantized rotated operands (fp32 [M, N])."""
    return _gemm("ufp4_gemm_fprop", X, W, out)


def ufp4_gemm_dgrad(dY: QTensor, Wt: QTensor, out=None):
    """dX = dY W, with Wt the column-wise quantization of W (fp32 [M, K_in])."""
    return _gemm("ufp4_gemm_dgrad", dY, Wt, out)


def ufp4_gemm_wgrad(dYt: QTensor, Xt: QTensor, out=None):
    """dW = dY^T X from the column-wise quantizations of dY and X (fp32 [N, K_in])."""
    return _gemm("ufp4_gemm_wgrad", dYt, Xt, out)


def _gemm_grouped(name, A: QTensor, B: QTensor, offsets, rows, cols, out=None):
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.float32, device=A.codes.device)
    a, b = A.c(), B.c()
    _check_matrix("out", out, rows, cols, A.codes.device)
    off = _i64arr(offsets)
    st = getattr(_lib(), name)(ctypes.byref(a), ctypes.byref(b), len(offsets) - 1, off,
                               _ptr(out), out.stride(0), _stream(out))
    _check(name, st)
    return out


def ufp4_gemm_fprop_grouped(Xp: QTensor, W: QTensor, offsets, out=None):
    G = len(offsets) - 1
    return _gemm_grouped("ufp4_gemm_fprop_grouped", Xp, W, offsets, Xp.P, W.P // G, out)


def ufp4_gemm_dgrad_grouped(dYp: QTensor, Wt: QTensor, offsets, out=None):
    G = len(offsets) - 1
    return _gemm_grouped("ufp4_gemm_dgrad_grouped", dYp, Wt, offsets, dYp.P, Wt.P // G, out)


def ufp4_gemm_wgrad_grouped(dYt: QTensor, Xt: QTensor, offsets, out=None):
    G = len(offsets) - 1
    return _gemm_grouped("ufp4_gemm_wgrad_grouped", dYt, Xt, offsets, G * dYt.P, Xt.P, out)


def ufp4_gemm_workspace_bytes(op, A: QTensor, B: QTensor, groups=0):
    a, b = A.c(), B.c()
    return int(_lib().ufp4_gemm_workspace_bytes(op, ctypes.byref(a), ctypes.byref(b), groups))


def ufp4_gemm_ws(op, A: QTensor, B: QTensor, offsets=None, out=None, workspace=None):
    """One of the GEMMs above (op = UFP4_GEMM_FPROP / DGRAD / WGRAD; dense when
    offsets is None, else grouped) through the workspace entry point.  With
    workspace=None a uint8 device buffer of the size the library asks for is
    allocated here (none when it asks for 0 bytes)."""
    G = 0 if offsets is None else len(offsets) - 1
    if G == 0:
        rows, cols = A.P, B.P
    elif op == UFP4_GEMM_WGRAD:
        rows, cols = G * A.P, B.P
    else:
        rows, cols = A.P, B.P // G
    dev = A.codes.device
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.float32, device=dev)
    a, b = A.c(), B.c()
    _check_matrix("out", out, rows, cols, dev)
    need = int(_lib().ufp4_gemm_workspace_bytes(op, ctypes.byref(a), ctypes.byref(b), G))
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None:
        _check_buffer("workspace", workspace, torch.uint8, need, dev)
    off = _i64arr(offsets) if G else None
    st = _lib().ufp4_gemm_ws(op, ctypes.byref(a), ctypes.byref(b), G, off, _ptr(out),
                             out.stride(0), _ptr(workspace) if workspace is not None else None,
                             workspace.numel() if workspace is not None else 0, _stream(out))
    _check("ufp4_gemm_ws", st)
    return out


def ufp4_transpose_qtensor(q: QTensor):
    dev = q.codes.device
    codes = torch.empty((q.K, q.P // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((q.K // q.cfg.block_cols, q.P // q.cfg.block_rows),
                         dtype=q.scales.dtype, device=dev)
    qc = q.c()
    st = _lib().ufp4_transpose_qtensor(ctypes.byref(qc), _ptr(codes), _ptr(scales),
                                       _stream(codes))
    _check("ufp4_transpose_qtensor", st)
    return QTensor(codes, scales, q.K, q.P, q.cfg)


def ufp4_philox_fill(seed, stream_id, first, n, device="cuda"):
    out = torch.empty(n, dtype=torch.int16, device=device)
    st = _lib().ufp4_philox_fill(int(seed), int(stream_id), int(first), int(n), _ptr(out),
                                 _stream(out))
    _check("ufp4_philox_fill", st)
    return out


def ufp4_stream_copy(src, dst):
    """Copy the bytes of the contiguous device tensor src into dst (same
    number of bytes) with the library's streaming copy kernel."""
    if not (src.is_cuda and dst.is_cuda):
        raise ValueError("ufp4_stream_copy: src and dst must be device tensors")
    if not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("ufp4_stream_copy: src and dst must be contiguous")
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n:
        raise ValueError("ufp4_stream_copy: src and dst differ in size")
    if src.device != dst.device:
        raise ValueError("ufp4_stream_copy: src and dst are on different devices")
    st = _lib().ufp4_stream_copy(_ptr(src), _ptr(dst), n, _stream(dst))
    _check("ufp4_stream_copy", st)
    return dst


def ufp4_codes_bytes(P, K):
    return int(_lib().ufp4_codes_bytes(int(P), int(K)))


def ufp4_scales_bytes(P, K, cfg):
    return int(_lib().ufp4_scales_bytes(int(P), int(K), ctypes.byref(cfg)))


def ufp4_status_string(status):
    return _lib().ufp4_status_string(int(status)).decode()
