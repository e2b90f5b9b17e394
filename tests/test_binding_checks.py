"""The Python binding's buffer checks, on the CPU.  The C ABI takes raw
device pointers and cannot see buffer sizes, so the binding rejects a wrong
dtype, a non-contiguous or too small buffer, a strided or too small output
matrix and a host tensor with ValueError before any library call."""
import pytest
import torch

import rht_bit_block_amd as U


def _x(rows=64, cols=128, dtype=torch.bfloat16):
    return torch.zeros((rows, cols), dtype=dtype)


def test_quant_rejects_bad_input():
    cfg = U.make_cfg()
    with pytest.raises(ValueError, match="bfloat16"):
        U.ufp4_rht_quant(_x(dtype=torch.float32), 0, cfg)
    with pytest.raises(ValueError, match="row-major"):
        U.ufp4_rht_quant(_x(128, 64).t(), 0, cfg)
    with pytest.raises(ValueError, match="GPU"):
        U.ufp4_rht_quant(_x(), 0, cfg)
    for fn in (lambda x: U.ufp4_rht_quant_dual(x, cfg, cfg),
               lambda x: U.ufp4_rht_quant_segmented(x, [0, 64], cfg),
               lambda x: U.ufp4_quant_diag(x, cfg)):
        with pytest.raises(ValueError, match="bfloat16"):
            fn(_x(dtype=torch.float16))
        with pytest.raises(ValueError, match="row-major"):
            fn(_x(128, 64).t())


def test_quant_rejects_bad_outputs():
    cfg = U.make_cfg()                       # 1 x 16 fp32 scales: [64, 64] codes, [64, 8] scales
    x = _x()
    ok_c = torch.empty((64, 64), dtype=torch.uint8)
    ok_s = torch.empty((64, 8), dtype=torch.float32)
    with pytest.raises(ValueError, match="codes must have dtype"):
        U.ufp4_rht_quant(x, 0, cfg, codes=torch.empty((64, 64), dtype=torch.int8), scales=ok_s)
    with pytest.raises(ValueError, match="codes holds"):
        U.ufp4_rht_quant(x, 0, cfg, codes=torch.empty((64, 63), dtype=torch.uint8), scales=ok_s)
    with pytest.raises(ValueError, match="codes must be contiguous"):
        U.ufp4_rht_quant(x, 0, cfg, codes=torch.empty((64, 128), dtype=torch.uint8)[:, ::2],
                         scales=ok_s)
    with pytest.raises(ValueError, match="scales must have dtype"):
        U.ufp4_rht_quant(x, 0, cfg, codes=ok_c, scales=torch.empty((64, 8), dtype=torch.uint8))
    with pytest.raises(ValueError, match="scales holds"):
        U.ufp4_rht_quant(x, 0, cfg, codes=ok_c, scales=torch.empty((64, 7), dtype=torch.float32))
    # column-wise: P = 128 rows of codes of K/2 = 32 bytes
    with pytest.raises(ValueError, match="codes holds"):
        U.ufp4_rht_quant(x, 1, cfg, codes=torch.empty((64, 64), dtype=torch.uint8)[:63],
                         scales=torch.empty((128, 4), dtype=torch.float32))
    pow2 = U.make_cfg(U.UFP4_E2M1, U.UFP4_RTNE, U.UFP4_SCALE_POW2, 32, 32, 1)
    with pytest.raises(ValueError, match="scales must have dtype"):
        U.ufp4_rht_quant(x, 0, pow2, codes=ok_c, scales=torch.empty(8, dtype=torch.float32))
    with pytest.raises(ValueError, match="scales holds"):
        U.ufp4_rht_quant(x, 0, pow2, codes=ok_c, scales=torch.empty(7, dtype=torch.uint8))
    with pytest.raises(ValueError, match="codes_col holds"):
        U.ufp4_rht_quant_dual(x, cfg, cfg, out_col=(torch.empty(10, dtype=torch.uint8), ok_s))
    with pytest.raises(ValueError, match="stats"):
        U.ufp4_quant_diag(x, cfg, stats=torch.empty(16, dtype=torch.int32))


def test_qtensor_and_output_checks():
    cfg = U.make_cfg()
    q = U.QTensor(torch.empty((64, 32), dtype=torch.uint8), torch.empty((64, 4), dtype=torch.float32),
                  64, 64, cfg)
    with pytest.raises(ValueError, match="GPU"):        # right sizes, host memory
        q.c()
    short = U.QTensor(torch.empty((64, 31), dtype=torch.uint8), q.scales, 64, 64, cfg)
    with pytest.raises(ValueError, match="codes holds"):
        short.c()
    wrong = U.QTensor(q.codes, torch.empty((64, 4), dtype=torch.float64), 64, 64, cfg)
    with pytest.raises(ValueError, match="scales must have dtype"):
        wrong.c()
    mx8 = U.make_cfg(U.UFP4_E4M3, U.UFP4_RTNE, U.UFP4_SCALE_POW2, 1, 32, 1)
    with pytest.raises(ValueError, match="codes holds"):      # E4M3: one byte per element
        U.QTensor(q.codes, torch.empty((64, 2), dtype=torch.uint8), 64, 64, mx8).c()
    dev = torch.device("cpu")
    f32 = torch.empty((64, 96), dtype=torch.float32)
    with pytest.raises(ValueError, match="float32"):
        U._check_matrix("out", f32.double(), 64, 96, dev)
    with pytest.raises(ValueError, match="unit column stride"):
        U._check_matrix("out", torch.empty((96, 64), dtype=torch.float32).t(), 64, 96, dev)
    with pytest.raises(ValueError, match="needs at least"):
        U._check_matrix("out", f32[:, :95], 64, 96, dev)
    with pytest.raises(ValueError, match="needs at least"):
        U._check_matrix("out", f32[:63], 64, 96, dev)
    with pytest.raises(ValueError, match="must be on"):
        U._check_matrix("out", f32, 64, 96, torch.device("cuda", 0))
    U._check_matrix("out", f32, 64, 96, dev)               # a host matrix of the host "device"
    U._check_matrix("out", torch.empty((0, 5), dtype=torch.float32), 0, 96, dev)   # empty
