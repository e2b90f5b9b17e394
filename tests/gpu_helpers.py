"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and the oracle on the same seeded bf16 bits, and compare."""
import numpy as np
import torch

import oracle as O
import rht_bit_block_amd as U

GRIDS = [U.UFP4_E1M2, U.UFP4_INT4, U.UFP4_E2M1]
GEMM_TOL = 1e-4   # relative Frobenius error vs the oracle's fp64 product


def spec_of(cfg):
    return O.QuantSpec(cfg.grid, cfg.rounding, cfg.scale_mode, cfg.block_rows, cfg.block_cols,
                       cfg.rht_n, cfg.sign_seed, cfg.sr_seed, cfg.sr_stream,
                       tensor_scale=float(cfg.tensor_scale))


def dev_bf16(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def host_bits(x):
    return x.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def rand_bits(rows, cols, seed, outlier_frac=0.01, outlier_scale=30.0):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((rows, cols)).astype(np.float32)
    m = rng.random((rows, cols)) < outlier_frac
    a[m] *= outlier_scale
    return torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f32_bits_equal(a, b):
    a = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    b = np.ascontiguousarray(b, dtype=np.float32).view(np.uint32)
    return np.array_equal(a, b)


def first_diff(a, b):
    a = np.asarray(a)
    b = np.asarray(b)
    idx = np.argwhere(a != b)
    return None if idx.size == 0 else (tuple(idx[0]), a[tuple(idx[0])], b[tuple(idx[0])], len(idx))


def compare_quant(bits, along, cfg, with_rotated=True):
    """Quantize on the GPU and in the oracle; assert bit equality."""
    x = dev_bf16(bits)
    q, rot = U.ufp4_rht_quant(x, along, cfg, rotated=with_rotated)
    torch.cuda.synchronize()
    ref = O.quantize(bits, along, spec_of(cfg))
    codes = q.codes.cpu().numpy()
    scales = q.scales.cpu().numpy()
    if with_rotated:
        r = rot.cpu().numpy()
        assert f32_bits_equal(r, ref["rotated"]), ("rotated", first_diff(r.view(np.uint32), ref["rotated"].view(np.uint32)))
    if cfg.scale_mode == U.UFP4_SCALE_F32:
        assert f32_bits_equal(scales, ref["scales"]), ("scales", first_diff(scales.view(np.uint32), ref["scales"].view(np.uint32)))
    else:
        assert np.array_equal(scales, ref["scales"]), ("scales", first_diff(scales, ref["scales"]))
    assert np.array_equal(codes, ref["codes"]), ("codes", first_diff(codes, ref["codes"]))
    return q, ref


def oracle_dequant64(ref, cfg):
    return O.dequant(ref["codes"], ref["scales"], spec_of(cfg), ref["P"], ref["K"])[1]
