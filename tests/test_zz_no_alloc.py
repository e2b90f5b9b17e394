"""The allocation-free variant of the level-statistics call, through the C
ABI: its statistics equal those of ufp4_quant_diag (caller workspace) bit
for bit on two calls in a row, the second on a smaller input (the library's
scratch array keeps the first call's partial sums, which the second call
must clear), and equal the oracle's on the smaller one."""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
import rht_bit_block_amd as U
from gpu_helpers import dev_bf16, rand_bits, spec_of

pytestmark = pytest.mark.gpu


def _noalloc(lib, x, cfg, stats):
    rows, cols = x.shape
    st = lib.ufp4_quant_diag_noalloc(ctypes.c_void_p(x.data_ptr()), rows, cols, x.stride(0),
                                     ctypes.byref(cfg), ctypes.c_void_p(stats.data_ptr()),
                                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == U.UFP4_OK, U.ufp4_status_string(st)


@pytest.mark.parametrize("grid,n,b", [(U.UFP4_E1M2, 16, 16), (U.UFP4_INT4, 128, 16),
                                      (U.UFP4_E2M1, 32, 32)])
def test_diag_noalloc_matches_workspace_call(grid, n, b):
    print("case: diag noalloc", grid, n, b, flush=True)
    lib = U.lib_handle()
    cfg = U.make_cfg(grid, U.UFP4_SR, U.UFP4_SCALE_F32, 1, b, n, sign_seed=71, sr_seed=72,
                     sr_stream=3)
    big = dev_bf16(rand_bits(1024, 2048, seed=grid + n))     # 2M elements: many workgroups
    small_bits = rand_bits(40, 256, seed=grid + n + 1)
    small = dev_bf16(small_bits)
    for x in (big, small):
        got = torch.full((16,), -1, dtype=torch.int64, device="cuda")
        _noalloc(lib, x, cfg, got)
        want = U.ufp4_quant_diag(x, cfg)
        torch.cuda.synchronize()
        assert torch.equal(got, want), (got.cpu().numpy(), want.cpu().numpy())
    ref = O.level_stats(O.quantize(small_bits, 0, spec_of(cfg)), grid)
    assert np.array_equal(got.cpu().numpy(), ref)


def test_diag_noalloc_errors_before_launch():
    """Arguments are validated before anything is enqueued (same rules as the
    workspace call): null stats, bad shapes, 2D blocks."""
    lib = U.lib_handle()
    x = dev_bf16(rand_bits(16, 64, seed=3))
    cfg = U.make_cfg()
    stats = torch.empty(16, dtype=torch.int64, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.ufp4_quant_diag_noalloc(ctypes.c_void_p(x.data_ptr()), 16, 64, 64, ctypes.byref(cfg),
                                       None, s) == U.UFP4_ERR_INVALID_ARG
    assert lib.ufp4_quant_diag_noalloc(ctypes.c_void_p(x.data_ptr()), 16, 40, 64, ctypes.byref(cfg),
                                       ctypes.c_void_p(stats.data_ptr()), s) == U.UFP4_ERR_SHAPE
    two_d = U.make_cfg(U.UFP4_E2M1, U.UFP4_RTNE, U.UFP4_SCALE_POW2, 32, 32, 1)
    assert lib.ufp4_quant_diag_noalloc(ctypes.c_void_p(x.data_ptr()), 16, 64, 64, ctypes.byref(two_d),
                                       ctypes.c_void_p(stats.data_ptr()), s) == U.UFP4_ERR_UNSUPPORTED
