"""Parity of the HIP path (through the C ABI) with the CPU oracle at sizes the
oracle finishes in seconds: several tiles / waves plus ragged tails, every
grid, rounding, Hadamard size and block shape, edge values, dequant, the
GEMMs (dense and grouped), the 2D transpose and the draw generator.

Bar: bit-exact rotated values, scales, codes, draws and dequant; GEMMs within
1e-4 relative Frobenius error of the oracle's fp64 product of its own
dequantized operands."""
import numpy as np
import pytest
import torch

import oracle as O
import rht_bit_block_amd as U
from gpu_helpers import (GEMM_TOL, GRIDS, compare_quant, dev_bf16, f32_bits_equal, first_diff,
                         oracle_dequant64, rand_bits, spec_of)

pytestmark = pytest.mark.gpu

NB = [(1, 16), (2, 16), (16, 16), (32, 16), (64, 16), (128, 16), (1, 32), (16, 32), (32, 32),
      (128, 32)]


def _print_case(*a):
    print("case:", *a, flush=True)


def test_philox_fill_matches_oracle():
    for seed, stream, first, n in [(2201, 0, 0, 4096), (2201, 1, 12345, 1000), (2 ** 63 + 5, 7, 2 ** 40 + 3, 777)]:
        _print_case("philox", seed, stream, first, n)
        got = U.ufp4_philox_fill(seed, stream, first, n).cpu().numpy().view(np.uint16)
        want = O.sr_draws(seed, stream, np.arange(first, first + n, dtype=np.uint64))
        assert np.array_equal(got, want)


@pytest.mark.parametrize("nbytes", [1, 15, 16, 17, 4096, 65536 * 16 + 5, (64 << 20) + 48 + 9])
def test_stream_copy(nbytes):
    """The streaming copy reproduces every byte (whole 16-byte vectors, one
    per thread, and the bytes past the last vector) and writes nothing past
    the end."""
    _print_case("stream copy", nbytes)
    g = torch.Generator(device="cuda")
    g.manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)
    guard = torch.full((nbytes + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    dst = guard[:nbytes]
    U.ufp4_stream_copy(src, dst)
    assert torch.equal(dst, src)
    assert torch.all(guard[nbytes:] == 0xA5)


@pytest.mark.parametrize("n,b", NB)
@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("rnd", [U.UFP4_RTNE, U.UFP4_SR])
def test_quant_rows(n, b, grid, rnd):
    _print_case("rows", n, b, grid, rnd)
    bits = rand_bits(40, 384, seed=n * 7 + b + grid)      # 40 rows: ragged against 64-lane waves
    cfg = U.make_cfg(grid, rnd, U.UFP4_SCALE_F32, 1, b, n, sign_seed=1000 + n, sr_seed=77, sr_stream=3)
    compare_quant(bits, 0, cfg)


@pytest.mark.parametrize("n,b", NB)
@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("rnd", [U.UFP4_RTNE, U.UFP4_SR])
def test_quant_cols(n, b, grid, rnd):
    _print_case("cols", n, b, grid, rnd)
    bits = rand_bits(384, 72, seed=n * 11 + b + grid)     # K = 384 (3 LDS tiles), P = 72 (ragged)
    cfg = U.make_cfg(grid, rnd, U.UFP4_SCALE_F32, 1, b, n, sign_seed=2000 + n, sr_seed=78, sr_stream=4)
    compare_quant(bits, 1, cfg)


@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("rnd", [U.UFP4_RTNE, U.UFP4_SR])
@pytest.mark.parametrize("n,b", [(1, 32), (16, 32), (32, 32), (1, 16), (8, 16), (16, 16)])
def test_quant_2d(grid, rnd, n, b):
    """Square blocks: K / b = 5 or 10 block columns (a wave takes 64 / b of
    them, so the last wave is partial for b = 32 and for b = 16 with K = 160:
    10 = 2 x 4 + 2)."""
    _print_case("2d", grid, rnd, n, b)
    bits = rand_bits(96, 160, seed=grid + 10 * rnd + n + b)
    cfg = U.make_cfg(grid, rnd, U.UFP4_SCALE_POW2, b, b, n, sign_seed=5, sr_seed=5201)
    compare_quant(bits, 0, cfg)


def _edge_bits():
    """Zeros, a zero block, subnormal and tiny values, huge values, exact grid
    ties after scaling, and +-qmax multiples."""
    rng = np.random.default_rng(99)
    a = rng.standard_normal((64, 256)).astype(np.float32)
    a[0] = 0.0                                            # all-zero row
    a[1, :32] = 0.0                                       # zero blocks inside a row
    a[2] = rng.standard_normal(256).astype(np.float32) * np.float32(1e-39)   # subnormals
    a[3] = rng.standard_normal(256).astype(np.float32) * np.float32(1e-30)
    a[4] = rng.standard_normal(256).astype(np.float32) * np.float32(1e30)
    a[5] = np.tile(np.arange(16, dtype=np.float32) / 2.0, 16)               # many exact ties
    a[6] = np.tile(np.array([7, -7, 3.5, -3.5, 0.5, 1.5, 2.5, 6, 5, -5, 1, 0, 0, 0, 0.25, 7],
                            dtype=np.float32), 16)
    a[7, ::2] = 0.0                                       # half zeros
    a[8] = np.float32(1.0)                                # constant rows
    a[9] = -np.float32(3.0)
    a[10:12] *= np.float32(2.0 ** -100)
    return torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("rnd", [U.UFP4_RTNE, U.UFP4_SR])
@pytest.mark.parametrize("n", [1, 16, 128])
def test_quant_edge_values(grid, rnd, n):
    _print_case("edge", grid, rnd, n)
    bits = _edge_bits()
    cfg = U.make_cfg(grid, rnd, U.UFP4_SCALE_F32, 1, 16, n, sign_seed=3, sr_seed=4, sr_stream=0)
    compare_quant(bits, 0, cfg)
    compare_quant(bits, 1, cfg.copy(rht_n=min(n, 64)))     # K = 64 rows along the columns
    cfg2 = U.make_cfg(grid, rnd, U.UFP4_SCALE_POW2, 32, 32, min(n, 32), sign_seed=3, sr_seed=4)
    compare_quant(bits, 0, cfg2)


@pytest.mark.parametrize("n,b", [(64, 16), (128, 16), (64, 32), (128, 32)])
@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("rnd", [U.UFP4_RTNE, U.UFP4_SR])
def test_quant_fused_stages(n, b, grid, rnd):
    """Without the rotated output the cross-lane butterflies run fused (one
    DPP fma per element, values negated in half the lanes, the quotients
    taken with the negated divisor): codes and scales stay bit-exact, for
    fp32 and power-of-two scales, two-level scaling, rows and columns, and
    the edge values (exact zeros, where only the sign of zero could differ)."""
    _print_case("fused", n, b, grid, rnd)
    rows = rand_bits(40, 384, seed=n + b + grid)
    cols = rand_bits(384, 72, seed=n + b + grid + 1)
    cfg = U.make_cfg(grid, rnd, U.UFP4_SCALE_F32, 1, b, n, sign_seed=3000 + n, sr_seed=79, sr_stream=5)
    compare_quant(rows, 0, cfg, with_rotated=False)
    compare_quant(cols, 1, cfg, with_rotated=False)
    compare_quant(_edge_bits(), 0, cfg, with_rotated=False)
    if b == 32:
        pow2 = U.make_cfg(grid, rnd, U.UFP4_SCALE_POW2, 1, 32, n, sign_seed=3100 + n, sr_seed=80)
        compare_quant(rows, 0, pow2, with_rotated=False)
        compare_quant(cols, 1, pow2, with_rotated=False)
        compare_quant(rows, 0, pow2.copy(tensor_scale=0.37), with_rotated=False)


def test_quant_empty():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    q, _ = U.ufp4_rht_quant(x, 0, U.make_cfg())
    assert q.codes.numel() == 0


@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("two_d", [0, 16, 32])
def test_dequant_bit_exact(grid, two_d):
    _print_case("dequant", grid, two_d)
    bits = rand_bits(64, 192, seed=grid)
    cfg = (U.make_cfg(grid, U.UFP4_SR, U.UFP4_SCALE_POW2, two_d, two_d, 1, sr_seed=9) if two_d
           else U.make_cfg(grid, U.UFP4_SR, U.UFP4_SCALE_F32, 1, 16, 16, sign_seed=8, sr_seed=9))
    q, ref = compare_quant(bits, 0, cfg, with_rotated=False)
    d = U.ufp4_dequant(q).cpu().numpy()
    want = O.dequant(ref["codes"], ref["scales"], spec_of(cfg), 64, 192)[0]
    assert f32_bits_equal(d, want)


def _gemm_case(PA, PB, K, cfg_a, cfg_b, seed):
    ta = rand_bits(PA, K, seed)
    tb = rand_bits(PB, K, seed + 1)
    qa, ra = compare_quant(ta, 0, cfg_a, with_rotated=False)
    qb, rb = compare_quant(tb, 0, cfg_b, with_rotated=False)
    C = U.ufp4_gemm_fprop(qa, qb).cpu().numpy()
    ref = O.gemm_ref(oracle_dequant64(ra, cfg_a), oracle_dequant64(rb, cfg_b))
    err = O.rel_fro(C, ref)
    assert err <= GEMM_TOL, err
    return err


@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("shape", [(256, 256, 256), (300, 270, 96), (17, 513, 48), (520, 64, 1024)])
def test_gemm_small(grid, shape):
    _print_case("gemm", grid, shape)
    PA, PB, K = shape
    n = 16 if K % 16 == 0 else 1
    cfg = U.make_cfg(grid, U.UFP4_RTNE, U.UFP4_SCALE_F32, 1, 16, n, sign_seed=21)
    _gemm_case(PA, PB, K, cfg, cfg, seed=PA + PB + K + grid)


def test_gemm_mixed_blocks_and_sr():
    cfg_a = U.make_cfg(U.UFP4_E1M2, U.UFP4_SR, U.UFP4_SCALE_F32, 1, 32, 32, sign_seed=4, sr_seed=1)
    cfg_b = U.make_cfg(U.UFP4_E1M2, U.UFP4_RTNE, U.UFP4_SCALE_F32, 1, 16, 32, sign_seed=4)
    _gemm_case(384, 320, 640, cfg_a, cfg_b, seed=5)


@pytest.mark.parametrize("grid", [U.UFP4_E2M1, U.UFP4_E1M2])
@pytest.mark.parametrize("b", [16, 32])
def test_gemm_2d_and_transpose(grid, b):
    """2D square blocks: quantize once, reuse transposed (S(B) = S(B^T));
    16 x 16 blocks run on the general kernel (the scaled matrix cores take
    32-element blocks)."""
    _print_case("2d gemm", grid, b)
    cfg = U.make_cfg(grid, U.UFP4_SR, U.UFP4_SCALE_POW2, b, b, 1, sr_seed=5201)
    tx, tw = rand_bits(320, 256, 1), rand_bits(288, 256, 2)
    qx, rx = compare_quant(tx, 0, cfg, with_rotated=False)
    qw, rw = compare_quant(tw, 0, cfg, with_rotated=False)
    # transpose utility == transposed oracle codes / scale grid
    qwt = U.ufp4_transpose_qtensor(qw)
    codes_t = O.unpack_nibbles(rw["codes"]).T
    assert np.array_equal(qwt.codes.cpu().numpy(), O.pack_nibbles(codes_t))
    assert np.array_equal(qwt.scales.cpu().numpy(), rw["scales"].T)
    # S(B) = S(B^T): quantizing W^T directly gives the transposed scale grid
    qwt2, _ = U.ufp4_rht_quant(dev_bf16(np.ascontiguousarray(tw.T)), 0, cfg)
    assert np.array_equal(qwt2.scales.cpu().numpy(), qw.scales.cpu().numpy().T)
    # FPROP with both, and a GEMM on the transposed operand (DGRAD-style)
    C = U.ufp4_gemm_fprop(qx, qw).cpu().numpy()
    dx, dw = oracle_dequant64(rx, cfg), oracle_dequant64(rw, cfg)
    assert O.rel_fro(C, O.gemm_ref(dx, dw)) <= GEMM_TOL
    tdy = rand_bits(320, 288, 3)
    qdy, rdy = compare_quant(tdy, 0, cfg, with_rotated=False)
    dX = U.ufp4_gemm_dgrad(qdy, qwt).cpu().numpy()
    assert O.rel_fro(dX, O.gemm_ref(oracle_dequant64(rdy, cfg), dw.T)) <= GEMM_TOL


DIAG_CASES = [(1, 16, U.UFP4_SCALE_F32), (16, 16, U.UFP4_SCALE_F32), (32, 32, U.UFP4_SCALE_F32),
              (128, 16, U.UFP4_SCALE_F32), (32, 32, U.UFP4_SCALE_POW2), (1, 32, U.UFP4_SCALE_POW2)]


@pytest.mark.parametrize("n,b,smode", DIAG_CASES)
@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("rnd", [U.UFP4_RTNE, U.UFP4_SR])
def test_quant_diag(n, b, smode, grid, rnd):
    """Level statistics (counts and exact error sums per level) equal the
    oracle's on several grid-stride waves plus a ragged row count."""
    _print_case("diag", n, b, smode, grid, rnd)
    bits = rand_bits(72, 512, seed=n + b + 5 * grid + rnd)
    cfg = U.make_cfg(grid, rnd, smode, 1, b, n, sign_seed=300 + n, sr_seed=91, sr_stream=2)
    got = U.ufp4_quant_diag(dev_bf16(bits), cfg).cpu().numpy()
    want = O.level_stats(O.quantize(bits, 0, spec_of(cfg)), grid)
    assert np.array_equal(got, want), (got, want)


def test_quant_diag_empty_and_reuse():
    """An empty operand yields zeros (the buffer is overwritten, not
    accumulated), and a second call on the same buffer starts from zero."""
    cfg = U.make_cfg(U.UFP4_E1M2, U.UFP4_RTNE, U.UFP4_SCALE_F32, 1, 16, 16, sign_seed=1)
    stats = torch.full((16,), 7, dtype=torch.int64, device="cuda")
    U.ufp4_quant_diag(torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"), cfg, stats=stats)
    assert torch.count_nonzero(stats).item() == 0
    bits = rand_bits(16, 256, seed=5)
    for _ in range(2):
        U.ufp4_quant_diag(dev_bf16(bits), cfg, stats=stats)
        want = O.level_stats(O.quantize(bits, 0, spec_of(cfg)), U.UFP4_E1M2)
        assert np.array_equal(stats.cpu().numpy(), want)


@pytest.mark.parametrize("P,K,b", [(32, 32, 32), (288, 544, 32), (1056, 800, 32), (4096, 4096, 32),
                                   (288, 544, 16), (16, 48, 16)])
def test_transpose_shapes(P, K, b):
    """The square-block transpose on tile-ragged shapes and a full-size
    operand: codes and scale grid exactly the transposed ones.  The operand is
    built from seeded random codes and E8M0 scales (a transpose only moves
    them)."""
    _print_case("transpose", P, K, b)
    rng = np.random.default_rng(P * 7 + K)
    codes = rng.integers(0, 16, (P, K), dtype=np.uint8)
    scales = rng.integers(100, 150, (P // b, K // b), dtype=np.uint8)
    cfg = U.make_cfg(U.UFP4_E2M1, U.UFP4_RTNE, U.UFP4_SCALE_POW2, b, b, 1)
    q = U.QTensor(torch.from_numpy(O.pack_nibbles(codes)).cuda(), torch.from_numpy(scales).cuda(),
                  P, K, cfg)
    qt = U.ufp4_transpose_qtensor(q)
    assert (qt.P, qt.K) == (K, P)
    assert np.array_equal(qt.codes.cpu().numpy(), O.pack_nibbles(np.ascontiguousarray(codes.T)))
    assert np.array_equal(qt.scales.cpu().numpy(), scales.T)


@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("K", [160, 384, 512])
def test_gemm_pow2_paths(grid, K):
    """Power-of-two 32 x 32 blocks through every GEMM path: K % 256 == 0
    (wide-step FP4 / FP8 scaled matrix cores), K % 128 == 0, and K = 160
    (split-bf16 fallback); 3 ragged row tiles of A, 2 of B."""
    _print_case("pow2 gemm", grid, K)
    cfg = U.make_cfg(grid, U.UFP4_SR, U.UFP4_SCALE_POW2, 32, 32, 1, sr_seed=77)
    ta, tb = rand_bits(544, K, 11), rand_bits(288, K, 12)
    qa, ra = compare_quant(ta, 0, cfg, with_rotated=False)
    qb, rb = compare_quant(tb, 0, cfg, with_rotated=False)
    C = U.ufp4_gemm_fprop(qa, qb).cpu().numpy()
    ref = O.gemm_ref(oracle_dequant64(ra, cfg), oracle_dequant64(rb, cfg))
    assert O.rel_fro(C, ref) <= GEMM_TOL


def _assert_q_equal(q, ref, tag):
    codes = q.codes.cpu().numpy().reshape(-1)
    scales = q.scales.cpu().numpy().reshape(-1)
    rc, rs = np.asarray(ref["codes"]).reshape(-1), np.asarray(ref["scales"]).reshape(-1)
    assert f32_bits_equal(scales, rs), (tag, "scales", first_diff(scales.view(np.uint32), rs.view(np.uint32)))
    assert np.array_equal(codes, rc), (tag, "codes", first_diff(codes, rc))


@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("rnd", [U.UFP4_RTNE, U.UFP4_SR])
@pytest.mark.parametrize("n,b", [(1, 16), (16, 16), (32, 32), (64, 16)])
def test_quant_dual(grid, rnd, n, b):
    """Both axes from one read == the oracle's row-wise and column-wise
    quantizations with their own signs and SR streams (ragged tiles on both
    axes: 272 = 2 x 128 + 16 rows, 80 = 64 + 16 columns; 320 x 192 for n > 16)."""
    _print_case("dual", grid, rnd, n, b)
    rows, cols = (272, 80) if n <= 16 else (320, 192)
    bits = rand_bits(rows, cols, 40 + n)
    cr = U.make_cfg(grid, rnd, U.UFP4_SCALE_F32, 1, b, n, sign_seed=11, sr_seed=3, sr_stream=0)
    cc = U.make_cfg(grid, rnd, U.UFP4_SCALE_F32, 1, b, n, sign_seed=12, sr_seed=3, sr_stream=1)
    qr, qc = U.ufp4_rht_quant_dual(dev_bf16(bits), cr, cc)
    torch.cuda.synchronize()
    _assert_q_equal(qr, O.quantize(bits, 0, spec_of(cr)), "row")
    _assert_q_equal(qc, O.quantize(bits, 1, spec_of(cc)), "col")


@pytest.mark.parametrize("rnd", [U.UFP4_RTNE, U.UFP4_SR])
def test_quant_dual_whole_tiles(rnd):
    """The dual kernel's path for workgroups whose two 128 x 64 tiles are both
    whole (second tile loaded during the first): 384 x 192 = 9 whole tiles,
    the last workgroup with one; segments of 384, 0 and 256 rows x 192 columns
    = 9 + 6 whole tiles, one workgroup taking the last tile of the first
    segment and the first of the third."""
    _print_case("dual whole tiles", rnd)
    cr = U.make_cfg(U.UFP4_E1M2, rnd, U.UFP4_SCALE_F32, 1, 16, 16, sign_seed=21, sr_seed=7, sr_stream=0)
    cc = U.make_cfg(U.UFP4_E1M2, rnd, U.UFP4_SCALE_F32, 1, 16, 16, sign_seed=22, sr_seed=7, sr_stream=1)
    bits = rand_bits(384, 192, 123)
    qr, qc = U.ufp4_rht_quant_dual(dev_bf16(bits), cr, cc)
    torch.cuda.synchronize()
    _assert_q_equal(qr, O.quantize(bits, 0, spec_of(cr)), "row")
    _assert_q_equal(qc, O.quantize(bits, 1, spec_of(cc)), "col")
    offs = [0, 384, 384, 640]
    bits = rand_bits(640, 192, 124)
    qr, qc = U.ufp4_rht_quant_dual(dev_bf16(bits), cr, cc, row_offsets=offs)
    torch.cuda.synchronize()
    _assert_q_equal(qr, O.quantize(bits, 0, spec_of(cr)), "row")
    segs = [O.quantize(bits[lo:hi], 1, spec_of(cc), elem_base=bits.shape[1] * lo)
            for lo, hi in zip(offs[:-1], offs[1:]) if hi > lo]
    ref = {"codes": np.concatenate([np.asarray(r["codes"]).reshape(-1) for r in segs]),
           "scales": np.concatenate([np.asarray(r["scales"]).reshape(-1) for r in segs])}
    _assert_q_equal(qc, ref, "col")


def test_quant_dual_segmented():
    """Dual call with expert segments (one empty) == the oracle's row-wise
    quantization and per-segment column-wise quantization."""
    _print_case("dual segmented")
    offs = [0, 96, 96, 160, 320]
    bits = rand_bits(320, 64, 77)
    cr = U.make_cfg(U.UFP4_E1M2, U.UFP4_SR, U.UFP4_SCALE_F32, 1, 32, 32, sign_seed=5, sr_seed=9, sr_stream=2)
    cc = U.make_cfg(U.UFP4_E1M2, U.UFP4_SR, U.UFP4_SCALE_F32, 1, 32, 32, sign_seed=6, sr_seed=9, sr_stream=3)
    qr, qc = U.ufp4_rht_quant_dual(dev_bf16(bits), cr, cc, row_offsets=offs)
    torch.cuda.synchronize()
    _assert_q_equal(qr, O.quantize(bits, 0, spec_of(cr)), "row")
    segs = [O.quantize(bits[lo:hi], 1, spec_of(cc), elem_base=bits.shape[1] * lo)
            for lo, hi in zip(offs[:-1], offs[1:]) if hi > lo]
    ref = {"codes": np.concatenate([np.asarray(r["codes"]).reshape(-1) for r in segs]),
           "scales": np.concatenate([np.asarray(r["scales"]).reshape(-1) for r in segs])}
    _assert_q_equal(qc, ref, "col")


@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("rnd", [U.UFP4_RTNE, U.UFP4_SR])
@pytest.mark.parametrize("n", [1, 16, 32, 128])
@pytest.mark.parametrize("along", [0, 1])
def test_quant_pow2_1x32(grid, rnd, n, along):
    """1 x 32 blocks with power-of-two (E8M0) scales, row- and column-wise,
    bit-exact with the oracle (rotated values, E8M0 bytes, codes)."""
    _print_case("pow2 1x32", grid, rnd, n, along)
    cfg = U.make_cfg(grid, rnd, U.UFP4_SCALE_POW2, 1, 32, n, sign_seed=21, sr_seed=4, sr_stream=1)
    rows, cols = (288, 416) if n <= 32 else (384, 384)
    compare_quant(rand_bits(rows, cols, 60 + n), along, cfg)


@pytest.mark.parametrize("grid", GRIDS)
def test_quant_dual_pow2(grid):
    _print_case("dual pow2", grid)
    bits = rand_bits(320, 192, 91)
    cr = U.make_cfg(grid, U.UFP4_SR, U.UFP4_SCALE_POW2, 1, 32, 32, sign_seed=1, sr_seed=2, sr_stream=0)
    cc = U.make_cfg(grid, U.UFP4_SR, U.UFP4_SCALE_POW2, 1, 32, 32, sign_seed=3, sr_seed=2, sr_stream=1)
    qr, qc = U.ufp4_rht_quant_dual(dev_bf16(bits), cr, cc)
    torch.cuda.synchronize()
    for q, ref in ((qr, O.quantize(bits, 0, spec_of(cr))), (qc, O.quantize(bits, 1, spec_of(cc)))):
        assert np.array_equal(q.scales.cpu().numpy().reshape(-1), np.asarray(ref["scales"]).reshape(-1))
        assert np.array_equal(q.codes.cpu().numpy().reshape(-1), np.asarray(ref["codes"]).reshape(-1))


@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("K", [160, 384, 512])
def test_gemm_pow2_1x32(grid, K):
    """GEMMs on 1 x 32 power-of-two operands: the scaled matrix cores take
    one E8M0 byte per row and 32-element block (K % 128 == 0), split-bf16
    otherwise."""
    _print_case("gemm pow2 1x32", grid, K)
    cfg = U.make_cfg(grid, U.UFP4_RTNE, U.UFP4_SCALE_POW2, 1, 32, 32, sign_seed=8)
    ta, tb = rand_bits(544, K, 31), rand_bits(288, K, 32)
    qa, ra = compare_quant(ta, 0, cfg, with_rotated=False)
    qb, rb = compare_quant(tb, 0, cfg, with_rotated=False)
    C = U.ufp4_gemm_fprop(qa, qb).cpu().numpy()
    ref = O.gemm_ref(oracle_dequant64(ra, cfg), oracle_dequant64(rb, cfg))
    assert O.rel_fro(C, ref) <= GEMM_TOL


def test_pow2_2d_exponent_clamp():
    """Blocks whose absmax exceeds qmax * 2^127 (bf16 values near the top of
    the range): the E8M0 exponent clamps at 127 and the values clamp at
    qmax, as in the oracle."""
    _print_case("pow2 clamp")
    bits = rand_bits(64, 64, 5)
    big = np.array([0x7F7F, 0xFF7F, 0x7F70, 0x7F60], dtype=np.uint16)   # ~3.39e38, -3.39e38, ...
    bits[0, 0:4] = big
    bits[40, 40:44] = big
    for grid in GRIDS:
        for cfg in (U.make_cfg(grid, U.UFP4_RTNE, U.UFP4_SCALE_POW2, 32, 32, 1),
                    U.make_cfg(grid, U.UFP4_SR, U.UFP4_SCALE_POW2, 1, 32, 1, sr_seed=3)):
            compare_quant(bits, 0, cfg)


@pytest.mark.parametrize("b", [16, 32])
def test_segmented_quant_and_grouped_gemms(b):
    """Four experts (one empty), per-expert transposed operands, and the
    three grouped GEMMs against per-expert oracle products (1 x 16 blocks: the
    16-wide GEMM kernel; 1 x 32: the 32-wide one)."""
    _print_case("grouped gemms", b)
    G, hidden, ffn = 4, 128, 96
    off = [0, 64, 64, 160, 256]               # padded token offsets (multiples of 32)
    T = off[-1]
    n = 32
    sx, sd, sw = 31, 32, 33
    tx = rand_bits(T, hidden, 40)
    tw = rand_bits(G * ffn, hidden, 41)
    tdy = rand_bits(T, ffn, 42)
    cx = U.make_cfg(U.UFP4_E1M2, U.UFP4_RTNE, U.UFP4_SCALE_F32, 1, b, n, sign_seed=sx)
    cd = U.make_cfg(U.UFP4_E1M2, U.UFP4_SR, U.UFP4_SCALE_F32, 1, b, n, sign_seed=sd, sr_seed=7, sr_stream=0)
    cw_row = cx
    # FPROP: X_perm rows, W stacked rows (both K = hidden)
    qx, rx = compare_quant(tx, 0, cx, with_rotated=False)
    qw, rw = compare_quant(tw, 0, cw_row, with_rotated=False)
    Y = U.ufp4_gemm_fprop_grouped(qx, qw, off).cpu().numpy()
    dxq, dwq = oracle_dequant64(rx, cx), oracle_dequant64(rw, cw_row)
    for g in range(G):
        ref = O.gemm_ref(dxq[off[g]:off[g + 1]], dwq[g * ffn:(g + 1) * ffn])
        if ref.size:
            assert O.rel_fro(Y[off[g]:off[g + 1]], ref) <= GEMM_TOL
    # DGRAD: dY_perm rows (K = ffn) x W^T per expert (segmented column-wise of W)
    cdg = cd.copy(sign_seed=sd)
    cwt = U.make_cfg(U.UFP4_E1M2, U.UFP4_RTNE, U.UFP4_SCALE_F32, 1, b, n, sign_seed=sd)
    qdy, rdy = compare_quant(tdy, 0, cdg, with_rotated=False)
    qwt = U.stacked(U.ufp4_rht_quant_segmented(dev_bf16(tw), [g * ffn for g in range(G + 1)], cwt), G)
    refs_wt = O.quantize_segmented(tw, [g * ffn for g in range(G + 1)], spec_of(cwt))
    got_codes = qwt.codes.cpu().numpy()
    want_codes = np.concatenate([r["codes"].ravel() for r in refs_wt])
    assert np.array_equal(got_codes, want_codes)
    dX = U.ufp4_gemm_dgrad_grouped(qdy, qwt, off).cpu().numpy()
    ddy = oracle_dequant64(rdy, cdg)
    for g in range(G):
        dwt = oracle_dequant64(refs_wt[g], cwt)
        ref = O.gemm_ref(ddy[off[g]:off[g + 1]], dwt)
        if ref.size:
            assert O.rel_fro(dX[off[g]:off[g + 1]], ref) <= GEMM_TOL
    # WGRAD: dY^T and X^T segments (K = expert tokens)
    cdt = U.make_cfg(U.UFP4_E1M2, U.UFP4_SR, U.UFP4_SCALE_F32, 1, b, n, sign_seed=sw, sr_seed=7, sr_stream=1)
    cxt = U.make_cfg(U.UFP4_E1M2, U.UFP4_RTNE, U.UFP4_SCALE_F32, 1, b, n, sign_seed=sw)
    qdyt = U.ufp4_rht_quant_segmented(dev_bf16(tdy), off, cdt)
    qxt = U.ufp4_rht_quant_segmented(dev_bf16(tx), off, cxt)
    r_dyt = O.quantize_segmented(tdy, off, spec_of(cdt))
    r_xt = O.quantize_segmented(tx, off, spec_of(cxt))
    assert np.array_equal(qdyt.codes.cpu().numpy(), np.concatenate([r["codes"].ravel() for r in r_dyt]))
    assert np.array_equal(qdyt.scales.cpu().numpy().view(np.uint32),
                          np.concatenate([r["scales"].ravel() for r in r_dyt]).view(np.uint32))
    dW = U.ufp4_gemm_wgrad_grouped(qdyt, qxt, off).cpu().numpy()
    for g in range(G):
        if off[g + 1] == off[g]:
            assert np.all(dW[g * ffn:(g + 1) * ffn] == 0)
            continue
        ref = O.gemm_ref(oracle_dequant64(r_dyt[g], cdt), oracle_dequant64(r_xt[g], cxt))
        assert O.rel_fro(dW[g * ffn:(g + 1) * ffn], ref) <= GEMM_TOL


def test_repeat_determinism():
    """Same inputs twice (different launch timing) give identical bits."""
    bits = rand_bits(128, 1024, 3)
    cfg = U.make_cfg(U.UFP4_E2M1, U.UFP4_SR, U.UFP4_SCALE_F32, 1, 16, 128, sign_seed=1, sr_seed=2)
    x = dev_bf16(bits)
    a, _ = U.ufp4_rht_quant(x, 0, cfg)
    b, _ = U.ufp4_rht_quant(x, 0, cfg)
    assert torch.equal(a.codes, b.codes) and torch.equal(a.scales, b.scales)
    C1 = U.ufp4_gemm_fprop(a, b)
    C2 = U.ufp4_gemm_fprop(a, b)
    assert torch.equal(C1, C2)


# ---------------------------------------------------------------------------
# MXFP8 (E4M3 elements, 1 x 32 E8M0 scales): [2DFP4] mixed-precision section.
# ---------------------------------------------------------------------------
def _mxfp8_cfg(n, sign_seed=0):
    return U.make_cfg(U.UFP4_E4M3, U.UFP4_RTNE, U.UFP4_SCALE_POW2, 1, 32, n, sign_seed=sign_seed)


@pytest.mark.parametrize("n", [1, 16, 32, 128])
@pytest.mark.parametrize("along", [0, 1])
def test_quant_mxfp8(n, along):
    """Bit-exact E4M3 codes, E8M0 scales and rotated values, row- and
    column-wise (40 rows / 72 columns: ragged against the lane and tile
    shapes)."""
    _print_case("mxfp8", n, along)
    bits = rand_bits(40, 384, seed=n + 3) if along == 0 else rand_bits(384, 72, seed=n + 4)
    q, ref = compare_quant(bits, along, _mxfp8_cfg(n, sign_seed=40 + n))
    assert q.codes.shape == (q.P, q.K)
    d = U.ufp4_dequant(q).cpu().numpy()
    assert f32_bits_equal(d, O.dequant(ref["codes"], ref["scales"], spec_of(q.cfg), q.P, q.K)[0])


def test_quant_mxfp8_edge_values():
    """Subnormal E4M3 results (elements 2^-7..2^-12 of their block maximum),
    ties between E4M3 neighbours, blocks at exactly 448 * 2^e, all-zero
    blocks and huge blocks at the exponent clamp."""
    _print_case("mxfp8 edges")
    rng = np.random.default_rng(77)
    x = rng.standard_normal((64, 256)).astype(np.float32)
    x[0:8, :32] *= np.float32(2.0 ** -12)
    x[0:8, 0] = 448.0                                   # e = 0, the rest subnormal E4M3
    x[8:16, 32:64] = np.float32(1.0625) * np.sign(x[8:16, 32:64])   # ties at e = -8
    x[8:16, 32] = 448.0 * 2.0 ** -8
    x[16:24, 64:96] = 0.0
    x[24:32, 96:128] = np.float32(3.0e38) * np.sign(x[24:32, 96:128])
    x[32:40, 128:160] = np.float32(2.0 ** -130)         # fp32/bf16 subnormals
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for along in (0, 1):
        compare_quant(bits if along == 0 else np.ascontiguousarray(bits.T), along, _mxfp8_cfg(1))


@pytest.mark.parametrize("shape", [(256, 256, 128), (300, 270, 384), (520, 64, 1024), (17, 513, 256)])
def test_gemm_mxfp8(shape):
    """MXFP8 x MXFP8 on the scaled matrix cores vs the oracle's fp64 product
    (several tiles, ragged rows; K a multiple of 128)."""
    _print_case("gemm mxfp8", shape)
    PA, PB, K = shape
    cfg = _mxfp8_cfg(16, sign_seed=5)
    _gemm_case(PA, PB, K, cfg, cfg, seed=PA + PB + K)


def test_gemm_mxfp8_unsupported_k():
    """K not a multiple of 128 is rejected before any launch."""
    cfg = _mxfp8_cfg(1)
    qa, _ = U.ufp4_rht_quant(dev_bf16(rand_bits(64, 160, 1)), 0, cfg)
    qb, _ = U.ufp4_rht_quant(dev_bf16(rand_bits(64, 160, 2)), 0, cfg)
    with pytest.raises(U.UFP4Error) as ei:
        U.ufp4_gemm_fprop(qa, qb)
    assert ei.value.status == U.UFP4_ERR_UNSUPPORTED


# ---------------------------------------------------------------------------
# Output leading dimension: C written into a wider buffer (ldc > P_B) by every
# kernel family; the columns past P_B keep their sentinel.
# ---------------------------------------------------------------------------
LDC_CASES = [
    ("fp32-scale 1x16", U.make_cfg(U.UFP4_E1M2, U.UFP4_RTNE, U.UFP4_SCALE_F32, 1, 16, 16, sign_seed=3), 384),
    ("fp32-scale 1x32", U.make_cfg(U.UFP4_INT4, U.UFP4_RTNE, U.UFP4_SCALE_F32, 1, 32, 32, sign_seed=3), 384),
    ("scaled FP4 K%256", U.make_cfg(U.UFP4_E2M1, U.UFP4_RTNE, U.UFP4_SCALE_POW2, 1, 32, 1), 512),
    ("scaled FP4 K%128", U.make_cfg(U.UFP4_E2M1, U.UFP4_RTNE, U.UFP4_SCALE_POW2, 1, 32, 1), 384),
    ("scaled FP8 E1M2", U.make_cfg(U.UFP4_E1M2, U.UFP4_RTNE, U.UFP4_SCALE_POW2, 1, 32, 1), 384),
    ("MXFP8", U.make_cfg(U.UFP4_E4M3, U.UFP4_RTNE, U.UFP4_SCALE_POW2, 1, 32, 1), 384),
    ("general (pow2, K%128 != 0)", U.make_cfg(U.UFP4_E2M1, U.UFP4_RTNE, U.UFP4_SCALE_POW2, 1, 32, 1), 160),
]


@pytest.mark.parametrize("name,cfg,K", LDC_CASES, ids=[c[0] for c in LDC_CASES])
def test_gemm_output_leading_dimension(name, cfg, K):
    _print_case("ldc", name, K)
    PA, PB, pad = 300, 270, 50
    ta, tb = rand_bits(PA, K, 61), rand_bits(PB, K, 62)
    qa, ra = compare_quant(ta, 0, cfg, with_rotated=False)
    qb, rb = compare_quant(tb, 0, cfg, with_rotated=False)
    buf = torch.full((PA, PB + pad), 12345.0, dtype=torch.float32, device="cuda")
    C = U.ufp4_gemm_fprop(qa, qb, out=buf[:, :PB])
    assert C.stride(0) == PB + pad
    host = buf.cpu().numpy()
    assert np.all(host[:, PB:] == 12345.0)
    ref = O.gemm_ref(oracle_dequant64(ra, cfg), oracle_dequant64(rb, cfg))
    assert O.rel_fro(host[:, :PB], ref) <= GEMM_TOL


@pytest.mark.parametrize("name,cfg,K", LDC_CASES, ids=[c[0] for c in LDC_CASES])
def test_gemm_output_huge_leading_dimension(name, cfg, K):
    """ldc so large that a 256-row tile of C spans 2 GiB or more: the epilogue
    takes its plain-store path (64-bit addresses, explicit bounds)."""
    _print_case("huge ldc", name, K)
    PA, PB = 40, 270
    ldc = (1 << 21) + 64
    ta, tb = rand_bits(PA, K, 63), rand_bits(PB, K, 64)
    qa, ra = compare_quant(ta, 0, cfg, with_rotated=False)
    qb, rb = compare_quant(tb, 0, cfg, with_rotated=False)
    buf = torch.full((PA, ldc), 12345.0, dtype=torch.float32, device="cuda")
    C = U.ufp4_gemm_fprop(qa, qb, out=buf[:, :PB])
    assert C.stride(0) == ldc
    assert torch.all(buf[:, PB:PB + 64] == 12345.0).item()
    assert torch.all(buf[:, ldc - 64:] == 12345.0).item()
    ref = O.gemm_ref(oracle_dequant64(ra, cfg), oracle_dequant64(rb, cfg))
    assert O.rel_fro(buf[:, :PB].cpu().numpy(), ref) <= GEMM_TOL
    del buf, C
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# fp32-scale GEMMs compute the exact sum of level products times scale
# products, rounded in fp32 only (the level dot products are exact, the scale
# products come from three-piece bf16 splits): against the oracle's fp64
# product of its fp32 dequantized operands the error is a few fp32 roundings,
# far inside the 1e-4 bar.  Rows span 10^+-4 and blocks within a row 10^+-2,
# so the scale pieces cover a wide exponent range.
# ---------------------------------------------------------------------------
F32_SCALE_TOL = 2e-6


def _wide_range_bits(rows, cols, seed, bc):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((rows, cols))
    a *= 10.0 ** rng.uniform(-4, 4, size=(rows, 1))
    a *= np.repeat(10.0 ** rng.uniform(-2, 2, size=(rows, cols // bc)), bc, axis=1)
    a[rng.random((rows, cols)) < 0.01] *= 30.0
    t = torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("bc", [16, 32])
@pytest.mark.parametrize("rnd", [U.UFP4_RTNE, U.UFP4_SR])
def test_gemm_fp32_scale_accuracy(grid, bc, rnd):
    _print_case("fp32-scale gemm accuracy", grid, bc, rnd)
    PA, PB, K = 290, 300, 512
    cfg = U.make_cfg(grid, rnd, U.UFP4_SCALE_F32, 1, bc, 16, sign_seed=17, sr_seed=23)
    qa, ra = compare_quant(_wide_range_bits(PA, K, 100 + grid, bc), 0, cfg, with_rotated=False)
    qb, rb = compare_quant(_wide_range_bits(PB, K, 200 + grid, bc), 0, cfg, with_rotated=False)
    C = U.ufp4_gemm_fprop(qa, qb).cpu().numpy()
    ref = O.gemm_ref(oracle_dequant64(ra, cfg), oracle_dequant64(rb, cfg))
    err = O.rel_fro(C, ref)
    print(f"  rel. Frobenius error {err:.3e}", flush=True)
    assert err <= F32_SCALE_TOL, err


# ---------------------------------------------------------------------------
# Last-round split of the fp32-scale GEMMs: when a launch's last round of
# workgroups (one per CU) is at most half full and tiles average 1024 or more
# K elements, each tile of that round is computed by two workgroups, one per
# K half, whose partial sums are added into C zeroed beforehand.  Here every
# tile is in the last round (fewer tiles than CUs).  Against the oracle at the
# fp32-scale bar, halves of unequal length (K = 1152), both kernels (1 x 16,
# 1 x 32), grouped launches with an empty expert, and bit-identical results
# on a second call.
# ---------------------------------------------------------------------------
def _assert_split(tiles, kavg):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rem = tiles % cus
    assert 0 < rem <= cus // 2 and kavg >= 1024, "the shape does not take the split path"


@pytest.mark.parametrize("grid,bc,K", [(U.UFP4_INT4, 16, 1152), (U.UFP4_E1M2, 32, 1024),
                                       (U.UFP4_E2M1, 16, 1024),
                                       # second halves ending inside a 128-element stage
                                       (U.UFP4_INT4, 16, 1040), (U.UFP4_E1M2, 32, 1056)])
def test_gemm_split_last_round(grid, bc, K):
    _print_case("split last round", grid, bc, K)
    PA, PB = 700, 300                                     # 3 x 2 ragged tiles
    _assert_split(3 * 2, K)
    cfg = U.make_cfg(grid, U.UFP4_RTNE, U.UFP4_SCALE_F32, 1, bc, 16, sign_seed=41)
    qa, ra = compare_quant(_wide_range_bits(PA, K, 300 + grid, bc), 0, cfg, with_rotated=False)
    qb, rb = compare_quant(_wide_range_bits(PB, K, 400 + grid, bc), 0, cfg, with_rotated=False)
    C1 = U.ufp4_gemm_fprop(qa, qb)
    C2 = U.ufp4_gemm_fprop(qa, qb)
    assert torch.equal(C1, C2)
    ref = O.gemm_ref(oracle_dequant64(ra, cfg), oracle_dequant64(rb, cfg))
    err = O.rel_fro(C1.cpu().numpy(), ref)
    print(f"  rel. Frobenius error {err:.3e}", flush=True)
    assert err <= F32_SCALE_TOL, err


def test_grouped_split_last_round():
    _print_case("grouped split last round")
    cfg = U.make_cfg(U.UFP4_INT4, U.UFP4_RTNE, U.UFP4_SCALE_F32, 1, 16, 16, sign_seed=43)
    # FPROP grouped along rows: experts of 384 and 256 tokens, F = 160 (3 tiles), K = 1024
    off, H, F = [0, 384, 640], 1024, 160
    _assert_split(3, H)
    qx, rx = compare_quant(rand_bits(off[-1], H, 50), 0, cfg, with_rotated=False)
    qw, rw = compare_quant(rand_bits(2 * F, H, 51), 0, cfg, with_rotated=False)
    Y1 = U.ufp4_gemm_fprop_grouped(qx, qw, off)
    Y2 = U.ufp4_gemm_fprop_grouped(qx, qw, off)
    assert torch.equal(Y1, Y2)
    Y = Y1.cpu().numpy()
    dx, dw = oracle_dequant64(rx, cfg), oracle_dequant64(rw, cfg)
    for g in range(2):
        ref = O.gemm_ref(dx[off[g]:off[g + 1]], dw[g * F:(g + 1) * F])
        assert O.rel_fro(Y[off[g]:off[g + 1]], ref) <= F32_SCALE_TOL, g
    # WGRAD grouped along K: experts of 1280, 256, 0 and 2560 tokens (1024 on
    # average), N = 96, H = 160 (one tile per expert)
    off, N, H = [0, 1280, 1536, 1536, 4096], 96, 160
    _assert_split(4, off[-1] // 4)
    cs = U.make_cfg(U.UFP4_INT4, U.UFP4_SR, U.UFP4_SCALE_F32, 1, 16, 16, sign_seed=44, sr_seed=5,
                    sr_stream=1)
    cr = U.make_cfg(U.UFP4_INT4, U.UFP4_RTNE, U.UFP4_SCALE_F32, 1, 16, 16, sign_seed=44)
    tdy, tx = rand_bits(off[-1], N, 52), rand_bits(off[-1], H, 53)
    qdyt = U.ufp4_rht_quant_segmented(dev_bf16(tdy), off, cs)
    qxt = U.ufp4_rht_quant_segmented(dev_bf16(tx), off, cr)
    dW = torch.full((4 * N, H), 7.0, dtype=torch.float32, device="cuda")
    U.ufp4_gemm_wgrad_grouped(qdyt, qxt, off, out=dW)
    dW2 = U.ufp4_gemm_wgrad_grouped(qdyt, qxt, off)
    assert torch.equal(dW, dW2)
    dW = dW.cpu().numpy()
    r_dyt = O.quantize_segmented(tdy, off, spec_of(cs))
    r_xt = O.quantize_segmented(tx, off, spec_of(cr))
    for g in range(4):
        blk = dW[g * N:(g + 1) * N]
        if off[g + 1] == off[g]:
            assert np.all(blk == 0.0), g
            continue
        ref = O.gemm_ref(oracle_dequant64(r_dyt[g], cs), oracle_dequant64(r_xt[g], cr))
        assert O.rel_fro(blk, ref) <= F32_SCALE_TOL, g


def test_split_beside_full_rounds():
    """Full rounds and a split last round in one launch: dense FPROP of 16 x 19
    = 304 tiles (48 split on 256 CUs) and WGRAD grouped along K with 3 experts
    of 6 x 16 = 96 tiles each (288 tiles, 32 split), every element against the
    oracle at the fp32-scale bar."""
    _print_case("split beside full rounds")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    cfg = U.make_cfg(U.UFP4_INT4, U.UFP4_RTNE, U.UFP4_SCALE_F32, 1, 16, 16, sign_seed=46)
    PA, PB, K = 4096, 4864, 1024
    T = (PA // 256) * (PB // 256)
    assert T > cus, "no full round before the split one"
    _assert_split(T, K)
    qa, ra = compare_quant(rand_bits(PA, K, 60), 0, cfg, with_rotated=False)
    qb, rb = compare_quant(rand_bits(PB, K, 61), 0, cfg, with_rotated=False)
    C = U.ufp4_gemm_fprop(qa, qb).cpu().numpy()
    ref = O.gemm_ref(oracle_dequant64(ra, cfg), oracle_dequant64(rb, cfg))
    assert O.rel_fro(C, ref) <= F32_SCALE_TOL
    # per-tile check: every 256 x 256 tile, so a wrong split tile cannot hide
    for i in range(0, PA, 256):
        for j in range(0, PB, 256):
            assert O.rel_fro(C[i:i + 256, j:j + 256], ref[i:i + 256, j:j + 256]) <= F32_SCALE_TOL, (i, j)
    assert np.array_equal(C, U.ufp4_gemm_fprop(qa, qb).cpu().numpy())
    off, N, H = [0, 1024, 2048, 3072], 1536, 4096          # 6 x 16 tiles per expert
    assert 3 * (N // 256) * (H // 256) > cus
    _assert_split(3 * (N // 256) * (H // 256), 1024)
    cs = U.make_cfg(U.UFP4_INT4, U.UFP4_SR, U.UFP4_SCALE_F32, 1, 16, 16, sign_seed=46, sr_seed=8,
                    sr_stream=1)
    tdy, tx = rand_bits(off[-1], N, 62), rand_bits(off[-1], H, 63)
    qdyt = U.ufp4_rht_quant_segmented(dev_bf16(tdy), off, cs)
    qxt = U.ufp4_rht_quant_segmented(dev_bf16(tx), off, cfg)
    dW = U.ufp4_gemm_wgrad_grouped(qdyt, qxt, off)
    assert torch.equal(dW, U.ufp4_gemm_wgrad_grouped(qdyt, qxt, off))
    dW = dW.cpu().numpy()
    r_dyt = O.quantize_segmented(tdy, off, spec_of(cs))
    r_xt = O.quantize_segmented(tx, off, spec_of(cfg))
    for g in range(3):
        ref = O.gemm_ref(oracle_dequant64(r_dyt[g], cs), oracle_dequant64(r_xt[g], cfg))
        blk = dW[g * N:(g + 1) * N]
        for i in range(0, N, 256):
            for j in range(0, H, 256):
                assert O.rel_fro(blk[i:i + 256, j:j + 256], ref[i:i + 256, j:j + 256]) <= F32_SCALE_TOL, (g, i, j)


def test_grouped_wgrad_dealt_tiles():
    """Skewed experts (one holds most tokens, one is empty): contiguous ranges
    of whole experts over the 8 XCDs would be unbalanced, so the tiles are
    dealt in runs over the XCDs, experts longest first (8 tiles per expert,
    16 experts).  Every expert's dW against the oracle, and a repeat."""
    _print_case("grouped wgrad dealt tiles")
    lens = [640, 32, 64, 0, 96, 32, 32, 128, 32, 64, 32, 32, 160, 32, 64, 32]
    off = [0]
    for n in lens:
        off.append(off[-1] + n)
    G, N, H = len(lens), 296, 800                        # 2 x 4 tiles per expert
    cs = U.make_cfg(U.UFP4_E1M2, U.UFP4_SR, U.UFP4_SCALE_F32, 1, 16, 32, sign_seed=45, sr_seed=6,
                    sr_stream=1)
    cr = U.make_cfg(U.UFP4_E1M2, U.UFP4_RTNE, U.UFP4_SCALE_F32, 1, 16, 32, sign_seed=45)
    tdy, tx = rand_bits(off[-1], N, 54), rand_bits(off[-1], H, 55)
    qdyt = U.ufp4_rht_quant_segmented(dev_bf16(tdy), off, cs)
    qxt = U.ufp4_rht_quant_segmented(dev_bf16(tx), off, cr)
    dW = U.ufp4_gemm_wgrad_grouped(qdyt, qxt, off)
    assert torch.equal(dW, U.ufp4_gemm_wgrad_grouped(qdyt, qxt, off))
    dW = dW.cpu().numpy()
    r_dyt = O.quantize_segmented(tdy, off, spec_of(cs))
    r_xt = O.quantize_segmented(tx, off, spec_of(cr))
    for g in range(G):
        blk = dW[g * N:(g + 1) * N]
        if lens[g] == 0:
            assert np.all(blk == 0.0), g
            continue
        ref = O.gemm_ref(oracle_dequant64(r_dyt[g], cs), oracle_dequant64(r_xt[g], cr))
        assert O.rel_fro(blk, ref) <= F32_SCALE_TOL, g


# ---------------------------------------------------------------------------
# fp32-scale GEMMs whose K ends inside a 128-wide raw stage (and K of a single
# step), for 16- and 32-wide K steps; ragged row tiles on both operands.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("bc,K", [(16, 16), (16, 48), (16, 208), (32, 32), (32, 96), (32, 160), (32, 224)])
def test_gemm_fp32_partial_stage(grid, bc, K):
    _print_case("fp32-scale gemm, partial stage", grid, bc, K)
    n = 16 if K % 16 == 0 else 1
    cfg = U.make_cfg(grid, U.UFP4_SR, U.UFP4_SCALE_F32, 1, bc, n, sign_seed=31, sr_seed=37)
    _gemm_case(272, 300, K, cfg, cfg, seed=K + 7 * bc + grid)


# ---------------------------------------------------------------------------
# An empty shared dimension (K = 0): C = 0 and no operand storage is read
# (it may be null, as torch's empty tensors are).  Covers the kernel families
# whose first K step used to be fetched before the loop: the general
# split-bf16 kernel (mixed block widths; grouped power-of-two operands) and
# the scaled-MFMA kernel of the uniform grids; grouped WGRAD with empty
# experts in the middle and at the end, with mixed block widths.
# ---------------------------------------------------------------------------
def _empty_q(P, cfg):
    return U.QTensor(torch.empty((P, 0), dtype=torch.uint8, device="cuda"),
                     torch.empty((P, 0), dtype=U.scales_dtype(cfg), device="cuda"), P, 0, cfg)


K0_CASES = [
    ("mixed 1x16 / 1x32 fp32", U.make_cfg(U.UFP4_E1M2, U.UFP4_RTNE, U.UFP4_SCALE_F32, 1, 16, 16, sign_seed=1),
     U.make_cfg(U.UFP4_E1M2, U.UFP4_RTNE, U.UFP4_SCALE_F32, 1, 32, 16, sign_seed=1)),
    ("1x16 fp32", U.make_cfg(U.UFP4_INT4, U.UFP4_RTNE, U.UFP4_SCALE_F32, 1, 16, 16, sign_seed=1), None),
    ("1x32 E8M0 E1M2", U.make_cfg(U.UFP4_E1M2, U.UFP4_RTNE, U.UFP4_SCALE_POW2, 1, 32, 1), None),
    ("1x32 E8M0 E2M1", U.make_cfg(U.UFP4_E2M1, U.UFP4_RTNE, U.UFP4_SCALE_POW2, 1, 32, 1), None),
    ("32x32 E8M0 INT4", U.make_cfg(U.UFP4_INT4, U.UFP4_RTNE, U.UFP4_SCALE_POW2, 32, 32, 1), None),
    ("MXFP8", U.make_cfg(U.UFP4_E4M3, U.UFP4_RTNE, U.UFP4_SCALE_POW2, 1, 32, 1), None),
]


@pytest.mark.parametrize("name,cfg_a,cfg_b", K0_CASES, ids=[c[0] for c in K0_CASES])
def test_gemm_empty_k(name, cfg_a, cfg_b):
    _print_case("K = 0", name)
    cfg_b = cfg_b or cfg_a
    PA, PB = 96, 64
    qa, qb = _empty_q(PA, cfg_a), _empty_q(PB, cfg_b)
    C = torch.full((PA, PB + 8), 7.0, dtype=torch.float32, device="cuda")
    U.ufp4_gemm_fprop(qa, qb, out=C[:, :PB])
    host = C.cpu().numpy()
    assert np.all(host[:, :PB] == 0.0) and np.all(host[:, PB:] == 7.0)
    if cfg_a.grid == U.UFP4_E4M3:
        return                                   # MXFP8 GEMMs are dense only
    G = 2
    Y = torch.full((PA, 32), 7.0, dtype=torch.float32, device="cuda")
    U.ufp4_gemm_fprop_grouped(qa, _empty_q(G * 32, cfg_b), [0, 32, PA], out=Y)
    assert torch.count_nonzero(Y).item() == 0


@pytest.mark.parametrize("bc_a,bc_b", [(16, 32), (32, 16), (16, 16)])
def test_grouped_wgrad_empty_experts(bc_a, bc_b):
    """Experts 1 and 3 (the last) have no tokens: their dW is zero and the
    others match per-expert oracle products (mixed block widths run on the
    general kernel, equal ones on the scale-product kernel)."""
    _print_case("wgrad empty experts", bc_a, bc_b)
    off = [0, 64, 64, 128, 128]
    G, N, H = 4, 96, 160
    T = off[-1]
    tdy, tx = rand_bits(T, N, 81), rand_bits(T, H, 82)
    ca = U.make_cfg(U.UFP4_E1M2, U.UFP4_SR, U.UFP4_SCALE_F32, 1, bc_a, 32, sign_seed=9, sr_seed=3, sr_stream=1)
    cb = U.make_cfg(U.UFP4_E1M2, U.UFP4_RTNE, U.UFP4_SCALE_F32, 1, bc_b, 32, sign_seed=9)
    qdyt = U.ufp4_rht_quant_segmented(dev_bf16(tdy), off, ca)
    qxt = U.ufp4_rht_quant_segmented(dev_bf16(tx), off, cb)
    dW = torch.full((G * N, H), 7.0, dtype=torch.float32, device="cuda")
    U.ufp4_gemm_wgrad_grouped(qdyt, qxt, off, out=dW)
    dW = dW.cpu().numpy()
    r_dyt = O.quantize_segmented(tdy, off, spec_of(ca))
    r_xt = O.quantize_segmented(tx, off, spec_of(cb))
    for g in range(G):
        blk = dW[g * N:(g + 1) * N]
        if off[g + 1] == off[g]:
            assert np.all(blk == 0.0), g
            continue
        ref = O.gemm_ref(oracle_dequant64(r_dyt[g], ca), oracle_dequant64(r_xt[g], cb))
        assert O.rel_fro(blk, ref) <= GEMM_TOL, g


# ---------------------------------------------------------------------------
# Grouped FPROP / DGRAD with power-of-two (E8M0) scales, 1 x 32 and 32 x 32
# blocks, every grid: per-expert products against the oracle's (one expert
# empty, experts of 32, 96 and 160 tokens).
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("br", [1, 32])
def test_grouped_gemms_pow2(grid, br):
    _print_case("grouped pow2", grid, br)
    G, H, F = 4, 256, 128
    off = [0, 32, 32, 128, 288]
    T = off[-1]
    n = 1 if br == 32 else 32
    cx = U.make_cfg(grid, U.UFP4_RTNE, U.UFP4_SCALE_POW2, br, 32, n, sign_seed=44)
    cd = U.make_cfg(grid, U.UFP4_SR, U.UFP4_SCALE_POW2, br, 32, n, sign_seed=45, sr_seed=5, sr_stream=0)
    tx, tw, tdy = rand_bits(T, H, 51), rand_bits(G * F, H, 52), rand_bits(T, F, 53)
    qx, rx = compare_quant(tx, 0, cx, with_rotated=False)
    qw, rw = compare_quant(tw, 0, cx, with_rotated=False)
    dxq, dwq = oracle_dequant64(rx, cx), oracle_dequant64(rw, cx)
    for ws in (False, True):   # scaled matrix cores; FP6 operands through a workspace
        Y = (U.ufp4_gemm_ws(U.UFP4_GEMM_FPROP, qx, qw, offsets=off) if ws
             else U.ufp4_gemm_fprop_grouped(qx, qw, off)).cpu().numpy()
        for g in range(G):
            if off[g + 1] > off[g]:
                ref = O.gemm_ref(dxq[off[g]:off[g + 1]], dwq[g * F:(g + 1) * F])
                assert O.rel_fro(Y[off[g]:off[g + 1]], ref) <= GEMM_TOL, ("fprop", ws, g)
    need = U.ufp4_gemm_workspace_bytes(U.UFP4_GEMM_FPROP, qx, qw, G)
    assert need == (0 if grid == U.UFP4_E2M1 else (T * H + 255) // 256 * 256 + G * F * H)
    # DGRAD: B = W^T of every expert.  1 x 32: per-expert column-wise
    # quantization (segmented); 32 x 32: each expert's W quantized once and
    # reused transposed (S(B) = S(B^T)), stacked.
    qdy, rdy = compare_quant(tdy, 0, cd.copy(sign_seed=46), with_rotated=False)
    cwt = cx.copy(sign_seed=46)
    if br == 1:
        qwt = U.stacked(U.ufp4_rht_quant_segmented(dev_bf16(tw), [g * F for g in range(G + 1)], cwt), G)
        refs = O.quantize_segmented(tw, [g * F for g in range(G + 1)], spec_of(cwt))
        dwt = [oracle_dequant64(r, cwt) for r in refs]
    else:
        qwe = U.ufp4_rht_quant(dev_bf16(tw), 0, cwt)[0]
        t = U.ufp4_transpose_qtensor(U.QTensor(qwe.codes[:F], qwe.scales[:F // 32], F, H, cwt))
        parts = [t]
        for g in range(1, G):
            parts.append(U.ufp4_transpose_qtensor(U.QTensor(qwe.codes[g * F:(g + 1) * F],
                                                            qwe.scales[g * F // 32:(g + 1) * F // 32],
                                                            F, H, cwt)))
        qwt = U.QTensor(torch.cat([p.codes for p in parts]), torch.cat([p.scales for p in parts]),
                        G * H, F, cwt)
        rwe = O.quantize(tw, 0, spec_of(cwt))
        dwe = oracle_dequant64(rwe, cwt)
        dwt = [np.ascontiguousarray(dwe[g * F:(g + 1) * F].T) for g in range(G)]
    ddy = oracle_dequant64(rdy, cd.copy(sign_seed=46))
    for ws in (False, True):
        dX = (U.ufp4_gemm_ws(U.UFP4_GEMM_DGRAD, qdy, qwt, offsets=off) if ws
              else U.ufp4_gemm_dgrad_grouped(qdy, qwt, off)).cpu().numpy()
        for g in range(G):
            if off[g + 1] > off[g]:
                ref = O.gemm_ref(ddy[off[g]:off[g + 1]], dwt[g])
                assert O.rel_fro(dX[off[g]:off[g + 1]], ref) <= GEMM_TOL, ("dgrad", ws, g)


@pytest.mark.parametrize("grid", GRIDS)
def test_grouped_wgrad_pow2(grid):
    """Grouped WGRAD with 1 x 32 E8M0 blocks on the scaled matrix cores: four
    token segments (one empty) of the segmented column-wise quantizations of
    dY and X, plain and through the workspace; segment lengths that are not
    multiples of 128 are refused (UFP4_ERR_UNSUPPORTED)."""
    _print_case("grouped wgrad pow2", grid)
    G, H, F = 4, 288, 160
    off = [0, 128, 128, 384, 640]
    T = off[-1]
    cdt = U.make_cfg(grid, U.UFP4_SR, U.UFP4_SCALE_POW2, 1, 32, 32, sign_seed=61, sr_seed=3, sr_stream=1)
    cxt = U.make_cfg(grid, U.UFP4_RTNE, U.UFP4_SCALE_POW2, 1, 32, 32, sign_seed=61)
    tdy, tx = rand_bits(T, F, 62), rand_bits(T, H, 63)
    qdyt = U.ufp4_rht_quant_segmented(dev_bf16(tdy), off, cdt)
    qxt = U.ufp4_rht_quant_segmented(dev_bf16(tx), off, cxt)
    r_dyt = O.quantize_segmented(tdy, off, spec_of(cdt))
    r_xt = O.quantize_segmented(tx, off, spec_of(cxt))
    assert np.array_equal(qdyt.codes.cpu().numpy(), np.concatenate([r["codes"].ravel() for r in r_dyt]))
    assert np.array_equal(qdyt.scales.cpu().numpy(), np.concatenate([r["scales"].ravel() for r in r_dyt]))
    for ws in (False, True):
        dW = torch.full((G * F, H), 7.0, dtype=torch.float32, device="cuda")
        if ws:
            U.ufp4_gemm_ws(U.UFP4_GEMM_WGRAD, qdyt, qxt, offsets=off, out=dW)
        else:
            U.ufp4_gemm_wgrad_grouped(qdyt, qxt, off, out=dW)
        dW = dW.cpu().numpy()
        for g in range(G):
            if off[g + 1] == off[g]:
                assert np.all(dW[g * F:(g + 1) * F] == 0), ("empty", ws)
                continue
            ref = O.gemm_ref(oracle_dequant64(r_dyt[g], cdt), oracle_dequant64(r_xt[g], cxt))
            assert O.rel_fro(dW[g * F:(g + 1) * F], ref) <= GEMM_TOL, ("wgrad", ws, g)
    off2 = [0, 96, 96, 384, 640]
    qdy2 = U.ufp4_rht_quant_segmented(dev_bf16(tdy), off2, cdt)
    qx2 = U.ufp4_rht_quant_segmented(dev_bf16(tx), off2, cxt)
    with pytest.raises(U.UFP4Error) as e:
        U.ufp4_gemm_wgrad_grouped(qdy2, qx2, off2)
    assert e.value.status == U.UFP4_ERR_UNSUPPORTED


@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("rnd", [U.UFP4_RTNE, U.UFP4_SR])
@pytest.mark.parametrize("b", [16, 32])
def test_quant_dual_n128(grid, rnd, b):
    """Dual-axis calls with n = 128 (128 x 128 tiles, one per workgroup; both
    dimensions are multiples of 128, so every tile is whole): 384 x 256 (six
    tiles) and 384 x 128 (three), and expert segments of 256, 0 and 128 rows,
    against the oracle's row-wise and (per-segment) column-wise quantizations."""
    _print_case("dual n128", grid, rnd, b)
    cr = U.make_cfg(grid, rnd, U.UFP4_SCALE_F32, 1, b, 128, sign_seed=61, sr_seed=5, sr_stream=0)
    cc = U.make_cfg(grid, rnd, U.UFP4_SCALE_F32, 1, b, 128, sign_seed=62, sr_seed=5, sr_stream=1)
    for rows, cols in ((384, 256), (384, 128)):
        bits = rand_bits(rows, cols, 70 + cols)
        qr, qc = U.ufp4_rht_quant_dual(dev_bf16(bits), cr, cc)
        torch.cuda.synchronize()
        _assert_q_equal(qr, O.quantize(bits, 0, spec_of(cr)), "row")
        _assert_q_equal(qc, O.quantize(bits, 1, spec_of(cc)), "col")
    offs = [0, 256, 256, 384]
    bits = rand_bits(384, 256, 79)
    qr, qc = U.ufp4_rht_quant_dual(dev_bf16(bits), cr, cc, row_offsets=offs)
    torch.cuda.synchronize()
    _assert_q_equal(qr, O.quantize(bits, 0, spec_of(cr)), "row")
    segs = [O.quantize(bits[lo:hi], 1, spec_of(cc), elem_base=bits.shape[1] * lo)
            for lo, hi in zip(offs[:-1], offs[1:]) if hi > lo]
    ref = {"codes": np.concatenate([np.asarray(r["codes"]).reshape(-1) for r in segs]),
           "scales": np.concatenate([np.asarray(r["scales"]).reshape(-1) for r in segs])}
    _assert_q_equal(qc, ref, "col")


@pytest.mark.parametrize("grid", [U.UFP4_E1M2, U.UFP4_INT4, U.UFP4_E2M1])
@pytest.mark.parametrize("br", [1, 32])
@pytest.mark.parametrize("K", [128, 384, 160])
def test_gemm_ws_fp6(grid, br, K):
    """The workspace entry point: E1M2 / INT4 with 32-element E8M0 blocks and
    K % 128 == 0 run as FP6 E2M3 operands after the expansion into the
    workspace; E2M1 and K = 160 take no workspace (0 bytes) and run as the
    plain call.  3 ragged row tiles of A, 2 of B; all three operations."""
    _print_case("gemm ws fp6", grid, br, K)
    cfg = U.make_cfg(grid, U.UFP4_SR if br == 32 else U.UFP4_RTNE, U.UFP4_SCALE_POW2, br, 32,
                     1 if br == 32 else 32, sign_seed=6, sr_seed=91)
    ta, tb = rand_bits(544, K, 41), rand_bits(288, K, 42)
    qa, ra = compare_quant(ta, 0, cfg, with_rotated=False)
    qb, rb = compare_quant(tb, 0, cfg, with_rotated=False)
    need = U.ufp4_gemm_workspace_bytes(U.UFP4_GEMM_FPROP, qa, qb)
    fp6 = grid != U.UFP4_E2M1 and K % 128 == 0
    assert need == ((544 * K + 255) // 256 * 256 + 288 * K if fp6 else 0)
    ref = O.gemm_ref(oracle_dequant64(ra, cfg), oracle_dequant64(rb, cfg))
    for op in (U.UFP4_GEMM_FPROP, U.UFP4_GEMM_DGRAD, U.UFP4_GEMM_WGRAD):
        C = U.ufp4_gemm_ws(op, qa, qb).cpu().numpy()
        err = O.rel_fro(C, ref)
        assert err <= GEMM_TOL, (op, err)
    # a workspace reused by a second, smaller call on the same stream
    if fp6:
        ws = torch.full((need,), 0xAB, dtype=torch.uint8, device="cuda")
        U.ufp4_gemm_ws(U.UFP4_GEMM_FPROP, qa, qb, workspace=ws)
        qa2 = U.QTensor(qa.codes[:256], qa.scales[:256 // br], 256, K, qa.cfg)
        C2 = U.ufp4_gemm_ws(U.UFP4_GEMM_FPROP, qa2, qb, workspace=ws).cpu().numpy()
        ra2 = dict(ra, codes=ra["codes"][:256], scales=ra["scales"][:256 // br], P=256)
        assert O.rel_fro(C2, O.gemm_ref(oracle_dequant64(ra2, cfg), oracle_dequant64(rb, cfg))) <= GEMM_TOL


@pytest.mark.parametrize("grid", [U.UFP4_E1M2, U.UFP4_INT4])
def test_gemm_ws_fp6_every_code(grid):
    """Random code bytes (every code of the grid, E1M2's negative zero
    included; INT4's nibble 8 is no code of {-7..7} and is replaced by 0) and
    random E8M0 scales straight into the FP6 path, against the oracle's decode
    of the same codes; the plain call agrees as well."""
    _print_case("gemm ws fp6 codes", grid)
    rng = np.random.default_rng(grid + 3)
    P_a, P_b, K = 320, 96, 256
    cfg = U.make_cfg(grid, U.UFP4_RTNE, U.UFP4_SCALE_POW2, 1, 32, 1)
    ca = rng.integers(0, 256, size=(P_a, K // 2), dtype=np.uint8)
    cb = rng.integers(0, 256, size=(P_b, K // 2), dtype=np.uint8)
    if grid == U.UFP4_INT4:
        for c in (ca, cb):
            c[(c & 0x0F) == 8] &= 0xF0
            c[(c >> 4) == 8] &= 0x0F
    sa = rng.integers(118, 136, size=(P_a, K // 32), dtype=np.uint8)
    sb = rng.integers(118, 136, size=(P_b, K // 32), dtype=np.uint8)
    dev = lambda a: torch.from_numpy(a).cuda()  # noqa: E731
    qa = U.QTensor(dev(ca), dev(sa), P_a, K, cfg)
    qb = U.QTensor(dev(cb), dev(sb), P_b, K, cfg)
    spec = spec_of(cfg)
    da = O.dequant(ca, sa, spec, P_a, K)[1]
    db = O.dequant(cb, sb, spec, P_b, K)[1]
    ref = O.gemm_ref(da, db)
    assert U.ufp4_gemm_workspace_bytes(U.UFP4_GEMM_FPROP, qa, qb) > 0
    C = U.ufp4_gemm_ws(U.UFP4_GEMM_FPROP, qa, qb).cpu().numpy()
    assert O.rel_fro(C, ref) <= GEMM_TOL
    C0 = U.ufp4_gemm_fprop(qa, qb).cpu().numpy()
    assert O.rel_fro(C0, ref) <= GEMM_TOL


TWO_LEVEL = [(U.UFP4_E1M2, 1, 32), (U.UFP4_INT4, 1, 32), (U.UFP4_E2M1, 1, 32),
             (U.UFP4_E1M2, 32, 1), (U.UFP4_E2M1, 32, 1), (U.UFP4_E4M3, 1, 32)]
# MXFP8 rounds to nearest even only
TWO_LEVEL_CASES = [(g, br, n, r) for g, br, n in TWO_LEVEL for r in (U.UFP4_RTNE, U.UFP4_SR)
                   if not (g == U.UFP4_E4M3 and r == U.UFP4_SR)]


@pytest.mark.parametrize("grid,br,n,rnd", TWO_LEVEL_CASES)
def test_two_level_quant(grid, br, n, rnd):
    """Two-level scaling (a per-tensor fp32 factor over power-of-two block
    scales): bit-exact codes, E8M0 bytes and dequantized values row-wise
    and column-wise (1D), and both sides of a dual-axis call with different
    factors."""
    _print_case("two-level quant", grid, br, n, rnd)
    ts = 0.37
    cfg = U.make_cfg(grid, rnd, U.UFP4_SCALE_POW2, br, 32, n, sign_seed=71, sr_seed=72,
                     tensor_scale=ts)
    bits = rand_bits(96, 192, 73)
    for along in ((0, 1) if br == 1 else (0,)):
        q, ref = compare_quant(bits, along, cfg, with_rotated=True)
        d = U.ufp4_dequant(q).cpu().numpy()
        want = O.dequant(ref["codes"], ref["scales"], spec_of(cfg), q.P, q.K)[0]
        assert f32_bits_equal(d, want), ("dequant", along)
    if br == 1 and grid != U.UFP4_E4M3:
        cr = cfg.copy(tensor_scale=1.9)
        cc = cfg.copy(tensor_scale=3.0e-4, sign_seed=74, sr_stream=1)
        qr, qc = U.ufp4_rht_quant_dual(dev_bf16(bits), cr, cc)
        for q, ref in ((qr, O.quantize(bits, 0, spec_of(cr))), (qc, O.quantize(bits, 1, spec_of(cc)))):
            assert np.array_equal(q.scales.cpu().numpy().reshape(-1), np.asarray(ref["scales"]).reshape(-1))
            assert np.array_equal(q.codes.cpu().numpy().reshape(-1), np.asarray(ref["codes"]).reshape(-1))


@pytest.mark.parametrize("grid,br,n", [c for c in TWO_LEVEL if c[0] != U.UFP4_E4M3] +
                         [(U.UFP4_E4M3, 1, 32)])
@pytest.mark.parametrize("K", [256, 160])
def test_two_level_gemm(grid, br, n, K):
    """GEMMs of two-level operands (different factors on A and B) against
    the oracle's product of the dequantized operands: the scaled matrix
    cores (K = 256), FP6 through a workspace (E1M2 / INT4), and the general
    kernel (K = 160; MXFP8 refuses it)."""
    _print_case("two-level gemm", grid, br, n, K)
    ca = U.make_cfg(grid, U.UFP4_RTNE, U.UFP4_SCALE_POW2, br, 32, n, sign_seed=81, tensor_scale=0.021)
    cb = ca.copy(tensor_scale=5.5)
    ta, tb = rand_bits(320, K, 82), rand_bits(288, K, 83)
    qa, ra = compare_quant(ta, 0, ca, with_rotated=False)
    qb, rb = compare_quant(tb, 0, cb, with_rotated=False)
    ref = O.gemm_ref(oracle_dequant64(ra, ca), oracle_dequant64(rb, cb))
    if grid == U.UFP4_E4M3 and K % 128:
        with pytest.raises(U.UFP4Error):
            U.ufp4_gemm_fprop(qa, qb)
        return
    C = U.ufp4_gemm_fprop(qa, qb).cpu().numpy()
    assert O.rel_fro(C, ref) <= GEMM_TOL
    if grid in (U.UFP4_E1M2, U.UFP4_INT4) and K % 128 == 0:
        assert U.ufp4_gemm_workspace_bytes(U.UFP4_GEMM_FPROP, qa, qb) > 0
        C6 = U.ufp4_gemm_ws(U.UFP4_GEMM_FPROP, qa, qb).cpu().numpy()
        assert O.rel_fro(C6, ref) <= GEMM_TOL
