"""Pins of the CPU oracle to facts fixed outside the oracle itself: the pages'
equations, closed forms, library routines and brute force on tiny inputs.

Each test names the page passage it checks.  Pages:
  [UFP4]  "Rethinking Shrinkage Bias in FP4 Pretraining of LLMs ... the UFP4
          Recipe" (hyper.ai summary: formats section, Method; abstract)
  [2DFP4] "Stable FP4 Training via Transposition-Invariant Block Quantization"
          (agifrontier tutorial: root cause, 2D square-block quantization)
"""
import os
import subprocess
import tempfile
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


# ---------------------------------------------------------------------------
# Philox4x32-10 (published method, Salmon et al. SC'11) against rocRAND's
# independent header-only engine, run on the host.
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def rocrand_ref():
    exe = os.path.join(tempfile.mkdtemp(), "philox_ref")
    src = os.path.join(HERE, "rocrand_philox_ref.cpp")
    r = subprocess.run(["hipcc", "-O1", "-o", exe, src], capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("hipcc host build of the rocRAND reference failed: " + r.stderr[-400:])
    return exe


def test_philox_matches_rocrand(rocrand_ref):
    rng = np.random.default_rng(7)
    cases = [(0, 0, 0), (123456789, 0xFFFFFFFF, 0), (2 ** 64 - 1, 3, 2 ** 40 + 5),
             (2201, 0, 1), (2201, 1, 2 ** 33 - 1)]
    for _ in range(60):
        cases.append((int(rng.integers(0, 2 ** 63)), int(rng.integers(0, 2 ** 32)),
                      int(rng.integers(0, 2 ** 61))))
    inp = "\n".join(f"{s} {ss} {b}" for s, ss, b in cases) + "\n"
    out = subprocess.run([rocrand_ref], input=inp, capture_output=True, text=True, check=True)
    lines = out.stdout.strip().splitlines()
    assert len(lines) == len(cases)
    for (s, ss, b), line in zip(cases, lines):
        ctr = [[b & 0xFFFFFFFF, b >> 32, ss & 0xFFFFFFFF, ss >> 32]]
        got = O.philox4x32_10(ctr, O.split_seed(s))[0]
        assert [int(x, 16) for x in line.split()] == [int(v) for v in got], (s, ss, b)


def test_sr_draw_layout_matches_rocrand_stream(rocrand_ref):
    """16-bit draws of 8 consecutive elements come from one Philox block."""
    seed, stream = 2201, 1
    e = np.arange(64, dtype=np.int64) + 8 * 1000
    r16 = O.sr_draws(seed, stream, e)
    inp = "".join(f"{seed} {stream} {g}\n" for g in range(1000, 1008))
    out = subprocess.run([rocrand_ref], input=inp, capture_output=True, text=True, check=True)
    words = [int(w, 16) for line in out.stdout.split("\n") if line for w in line.split()]
    want = []
    for w in words:
        want += [w & 0xFFFF, w >> 16]
    assert r16.tolist() == want


# ---------------------------------------------------------------------------
# bf16 decode against torch's cast.
# ---------------------------------------------------------------------------
def test_bf16_decode_matches_torch():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    mine = O.bf16_bits_to_f32(bits)
    fin = np.isfinite(t)
    assert np.array_equal(mine[fin].view(np.uint32), t[fin].view(np.uint32))
    assert np.array_equal(np.isnan(mine), np.isnan(t))


# ---------------------------------------------------------------------------
# [UFP4] Method, Sylvester recursion and orthogonality H_n^T H_n = I.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64, 128])
def test_fwht_is_sylvester_hadamard(n):
    H = O.fwht(np.eye(n, dtype=np.float64), n)           # rows e_i H
    assert np.array_equal(H, scipy.linalg.hadamard(n).astype(np.float64))
    Hn = H / np.sqrt(n)
    assert np.allclose(Hn.T @ Hn, np.eye(n), atol=1e-15, rtol=0)


@pytest.mark.parametrize("n", [4, 16, 64])
def test_hadamard_orthogonal_exact_for_powers_of_four(n):
    H = O.fwht(np.eye(n, dtype=np.float64), n) * O.rht_norm_const(n)   # c_n exact
    assert np.array_equal(H.T @ H, np.eye(n))


def test_norm_const_is_nearest_fp32():
    for n in [1, 2, 4, 8, 16, 32, 64, 128]:
        c = O.rht_norm_const(n)
        exact = 1 / np.sqrt(np.float64(n))
        below, above = np.nextafter(c, np.float32(0)), np.nextafter(c, np.float32(1))
        assert abs(float(c) - exact) <= abs(float(below) - exact)
        assert abs(float(c) - exact) <= abs(float(above) - exact)
    assert O.rht_norm_const(16) == np.float32(0.25) and O.rht_norm_const(1) == 1


@pytest.mark.parametrize("n", [2, 16, 32, 128])
def test_signs_are_pm_one_and_seeded(n):
    s = O.rht_signs(2101, n)
    assert set(np.unique(s)) <= {-1.0, 1.0}
    assert np.array_equal(s, O.rht_signs(2101, n))
    assert np.array_equal(O.rht_signs(2101, 128)[:n], s)   # prefix property
    assert not np.array_equal(O.rht_signs(2102, 128), O.rht_signs(2101, 128))


# ---------------------------------------------------------------------------
# [UFP4] Method, invariance: X W^T = (X H')(W H')^T with H' = S_n H_n, also
# block-diagonally along K (K a multiple of n) and with zero-padded rows.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n", [16, 32, 128])
def test_rotation_cancels_on_shared_dimension(n):
    rng = np.random.default_rng(n)
    X = rng.standard_normal((24, 4 * n))
    W = rng.standard_normal((40, 4 * n))
    eps = np.tile(O.rht_signs(99, n), 4)
    rot = lambda A: O.fwht(A * eps, n) / np.sqrt(n)  # noqa: E731  (fp64)
    ref = X @ W.T
    got = rot(X) @ rot(W).T
    assert np.abs(got - ref).max() <= 1e-12 * np.abs(ref).max()
    # the oracle's fp32 rotation agrees with the fp64 one within its bound
    Xf = X.astype(np.float32)
    y32 = O.rht(Xf, n, 99).astype(np.float64)
    y64 = rot(Xf.astype(np.float64))
    bound = (np.log2(n) + 1) * 2.0 ** -24 * np.abs(Xf).reshape(24, 4, n).sum(-1).max() / np.sqrt(n)
    assert np.abs(y32 - y64).max() <= bound


def test_rht_closed_forms():
    n = 16
    eps = O.rht_signs(5, n).astype(np.float32)
    # x = eps => S x = ones => H ones = (n, 0, ...) => y = (n c_n, 0...) = (4, 0...)
    y = O.rht(eps[None, :], n, 5)
    assert y[0, 0] == np.float32(4.0) and np.all(y[0, 1:] == 0)
    # one-hot input -> every entry +-c_n
    for n in (16, 32, 128):
        e = np.zeros((1, n), np.float32)
        e[0, 3] = 1
        y = O.rht(e, n, 11)
        assert np.all(np.abs(y) == O.rht_norm_const(n))
    # n = 1 is the identity (H_1 = [1])
    a = np.random.default_rng(0).standard_normal((3, 8)).astype(np.float32)
    assert np.array_equal(O.rht(a, 1, 0), a)


# ---------------------------------------------------------------------------
# Scales. [UFP4] formats: s_B = absmax / qmax.  [2DFP4] 2D section:
# S = 2^ceil(log2(2M/(Qp - Qn))) keeps the block maximum inside the range.
# ---------------------------------------------------------------------------
def test_f32_scale_within_one_ulp():
    rng = np.random.default_rng(1)
    M = np.abs(rng.standard_normal(20000)).astype(np.float32) * np.float32(3.0)
    for g in (O.E1M2, O.INT4, O.E2M1):
        s = O.scale_f32(M, g)
        err = np.abs(s.astype(np.float64) * O.QMAX[g] - M.astype(np.float64))
        ulp = np.spacing(s).astype(np.float64) * O.QMAX[g]
        assert np.all(err <= 0.5 * ulp + 1e-300)


def test_pow2_exponent_brackets_block_max_exactly():
    rng = np.random.default_rng(2)
    M = np.concatenate([np.abs(rng.standard_normal(500)) * 10.0 ** rng.integers(-30, 30, 500),
                        [6.0, 1.75, 7.0, 12.0, 3.5, 448.0, 896.0, 0.0, 1e-40]]).astype(np.float32)
    for g in (O.E1M2, O.INT4, O.E2M1, O.E4M3):
        e = O.scale_pow2_exponent(M, g)
        assert np.array_equal(e, O.scale_pow2_exponent_exact(M, g))
        q = Fraction(O.QMAX[g]).limit_denominator(8)
        for m, ee in zip(M, e):
            if m == 0:
                assert ee == -127
                continue
            fm = Fraction(float(m))
            assert fm <= q * Fraction(2) ** int(ee)
            if ee > -127:
                assert fm > q * Fraction(2) ** (int(ee) - 1)


def _tensor_bits(P, K, seed, scale=1.0):
    x = torch.from_numpy(np.random.default_rng(seed).standard_normal((P, K)).astype(np.float32) * scale)
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_e1m2_equals_int4_over_four():
    """Uniform grids: E1M2 levels are INT4 levels / 4, so scales differ by
    exactly 4 and the level indices coincide (power-of-two scaling commutes
    with round-to-nearest)."""
    t = _tensor_bits(64, 256, 3)
    for rnd in (O.RTNE, O.SR):
        a = O.quantize(t, 0, O.QuantSpec(O.E1M2, rnd, O.SCALE_F32, 1, 16, 16, 7, 9, 0))
        b = O.quantize(t, 0, O.QuantSpec(O.INT4, rnd, O.SCALE_F32, 1, 16, 16, 7, 9, 0))
        assert np.array_equal(a["scales"], (b["scales"] * np.float32(4)).astype(np.float32))
        ka, na = O.decode_index(a["code"], O.E1M2)
        kb, nb = O.decode_index(b["code"], O.INT4)
        assert np.array_equal(ka, kb) and np.array_equal(na, nb)


@pytest.mark.parametrize("grid", [O.E2M1, O.E1M2])
@pytest.mark.parametrize("b", [16, 32])
def test_square_block_scale_transpose_invariant(grid, b):
    """[2DFP4] 2D section: S(B) = S(B^T) for square blocks (its block-size
    comparison favours 16 x 16 to 32 x 32)."""
    t = _tensor_bits(128, 96, 4)
    spec = O.QuantSpec(grid, O.RTNE, O.SCALE_POW2, b, b, 1)
    a = O.quantize(t, 0, spec)
    b = O.quantize(t, 1, spec)          # logical operand T^T
    assert np.array_equal(a["scales"].T, b["scales"])
    assert np.array_equal(a["code"].T, b["code"])     # RTNE: codes transpose too
    # 1 x 32 blocks do not have the property (the motivation on the page)
    spec1 = O.QuantSpec(grid, O.RTNE, O.SCALE_POW2, 1, 32, 1)
    a1 = O.quantize(t, 0, spec1)
    b1 = O.quantize(t, 1, spec1)
    assert not np.array_equal(O.scale_per_element(a1["scales"], spec1, 128, 96).T,
                              O.scale_per_element(b1["scales"], spec1, 96, 128))


# ---------------------------------------------------------------------------
# Rounding.  [UFP4] formats: RTNE and SR onto the codebook.
# ---------------------------------------------------------------------------
def _sweep(qmax):
    base = np.linspace(0, qmax, 40001)
    ties = np.arange(0, qmax * 8 + 1) / 8.0
    extra = np.array([np.nextafter(t, -1) for t in ties if t > 0] + [np.nextafter(t, 10) for t in ties])
    return np.unique(np.concatenate([base, ties, extra, [qmax]]).astype(np.float32).astype(np.float64))


@pytest.mark.parametrize("grid,delta", [(O.E1M2, 0.25), (O.INT4, 1.0)])
def test_rtne_uniform_is_rint(grid, delta):
    m = _sweep(O.QMAX[grid])
    m = m[m <= O.QMAX[grid]]
    assert np.array_equal(O.round_rtne_index(m, grid), np.rint(m / delta).astype(np.int64))


def test_rtne_e2m1_is_one_mantissa_bit_round_half_even():
    m = _sweep(6.0)
    m = m[m <= 6.0]
    # reformulation: spacing 0.5 below 2 (incl. subnormals), 2^(e-1) above
    e = np.floor(np.log2(np.maximum(m, 1.0)))
    spacing = np.where(m < 2.0, 0.5, 2.0 ** (e - 1))
    val = np.rint(m / spacing) * spacing
    got = O.LEVELS[O.E2M1][O.round_rtne_index(m, O.E2M1)]
    assert np.array_equal(got, np.minimum(val, 6.0))


@pytest.mark.parametrize("grid", [O.E1M2, O.INT4, O.E2M1])
def test_sr_probability_exact(grid):
    """Enumerating all 2^16 draws: P(round up) = ceil(f 2^16) / 2^16, and the
    result is always one of the two neighbouring levels."""
    L = O.LEVELS[grid]
    r = np.arange(65536)
    rng = np.random.default_rng(5)
    for m in np.concatenate([rng.uniform(0, L[-1], 25), L, [L[-1]]]).astype(np.float32):
        m = float(m)
        k = O.round_sr_index(np.full(r.size, m), grid, r)
        lo = np.searchsorted(L, m, side="right") - 1
        if lo == L.size - 1:
            assert np.all(k == lo)
            continue
        f = (m - L[lo]) / (L[lo + 1] - L[lo])
        assert set(np.unique(k)) <= {lo, lo + 1}
        assert (k == lo + 1).sum() == int(np.ceil(f * 65536))


@pytest.mark.parametrize("grid", [O.E1M2, O.E2M1])
def test_sr_mean_error_vanishes(grid):
    """[2DFP4] 2D section: E[roundS(x)] = x, with draws from the real
    Philox stream: |mean - m| <= 5 sigma / sqrt(N) + spacing 2^-16."""
    N = 1 << 20
    r16 = O.sr_draws(31337, 0, np.arange(N))
    L = O.LEVELS[grid]
    for m in (0.1, 0.6, 1.3, 1.7):
        k = O.round_sr_index(np.full(N, m), grid, r16)
        vals = L[k]
        lo = np.searchsorted(L, m, side="right") - 1
        gap = L[lo + 1] - L[lo]
        sigma = gap / 2
        assert abs(vals.mean() - m) <= 5 * sigma / np.sqrt(N) + gap * 2.0 ** -16


def _bin_bias(grid):
    """E[rho(t) - t | t in bin of q_i] by dense integration of the oracle's
    RTNE, for every interior level q_i."""
    L = O.LEVELS[grid]
    t = np.linspace(0, L[-1], 2_000_001)[1:-1]
    k = O.round_rtne_index(t, grid)
    out = {}
    for i in range(1, L.size - 1):
        sel = k == i
        out[L[i]] = float((L[i] - t[sel]).mean())
    return out


@pytest.mark.parametrize("grid", [O.E1M2, O.INT4, O.E2M1])
def test_bin_bias_closed_form(grid):
    """[UFP4] Method, Shrinkage Bias: E[rho(t) - t | t in B_i] =
    (l_i - r_i)/2 = (2 q_i - q_{i-1} - q_{i+1}) / 4 under a locally uniform
    density; zero for uniform grids, nonzero at E2M1's spacing changes."""
    L = O.LEVELS[grid]
    got = _bin_bias(grid)
    for i in range(1, L.size - 1):
        closed = (2 * L[i] - L[i - 1] - L[i + 1]) / 4
        assert abs(got[L[i]] - closed) <= 1e-5 * max(1.0, L[-1])
    if grid == O.E2M1:
        assert abs(got[2.0] + 0.125) < 1e-5 and abs(got[4.0] + 0.25) < 1e-5
        assert all(abs(got[q]) < 1e-5 for q in (0.5, 1.0, 1.5, 3.0))
    else:
        assert all(abs(v) < 1e-5 for v in got.values())


# ---------------------------------------------------------------------------
# Encoding.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("grid", [O.E1M2, O.INT4, O.E2M1])
def test_encode_round_trip_and_canonical_zero(grid):
    k = np.repeat(np.arange(8), 2)
    neg = np.tile([False, True], 8)
    c = O.encode(k, neg, grid)
    assert c[0] == 0 and c[1] == 0                # -0 encodes as +0
    assert len(set(c.tolist())) == 15
    kk, nn = O.decode_index(c, grid)
    assert np.array_equal(kk, k) and np.array_equal(nn, neg & (k > 0))
    if grid == O.E2M1:   # OCP FP4 bit pattern: sign | exp(2) | mantissa(1)
        assert O.encode([7], [True], grid)[0] == 0b1111 and O.encode([2], [False], grid)[0] == 0b0010
    if grid == O.INT4:
        assert O.encode([7], [True], grid)[0] == 0b1001
    p = O.pack_nibbles(c.reshape(1, -1))
    assert np.array_equal(O.unpack_nibbles(p)[0], c)
    assert p[0, 1] == (c[2] | (c[3] << 4))


# ---------------------------------------------------------------------------
# Dequantization and GEMM: brute force and the lossless special case.
# ---------------------------------------------------------------------------
def test_gemm_brute_force_tiny():
    rng = np.random.default_rng(9)
    spec = O.QuantSpec(O.E2M1, O.RTNE, O.SCALE_F32, 1, 16, 16, 3)
    ta, tb = _tensor_bits(3, 32, 10), _tensor_bits(2, 32, 11)
    qa, qb = O.quantize(ta, 0, spec), O.quantize(tb, 0, spec)
    _, da = O.dequant(qa["codes"], qa["scales"], spec, 3, 32)
    _, db = O.dequant(qb["codes"], qb["scales"], spec, 2, 32)
    C = O.gemm_ref(da, db)
    for p in range(3):
        for q in range(2):
            acc = Fraction(0)
            for k in range(32):
                acc += Fraction(float(da[p, k])) * Fraction(float(db[q, k]))
            assert abs(float(acc) - C[p, q]) <= 1e-12 * max(1.0, abs(float(acc)))
    del rng


def test_lossless_on_grid_inputs():
    """n = 1 and every 1 x 16 block a multiple of (absmax / 7) on the INT4 grid:
    Q(T) = T, so the quantized GEMM equals the textbook product X W^T."""
    rng = np.random.default_rng(12)
    P, Q, K = 8, 6, 64

    def on_grid(rows):
        k = rng.integers(-7, 8, (rows, K)).astype(np.float64)
        k[:, ::16] = 7                                   # absmax 7 in every block
        s = 2.0 ** rng.integers(-4, 4, (rows, K // 16))
        return k * np.repeat(s, 16, axis=1)

    X, W = on_grid(P), on_grid(Q)
    tb = lambda A: torch.from_numpy(A.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)  # noqa: E731
    spec = O.QuantSpec(O.INT4, O.RTNE, O.SCALE_F32, 1, 16, 1)
    qx, qw = O.quantize(tb(X), 0, spec), O.quantize(tb(W), 0, spec)
    _, dx = O.dequant(qx["codes"], qx["scales"], spec, P, K)
    _, dw = O.dequant(qw["codes"], qw["scales"], spec, Q, K)
    assert np.array_equal(dx, X) and np.array_equal(dw, W)
    assert np.array_equal(O.gemm_ref(dx, dw), X @ W.T)


def test_dequant_fp32_is_rounded_exact():
    t = _tensor_bits(16, 64, 13)
    spec = O.QuantSpec(O.E1M2, O.SR, O.SCALE_F32, 1, 16, 16, 1, 2, 3)
    q = O.quantize(t, 0, spec)
    d32, d64 = O.dequant(q["codes"], q["scales"], spec, 16, 64)
    assert np.array_equal(d32, d64.astype(np.float32))
    # scales reproduce the block absmax through the top level
    M = O.block_absmax(q["rotated"], 1, 16)
    assert np.array_equal(q["scales"], O.scale_f32(M, O.E1M2))


def test_quantize_error_small_relative_to_scale():
    """Every dequantized element is within one level spacing * s of y (SR) or
    half a spacing (RTNE, uniform grid)."""
    t = _tensor_bits(32, 128, 14)
    for rnd, frac in ((O.RTNE, 0.5), (O.SR, 1.0)):
        spec = O.QuantSpec(O.INT4, rnd, O.SCALE_F32, 1, 16, 16, 4, 5, 6)
        q = O.quantize(t, 0, spec)
        _, d = O.dequant(q["codes"], q["scales"], spec, 32, 128)
        s = O.scale_per_element(q["scales"], spec, 32, 128)
        assert np.all(np.abs(d - q["rotated"]) <= frac * s * (1 + 1e-6) + 1e-30)


def test_segmented_draw_indices_continue():
    t = _tensor_bits(64, 16, 15)
    spec = O.QuantSpec(O.E1M2, O.SR, O.SCALE_F32, 1, 32, 32, 1, 7, 1)
    segs = O.quantize_segmented(t, [0, 32, 64], spec)
    whole_first = O.quantize(t[:32], 1, spec)
    assert np.array_equal(segs[0]["codes"], whole_first["codes"])
    second = O.quantize(t[32:], 1, spec, elem_base=16 * 32)
    assert np.array_equal(segs[1]["codes"], second["codes"])


@pytest.mark.parametrize("grid", [O.E1M2, O.INT4, O.E2M1])
def test_pow2_1x32_lossless_on_grid(grid):
    """1 x 32 power-of-two blocks ([2DFP4] scale equation applied to 1D
    blocks): a tensor whose blocks are codebook levels times 2^e, with the
    largest level present in every block, is reproduced exactly by
    quantization + dequantization, and the stored exponent is e."""
    rng = np.random.default_rng(5)
    lv = O.LEVELS[grid]
    P, K = 8, 128
    e = rng.integers(-20, 20, size=(P, K // 32))
    idx = rng.integers(0, len(lv), size=(P, K))
    sgn = rng.choice([-1.0, 1.0], size=(P, K))
    idx[:, ::32] = len(lv) - 1                       # qmax in every block
    vals = sgn * lv[idx] * np.repeat(2.0 ** e, 32, axis=1)
    bits = torch.from_numpy(vals.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.bf16_bits_to_f32(bits).astype(np.float64), vals)   # exact in bf16
    spec = O.QuantSpec(grid, O.RTNE, O.SCALE_POW2, 1, 32, 1)
    r = O.quantize(bits, 0, spec)
    assert np.array_equal(r["scales"].astype(np.int64), e + 127)
    d32, d64 = O.dequant(r["codes"], r["scales"], spec, P, K)
    assert np.array_equal(d64, vals)


# ---------------------------------------------------------------------------
# Worked examples of the printed equations (tests/golden/, each file cites
# its passage; the numbers were worked out by hand, not by the oracle).
# ---------------------------------------------------------------------------
GOLDEN = os.path.join(HERE, "golden")
GRID_NAMES = {"e1m2": O.E1M2, "int4": O.INT4, "e2m1": O.E2M1}


def _golden_rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def _golden_blocks(name):
    blocks, cur = {}, None
    with open(os.path.join(GOLDEN, name)) as f:
        for ln in f:
            if ln.startswith("# n="):
                cur = int(ln[4:])
                blocks[cur] = []
            elif ln.strip() and not ln.startswith("#"):
                blocks[cur].append([float(v) for v in ln.split()])
    return {n: np.array(m) for n, m in blocks.items()}


def test_golden_sylvester_matrices():
    """[UFP4] Method, Sylvester recursion from H_1 = [1]."""
    for n, m in _golden_blocks("sylvester_h4.txt").items():
        assert np.array_equal(O.fwht(np.eye(n, dtype=np.float64), n), m)


def test_golden_bin_bias():
    """[UFP4] Method, bin-asymmetry equation: the oracle's rounding, averaged
    over a locally uniform density in each bin, gives the worked values."""
    rows = _golden_rows("bin_bias.txt")
    by_grid = {}
    for g, q, b in rows:
        by_grid.setdefault(GRID_NAMES[g], []).append((float(q), float(b)))
    for grid, entries in by_grid.items():
        L = O.LEVELS[grid]
        assert len(entries) == L.size - 2          # every interior level listed
        got = _bin_bias(grid)
        for q, b in entries:
            assert abs(got[q] - b) <= 1e-5 * max(1.0, float(L[-1]))


def test_golden_pow2_scale_exponents():
    """[2DFP4] truncation-free scale equation, worked by hand."""
    for g, m, e in _golden_rows("pow2_scale.txt"):
        got = O.scale_pow2_exponent(np.array([float(m)], dtype=np.float32), GRID_NAMES[g])
        assert int(got[0]) == int(e), (g, m)


# ---------------------------------------------------------------------------
# Quantization diagnostics (level statistics).  [UFP4] Method: bin-asymmetry
# equation and bucket utilisation.
# ---------------------------------------------------------------------------
def _pow2_scale_blocks(grid, P, K, seed, j=0):
    """bf16 bits whose 1 x 16 blocks each hold q_max * 2^j as their largest
    magnitude, so s = 2^j exactly and t = y / 2^j."""
    rng = np.random.default_rng(seed)
    qmax = O.QMAX[grid]
    x = rng.uniform(-qmax, qmax, (P, K)) * 2.0 ** j
    x[:, ::16] = qmax * 2.0 ** j * np.where(rng.random((P, K // 16)) < 0.5, -1.0, 1.0)
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _brute_stats(bits, grid, rounding, j, spec):
    """Exact rationals: t = y / 2^j, level by exhaustive nearest search (ties
    to the even index) or k_lo + [r16 < f 2^16], error rounded half-even."""
    L = [Fraction(float(v)) for v in O.LEVELS[grid]]
    P, K = bits.shape
    y = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    r16 = O.sr_draws(spec.sr_seed, spec.sr_stream, np.arange(P * K, dtype=np.uint64)).reshape(P, K)
    cnt, tot = [0] * 8, [0] * 8
    for p in range(P):
        for k in range(K):
            t = abs(Fraction(float(y[p, k])) / Fraction(2) ** j)
            if rounding == O.RTNE:
                d = [abs(t - lv) for lv in L]
                best = min(d)
                cand = [i for i in range(8) if d[i] == best]
                idx = next((i for i in cand if i % 2 == 0), cand[0])
            else:
                lo = max(i for i in range(8) if L[i] <= t)
                if lo == 7:
                    idx = 7
                else:
                    f = (t - L[lo]) / (L[lo + 1] - L[lo])
                    idx = lo + (1 if int(r16[p, k]) < f * 65536 else 0)
            cnt[idx] += 1
            tot[idx] += round((L[idx] - t) * 2 ** 28)
    return np.array(cnt + tot, dtype=np.int64)


@pytest.mark.parametrize("grid", [O.E1M2, O.INT4, O.E2M1])
@pytest.mark.parametrize("rounding", [O.RTNE, O.SR])
def test_level_stats_brute_force(grid, rounding):
    spec = O.QuantSpec(grid, rounding, O.SCALE_F32, 1, 16, 1, 0, 4242, 3)
    for j in (0, -5):
        bits = _pow2_scale_blocks(grid, 6, 64, seed=11 + grid + 3 * rounding - j, j=j)
        q = O.quantize(bits, 0, spec)
        assert np.array_equal(O.level_stats(q, grid), _brute_stats(bits, grid, rounding, j, spec))


@pytest.mark.parametrize("grid", [O.E1M2, O.INT4, O.E2M1])
def test_level_stats_sr_unbiased(grid):
    """[2DFP4] SR equation E[roundS(x)] = x: the pooled error mean vanishes."""
    t = _tensor_bits(128, 1024, 9)
    st = O.level_stats(O.quantize(t, 0, O.QuantSpec(grid, O.SR, O.SCALE_F32, 1, 16, 16, 3, 77, 1)), grid)
    n = st[:8].sum()
    assert n == t.size
    gap = float(np.max(np.diff(O.LEVELS[grid])))
    mean = st[8:].sum() * 2.0 ** -28 / n
    assert abs(mean) < 5 * gap / np.sqrt(n)


def test_level_stats_match_bin_asymmetry_values():
    """RTNE on a uniform spread of t (s = 1 blocks): each interior level's
    mean error is the worked value of tests/golden/bin_bias.txt, up to the
    spacing h of the spread."""
    rows = _golden_rows("bin_bias.txt")
    for gname, grid in GRID_NAMES.items():
        qmax = O.QMAX[grid]
        h = 2.0 ** -7 if grid == O.E1M2 else 2.0 ** -5
        vals = np.arange(0.0, qmax, h)
        n_blk = -(-vals.size // 15)
        x = np.zeros((n_blk, 16))
        flat = np.concatenate([vals, np.zeros(n_blk * 15 - vals.size)])
        x[:, 1:] = flat.reshape(n_blk, 15)
        x[:, 0] = qmax                                  # block max: s = 1
        bits = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy(), x)
        st = O.level_stats(O.quantize(bits, 0, O.QuantSpec(grid, O.RTNE, O.SCALE_F32, 1, 16, 1)), grid)
        L = list(O.LEVELS[grid])
        for g, q, b in rows:
            if g != gname:
                continue
            i = L.index(float(q))
            mean = st[8 + i] * 2.0 ** -28 / st[i]
            assert abs(mean - float(b)) <= h, (gname, q, mean)


# ---------------------------------------------------------------------------
# MXFP8 (E4M3 elements, 1 x 32 power-of-two scales).  [2DFP4] mixed-precision
# section: Query/Key projections stay in MXFP8.  The format itself is pinned
# to torch's float8_e4m3fn (an independent implementation of OCP E4M3).
# ---------------------------------------------------------------------------
def test_e4m3_levels_are_torch_e4m3fn():
    codes = torch.arange(127, dtype=torch.uint8)
    want = codes.view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(O.LEVELS[O.E4M3], want)
    assert O.QMAX[O.E4M3] == 448.0


def test_e4m3_rtne_matches_torch_cast():
    rng = np.random.default_rng(12)
    v = np.concatenate([rng.uniform(-448, 448, 20000), rng.uniform(-0.02, 0.02, 20000),
                        [0.0, 448.0, -448.0, 1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10]])
    v = v.astype(np.float32)
    k = O.round_rtne_index(np.abs(v).astype(np.float64), O.E4M3)
    got = O.encode(k, v < 0, O.E4M3)
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    want = np.where(want == 0x80, 0, want)          # canonical zero (no -0)
    assert np.array_equal(got, want)


def test_mxfp8_quantize_dequant_bound():
    """Power-of-two 1 x 32 blocks: every |v| <= 448 and the dequantized value
    is within half an E4M3 spacing of y (relative 2^-4, or 2^-10 * 2^e in the
    subnormal range)."""
    t = _tensor_bits(64, 256, 21, scale=3.0)
    spec = O.QuantSpec(O.E4M3, O.RTNE, O.SCALE_POW2, 1, 32, 1)
    q = O.quantize(t, 0, spec)
    assert q["codes"].shape == (64, 256) and q["codes"].dtype == np.uint8
    e = q["scales"].astype(np.int64) - 127
    y = O.bf16_bits_to_f32(t).astype(np.float64)
    d = O.dequant(q["codes"], q["scales"], spec, 64, 256)[1]
    s = np.repeat(np.exp2(e.astype(np.float64)), 32, axis=1)
    bound = np.maximum(np.abs(y) * 2.0 ** -4, s * 2.0 ** -10)
    assert np.all(np.abs(d - y) <= bound)
    M = np.abs(y).reshape(64, 8, 32).max(axis=2)
    assert np.all(M <= 448.0 * np.exp2(e.astype(np.float64)))
    assert np.all((M == 0) | (M > 448.0 * np.exp2(e.astype(np.float64) - 1)) | (e == -127))


def test_mxfp8_lossless_on_grid():
    """Values already on the scaled E4M3 grid come back exactly."""
    rng = np.random.default_rng(5)
    L = O.LEVELS[O.E4M3]
    k = rng.integers(0, 127, (16, 64))
    k[:, ::32] = 126                                  # block max 448: e = 0
    sign = np.where(rng.random((16, 64)) < 0.5, -1.0, 1.0)
    y = (sign * L[k]).astype(np.float32)
    bits = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.bf16_bits_to_f32(bits), y)         # E4M3 values are bf16 values
    spec = O.QuantSpec(O.E4M3, O.RTNE, O.SCALE_POW2, 1, 32, 1)
    q = O.quantize(bits, 0, spec)
    assert np.all(q["scales"] == 127)
    assert np.array_equal(O.dequant(q["codes"], q["scales"], spec, 16, 64)[1], y.astype(np.float64))


# ---------------------------------------------------------------------------
# Two-level scaling ([UFP4] Method: the scaling hierarchy -- single-level,
# two-level or block -- is orthogonal to the format): a per-tensor fp32
# factor s_T over power-of-two block scales, an element standing for
# level * 2^e * s_T.
# ---------------------------------------------------------------------------
TWO_LEVEL_CASES = [(O.E1M2, 1, 32), (O.INT4, 1, 32), (O.E2M1, 32, 32), (O.E4M3, 1, 32)]


@pytest.mark.parametrize("grid,br,bc", TWO_LEVEL_CASES)
@pytest.mark.parametrize("j", [-3, 5])
def test_two_level_power_of_two_factor_shifts_exponents(grid, br, bc, j):
    """s_T = 2^j only moves every block exponent by -j: the codes and the
    dequantized values equal the single-level ones (a factor applied the
    wrong way round, or left out of the dequantization, changes them)."""
    t = _tensor_bits(64, 128, 21 + grid)
    n = 1 if br > 1 else 32
    one = O.QuantSpec(grid, O.RTNE, O.SCALE_POW2, br, bc, n, 3)
    two = O.QuantSpec(grid, O.RTNE, O.SCALE_POW2, br, bc, n, 3, tensor_scale=float(2.0 ** j))
    q1, q2 = O.quantize(t, 0, one), O.quantize(t, 0, two)
    assert np.array_equal(q1["codes"], q2["codes"])
    assert np.array_equal(q2["scales"].astype(np.int64), q1["scales"].astype(np.int64) - j)
    d1 = O.dequant(q1["codes"], q1["scales"], one, 64, 128)[1]
    d2 = O.dequant(q2["codes"], q2["scales"], two, 64, 128)[1]
    assert np.array_equal(d1, d2)
    unit = O.QuantSpec(grid, O.RTNE, O.SCALE_POW2, br, bc, n, 3, tensor_scale=1.0)
    qu = O.quantize(t, 0, unit)
    assert np.array_equal(qu["codes"], q1["codes"]) and np.array_equal(qu["scales"], q1["scales"])


@pytest.mark.parametrize("grid,br,bc", TWO_LEVEL_CASES)
@pytest.mark.parametrize("s_t", [0.7, 1.3, 3.0e-3])
def test_two_level_block_scale_brackets_and_error(grid, br, bc, s_t):
    """For any s_T the block scale is the least power-of-two multiple of s_T
    whose q_max multiple covers the block (up to the fp32 rounding of the
    normalization, 2^-23 relative), and every RTNE-dequantized element lies
    within half the widest level gap times that scale of its rotated value."""
    t = _tensor_bits(64, 128, 31 + grid)
    n = 1 if br > 1 else 32
    spec = O.QuantSpec(grid, O.RTNE, O.SCALE_POW2, br, bc, n, 9, tensor_scale=s_t)
    q = O.quantize(t, 0, spec)
    st = float(np.float32(s_t))
    d = O.dequant(q["codes"], q["scales"], spec, 64, 128)[1]
    s = O.scale_per_element(q["scales"], spec, 64, 128)          # 2^e * s_T
    y = q["rotated"].astype(np.float64)
    M = O.block_absmax(y.astype(np.float32), br, bc).astype(np.float64)
    S = s.reshape(64 // br, br, 128 // bc, bc)[:, 0, :, 0]
    qmax = O.QMAX[grid]
    tol = 2.0 ** -22
    assert np.all(M <= qmax * S * (1 + tol))                    # the scale covers the block
    assert np.all(qmax * S / 2 < M * (1 + tol))                 # and no smaller one would
    gap = np.max(np.diff(O.LEVELS[grid]))
    assert np.all(np.abs(d - y) <= 0.5 * gap * s * (1 + tol) + 1e-30)
    assert np.allclose(s / st, np.exp2(np.round(np.log2(s / st))), rtol=0, atol=0)
