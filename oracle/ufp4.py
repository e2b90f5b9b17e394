"""Plain CPU oracle of the UFP4 hot path: RHT, blockwise 4-bit quantization,
dequantization and the block-scaled 4-bit GEMMs.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).  Slow and literal on
purpose: every step follows the pages in their order, in numpy float32 where
the method computes in fp32 (numpy float32 arithmetic is IEEE round-to-nearest
-even with no fused multiply-add) and in float64 / exact rationals where a
decision must be exact.

Pages cited (by title, section, equation):
  [UFP4]  "Rethinking Shrinkage Bias in FP4 Pretraining of LLMs: Geometric
          Origin, Systemic Impact and the UFP4 Recipe" -- hyper.ai summary
          (sections: formats and blockwise quantization, Method, Experiments)
          and chatpaper abstract.
  [2DFP4] "Stable FP4 Training via Transposition-Invariant Block
          Quantization" -- agifrontier tutorial (sections: the root cause,
          2D square-block quantization).

Readings of steps the pages leave open are marked READING and listed in the
design notes; each one is a single deterministic choice, so exactly one bit
pattern is correct for every output.
"""
from dataclasses import dataclass
from fractions import Fraction

import numpy as np

from .philox import philox4x32_10, split_seed

# ---------------------------------------------------------------------------
# Codebooks.  [UFP4] formats section: each format defines a normalized
# codebook G with a fixed set of levels; the Method section contrasts the
# non-uniform E2M1 grid with the uniform E1M2 / INT4 grids.
# READING: E1M2 = {0, +-0.25, ..., +-1.75} (1 exponent bit, 2 mantissa bits,
# its levels are k/4), INT4 = {-7..7} (symmetric, -8 unused), E2M1 = the
# OCP-MX FP4 magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}.
# ---------------------------------------------------------------------------
E1M2, INT4, E2M1, E4M3 = 0, 1, 2, 3
RTNE, SR = 0, 1
SCALE_F32, SCALE_POW2 = 0, 1
SIGN_STREAM = 0xFFFFFFFF  # Philox counter word reserved for the sign draw

LEVELS = {
    E1M2: np.array([0.0, 0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75]),
    INT4: np.arange(8, dtype=np.float64),
    E2M1: np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]),
}


def _e4m3_magnitudes():
    """OCP FP8 E4M3 (the MXFP8 element format): bit pattern b = 8 e + m with
    e = 0 subnormal (m/8 * 2^-6), else (1 + m/8) * 2^(e - 7); pattern 0x7F is
    NaN, so 127 finite magnitudes, 0 .. 448, ascending in b."""
    out = []
    for b in range(127):
        e, m = b >> 3, b & 7
        out.append(m / 8.0 * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(out)


# [2DFP4] mixed-precision section: the Query/Key projections keep MXFP8 (E4M3
# elements, power-of-two scale per 1 x 32 block).  READING: the level set is
# every finite E4M3 magnitude and the scale follows the same truncation-free
# power-of-two rule with q_max = 448; ties go to the even pattern (IEEE RNE).
LEVELS[E4M3] = _e4m3_magnitudes()
QMAX = {g: float(LEVELS[g][-1]) for g in LEVELS}
SIGN_BIT = {E1M2: 8, INT4: 8, E2M1: 8, E4M3: 128}


@dataclass(frozen=True)
class QuantSpec:
    """Everything the pages make a parameter of one quantization."""
    grid: int = E1M2            # codebook G
    rounding: int = RTNE        # RTNE or SR
    scale_mode: int = SCALE_F32  # absmax/qmax in fp32, or power of two
    block_rows: int = 1         # 1 for 1 x b blocks, b for b x b blocks
    block_cols: int = 16        # block extent along K
    rht_n: int = 16             # Hadamard size; 1 disables the rotation
    sign_seed: int = 0
    sr_seed: int = 0
    sr_stream: int = 0
    tensor_scale: float = 0.0   # two-level scaling (power-of-two blocks only); 0: none


# ---------------------------------------------------------------------------
# bf16 decode: a bf16 value is the upper half of an fp32 word.
# ---------------------------------------------------------------------------
def bf16_bits_to_f32(bits):
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


# ---------------------------------------------------------------------------
# Random signs S_n = diag(eps).  [UFP4] Method: RHT multiplies by a random
# +-1 diagonal before the Hadamard matrix, H'_n = S_n H_n.
# READING: eps_i (i < n <= 128) is bit i of one Philox4x32-10 block with
# key = sign_seed and counter (0, 0, 0xFFFFFFFF, 0); bit 1 means -1.  The
# same S_n is used for every length-n chunk along K and by both operands of a
# GEMM, which is what makes the rotation cancel (Method, invariance equation).
# ---------------------------------------------------------------------------
def rht_signs(sign_seed, n):
    if n < 1 or n > 128 or (n & (n - 1)):
        raise ValueError("n must be a power of two in [1, 128]")
    words = philox4x32_10([[0, 0, SIGN_STREAM, 0]], split_seed(sign_seed))[0]
    idx = np.arange(n)
    bit = (words[idx >> 5].astype(np.uint64) >> (idx & 31).astype(np.uint64)) & np.uint64(1)
    return np.where(bit == 1, -1.0, 1.0)


def rht_norm_const(n):
    """c_n = fp32 nearest to n^(-1/2), found by exact rational comparison.

    [UFP4] Method, Sylvester recursion: every doubling multiplies by 1/sqrt(2),
    so H_n = n^(-1/2) * (+-1 Sylvester matrix).  READING: the fp32 path applies
    the whole factor as one final multiply by c_n.
    """
    cand = np.float32(1.0 / np.sqrt(np.float64(n)))
    options = [np.nextafter(cand, np.float32(0)), cand, np.nextafter(cand, np.float32(1))]
    # 1/sqrt(n) is irrational or exactly representable, so no ties occur;
    # |c^2 - 1/n| orders the neighbours the same way |c - n^-1/2| does.
    best = min(options, key=lambda c: abs(Fraction(float(c)) ** 2 - Fraction(1, n)))
    return np.float32(best)


def fwht(x, n):
    """Unnormalized Walsh-Hadamard transform of every length-n chunk of the
    last axis, computed in the dtype of x.

    [UFP4] Method, Sylvester recursion H_2n = [[H_n, H_n], [H_n, -H_n]] / sqrt 2.
    READING (fixed stage order): for h = 1, 2, 4, ..., n/2, each pair (i, i+h)
    with bit h of i clear becomes (x_i + x_{i+h}, x_i - x_{i+h}).  The result
    is x times the +-1 Sylvester matrix of order n.
    """
    x = np.array(x, copy=True)
    shape = x.shape
    if shape[-1] % n:
        raise ValueError("last axis must be a multiple of n")
    h = 1
    while h < n:
        v = x.reshape(-1, n // (2 * h), 2, h)
        lo = v[:, :, 0, :].copy()
        hi = v[:, :, 1, :].copy()
        v[:, :, 0, :] = lo + hi
        v[:, :, 1, :] = lo - hi
        x = v.reshape(shape)
        h *= 2
    return x


def rht(a, n, sign_seed):
    """y = RN(fwht(S_n a) * c_n) chunk by chunk along the last axis (fp32).

    [UFP4] Method: X H'_n with H'_n = S_n H_n, applied along the shared GEMM
    dimension K; READING: K > n uses the block-diagonal I (x) H'_n.
    """
    a = np.asarray(a, dtype=np.float32)
    if n == 1:
        return a.copy()
    eps = rht_signs(sign_seed, n).astype(np.float32)
    reps = a.shape[-1] // n
    x = a * np.tile(eps, reps)               # exact: multiply by +-1
    y = fwht(x, n)
    return (y * rht_norm_const(n)).astype(np.float32)


# ---------------------------------------------------------------------------
# Block partition and scales.
# [UFP4] formats section: contiguous blocks share one scale s_B = block absmax
# divided by the largest level of the codebook.  [2DFP4] root-cause section:
# 1 x 16 / 1 x 32 groups; 2D section: b x b square blocks and the
# truncation-free power-of-two scale S = 2^ceil(log2(2M / (Qp - Qn))).
# ---------------------------------------------------------------------------
def block_absmax(y, br, bc):
    P, K = y.shape
    if P % br or K % bc:
        raise ValueError("operand not divisible into blocks")
    v = np.abs(y.astype(np.float32)).reshape(P // br, br, K // bc, bc)
    return v.max(axis=(1, 3))                  # [P/br, K/bc] fp32


def scale_f32(M, grid):
    """s_B = RN_fp32(M_B / qmax); numpy float32 division is correctly rounded."""
    return (np.asarray(M, np.float32) / np.float32(QMAX[grid])).astype(np.float32)


def scale_pow2_exponent(M, grid):
    """Least integer e with M <= qmax * 2^e (= ceil(log2(2M/(Qp-Qn))) with
    Qp = -Qn = qmax), clamped to [-127, 127]; M = 0 gives -127 (READING).

    Decided exactly: qmax * 2^e and M are both exact in float64."""
    M = np.asarray(M, dtype=np.float64)
    q = QMAX[grid]
    with np.errstate(divide="ignore"):
        e = np.ceil(np.log2(np.where(M > 0, M / q, 1.0))).astype(np.int64)
    # correct the float64 estimate by exact comparisons
    for _ in range(3):
        e = np.where(M > q * np.exp2(e.astype(np.float64)), e + 1, e)
        e = np.where((M > 0) & (M <= q * np.exp2((e - 1).astype(np.float64))), e - 1, e)
    e = np.where(M > 0, e, -127)
    return np.clip(e, -127, 127)


def scale_pow2_exponent_exact(M, grid):
    """Same as scale_pow2_exponent, one block at a time with Fractions."""
    q = Fraction(QMAX[grid]).limit_denominator(8)
    out = []
    for m in np.asarray(M, dtype=np.float64).ravel():
        if m == 0:
            out.append(-127)
            continue
        fm = Fraction(float(m))
        e = 0
        while fm > q * Fraction(2) ** e:
            e += 1
        while fm <= q * Fraction(2) ** (e - 1):
            e -= 1
        out.append(max(-127, min(127, e)))
    return np.array(out, dtype=np.int64).reshape(np.shape(M))


# ---------------------------------------------------------------------------
# Stochastic-rounding draws.  READING: 16 random bits per element; element e
# (its row-major index in the logical P x K operand, plus elem_base) takes the
# 16-bit half (e & 1) of word ((e & 7) >> 1) of the Philox block with key =
# sr_seed and counter (low32(e >> 3), high32(e >> 3), sr_stream, 0).
# ---------------------------------------------------------------------------
def sr_draws(sr_seed, sr_stream, elem_idx):
    e = np.asarray(elem_idx, dtype=np.uint64).ravel()
    g = e >> np.uint64(3)
    uniq, inv = np.unique(g, return_inverse=True)
    ctr = np.zeros((uniq.size, 4), dtype=np.uint64)
    ctr[:, 0] = uniq & np.uint64(0xFFFFFFFF)
    ctr[:, 1] = uniq >> np.uint64(32)
    ctr[:, 2] = np.uint64(int(sr_stream) & 0xFFFFFFFF)
    blocks = philox4x32_10(ctr, split_seed(sr_seed))
    word = ((e & np.uint64(7)) >> np.uint64(1)).astype(np.int64)
    half = (e & np.uint64(1)).astype(np.uint32)
    w = blocks[inv, word]
    return ((w >> (np.uint32(16) * half)) & np.uint32(0xFFFF)).astype(np.uint16).reshape(np.shape(elem_idx))


# ---------------------------------------------------------------------------
# Rounding onto the codebook.  [UFP4] formats section: deterministic
# round-to-nearest-even, or stochastic rounding that picks a neighbouring
# level with probability proportional to the distance; [2DFP4] 2D section:
# SR is unbiased, E[roundS(x)] = x.
# READING: rounding acts on the magnitude m = |v|, the sign is put back
# afterwards; RTNE ties go to the level with even index (for E2M1 this is
# IEEE round-half-even on the 1-bit mantissa).
# ---------------------------------------------------------------------------
def round_rtne_index(m, grid):
    """Nearest level index, ties to the even index (by definition: argmin)."""
    L = LEVELS[grid]
    m = np.asarray(m, dtype=np.float64)
    d = np.abs(m[..., None] - L)              # exact in float64
    is_min = d == d.min(axis=-1, keepdims=True)
    # among the (at most two) nearest levels prefer the even index
    idx = np.arange(L.size)
    even_hit = is_min & (idx % 2 == 0)
    has_even = even_hit.any(axis=-1)
    first_even = np.argmax(even_hit, axis=-1)
    first_any = np.argmax(is_min, axis=-1)
    return np.where(has_even, first_even, first_any).astype(np.int64)


def round_sr_index(m, grid, r16):
    """k = k_lo + [r16 < f * 2^16], f = (m - L[k_lo]) / (L[k_lo+1] - L[k_lo])."""
    L = LEVELS[grid]
    m = np.asarray(m, dtype=np.float64)
    k_lo = np.searchsorted(L, m, side="right") - 1
    k_lo = np.clip(k_lo, 0, L.size - 1)
    top = k_lo == L.size - 1
    k_hi = np.minimum(k_lo + 1, L.size - 1)
    gap = np.where(top, 1.0, L[k_hi] - L[k_lo])
    f = np.where(top, 0.0, (m - L[k_lo]) / gap)    # exact: gaps are powers of two
    up = np.asarray(r16, dtype=np.float64) < f * 65536.0
    return (k_lo + up.astype(np.int64)).astype(np.int64)


# ---------------------------------------------------------------------------
# Encoding and packing.  READING: E1M2 and E2M1 nibbles are sign-magnitude
# (sign * 8 + level index; for E2M1 this is the OCP FP4 bit pattern), INT4 is
# the two's complement of +-k; zero is always code 0; byte j of a row holds
# the codes of elements 2j (low nibble) and 2j+1 (high nibble).
# ---------------------------------------------------------------------------
def encode(k, neg, grid):
    k = np.asarray(k, dtype=np.int64)
    neg = np.asarray(neg, dtype=bool) & (k > 0)
    if grid == INT4:
        return np.where(neg, (-k) & 0xF, k).astype(np.uint8)
    return (np.where(neg, SIGN_BIT[grid], 0) + k).astype(np.uint8)


def decode_index(code, grid):
    """Inverse of encode: (level index k, negative?)."""
    c = np.asarray(code, dtype=np.int64)
    if grid == INT4:
        sv = np.where(c >= 8, c - 16, c)
        return np.abs(sv), sv < 0
    sb = SIGN_BIT[grid]
    return c & (sb - 1), (c & sb) != 0


def code_bytes(code, grid):
    """Stored codes: 4-bit codes two per byte, E4M3 codes one per byte."""
    return np.asarray(code, dtype=np.uint8) if grid == E4M3 else pack_nibbles(code)


def code_values(codes, grid, P, K):
    """Inverse of code_bytes: the per-element codes [P, K]."""
    c = np.asarray(codes, dtype=np.uint8)
    return c.reshape(P, K) if grid == E4M3 else unpack_nibbles(c.reshape(P, K // 2))


def pack_nibbles(codes):
    c = np.asarray(codes, dtype=np.uint8)
    if c.shape[-1] % 2:
        raise ValueError("K must be even")
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


# ---------------------------------------------------------------------------
# The quantizer, step by step.
# ---------------------------------------------------------------------------
def _expand(blockwise, br, bc):
    return np.repeat(np.repeat(blockwise, br, axis=0), bc, axis=1)


def quantize(t_bits, along, spec, elem_base=0, row_index=None, col_index=None, K_total=None):
    """Quantize a bf16 tensor given as uint16 bits [R, C].

    along = 0: the logical operand is A = T (K = C); along = 1: A = T^T (K = R).
    row_index / col_index / K_total (optional): position of the given rows
    and columns inside a larger logical operand with K_total columns, used
    only to index the stochastic-rounding draws (lets a caller quantize a
    sample of a large operand; blocks and rotation chunks must lie inside
    the sample).  Returns a dict with 'rotated' fp32 [P, K],
    'codes' uint8 [P, K/2], 'scales' (fp32 [P, K/bc] or uint8 [P/br, K/bc] as
    E8M0 = e + 127), the unpacked 'code' nibbles, the clamped normalized
    values 'v' the rounding acts on and the chosen level indices 'k'.
    """
    t = np.asarray(t_bits, dtype=np.uint16)
    A = t.T if along == 1 else t
    P, K = A.shape
    n, br, bc = spec.rht_n, spec.block_rows, spec.block_cols
    if K % n or K % bc or P % br:
        raise ValueError("shape not divisible by rht_n / block")
    grid = spec.grid
    qmax = np.float32(QMAX[grid])

    # a1: bf16 -> fp32 (exact)
    a = bf16_bits_to_f32(A)
    # a2-a3: signs, Hadamard, normalization
    y = rht(a, n, spec.sign_seed)
    # a4: block absmax
    M = block_absmax(y, br, bc)
    # a5: scale
    if spec.scale_mode == SCALE_F32:
        s_blk = scale_f32(M, grid)
        scales = s_blk
        s_full = _expand(s_blk, br, bc)
        # a6: v = RN(y / s_B), clamped to +-qmax (RN may overshoot by one ulp);
        # a zero scale gives v = 0 (READING)
        with np.errstate(divide="ignore", invalid="ignore"):
            v = (y / np.where(s_full == 0, np.float32(1), s_full)).astype(np.float32)
        v = np.where(s_full == 0, np.float32(0), v)
    else:
        # Two-level scaling ([UFP4] Method: the scaling hierarchy -- single,
        # two-level or block -- is orthogonal to the format).  READING: a
        # per-tensor fp32 factor s_T > 0 over the power-of-two block scales:
        # the rotated values are first multiplied by m_T = RN_fp32(1 / s_T),
        # u = RN_fp32(y * m_T), and u is quantized with power-of-two block
        # scales as above; an element stands for level * 2^e * s_T.
        u = y
        if spec.tensor_scale:
            m_t = np.float32(1.0) / np.float32(spec.tensor_scale)
            u = (y.astype(np.float64) * np.float64(m_t)).astype(np.float32)
            M = block_absmax(u, br, bc)
        e_blk = scale_pow2_exponent(M, grid)
        scales = (e_blk + 127).astype(np.uint8)
        s_full = _expand(np.exp2(e_blk.astype(np.float64)).astype(np.float32), br, bc)
        v = (u / s_full).astype(np.float32)      # power-of-two divisor
    v = np.minimum(np.maximum(v, -qmax), qmax)

    m = np.abs(v).astype(np.float64)
    neg = v < 0
    if spec.rounding == RTNE:
        k = round_rtne_index(m, grid)
    else:
        rows = np.arange(P, dtype=np.int64) if row_index is None else np.asarray(row_index, np.int64)
        cols = np.arange(K, dtype=np.int64) if col_index is None else np.asarray(col_index, np.int64)
        kt = K if K_total is None else int(K_total)
        e_idx = int(elem_base) + rows[:, None] * kt + cols[None, :]
        r16 = sr_draws(spec.sr_seed, spec.sr_stream, e_idx)
        k = round_sr_index(m, grid, r16)
    code = encode(k, neg, grid)
    return {"rotated": y, "code": code, "codes": code_bytes(code, grid), "scales": scales,
            "P": P, "K": K, "v": v, "k": k}


def quantize_segmented(t_bits, offsets, spec):
    """Column-wise quantization of row segments of T [R, C]: segment g is
    rows [o_g, o_{g+1}) and yields the logical operand T[o_g:o_{g+1}]^T of
    shape [C, L_g].  Draw indices continue across segments: segment g starts
    at element C * o_g.  Used for the per-expert transposed operands."""
    out = []
    for g in range(len(offsets) - 1):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        out.append(quantize(np.asarray(t_bits)[lo:hi], 1, spec,
                            elem_base=np.asarray(t_bits).shape[1] * lo))
    return out


# ---------------------------------------------------------------------------
# Quantization diagnostics.  [UFP4] Method, Shrinkage Bias: for a level q_i
# the mean rounding error over its bin, E[rho(t) - t | t in B_i], is what the
# bin-asymmetry equation predicts; the Method section also speaks of the
# bucket utilisation the RHT improves.  READING: per magnitude level index k,
# count the elements rounded to level k and sum rint((L_k - |t|) * 2^28) over
# them (t = the clamped normalized value, magnitudes so both signs pool;
# integer units of 2^-28 make the sum exact and order-free).
# ---------------------------------------------------------------------------
def level_stats(q, grid):
    """q: a quantize() result.  Returns int64 [16]: counts [0:8], error sums
    in units of 2^-28 [8:16]."""
    k = np.asarray(q["k"], dtype=np.int64).reshape(-1)
    t = np.abs(np.asarray(q["v"], dtype=np.float32).astype(np.float64)).reshape(-1)
    err = LEVELS[grid][k] - t                    # exact in float64
    efx = np.rint(err * 2.0 ** 28).astype(np.int64)
    out = np.zeros(16, dtype=np.int64)
    out[:8] = np.bincount(k, minlength=8)
    for lev in range(8):
        out[8 + lev] = int(efx[k == lev].sum())
    return out


# ---------------------------------------------------------------------------
# Dequantization.  [UFP4] formats section: Q_G(T) denotes the dequantized
# tensor (level times block scale), in the rotated basis.
# ---------------------------------------------------------------------------
def level_values(code, grid):
    k, neg = decode_index(code, grid)
    lv = LEVELS[grid][k]
    return np.where(neg, -lv, lv)


def scale_per_element(scales, spec, P, K):
    br, bc = spec.block_rows, spec.block_cols
    if spec.scale_mode == SCALE_F32:
        s = np.asarray(scales, dtype=np.float32).reshape(P // br, K // bc)
        return _expand(s, br, bc).astype(np.float64)
    e = np.asarray(scales, dtype=np.int64).reshape(P // br, K // bc) - 127
    s = _expand(np.exp2(e.astype(np.float64)), br, bc)
    if spec.tensor_scale:                        # two-level: 2^e * s_T, exact in float64
        s = s * np.float64(np.float32(spec.tensor_scale))
    return s


def dequant(codes_packed, scales, spec, P, K):
    """Returns (fp32 RN(level * s), exact float64 level * s)."""
    code = code_values(codes_packed, spec.grid, P, K)
    lv = level_values(code, spec.grid)                       # exact
    s = scale_per_element(scales, spec, P, K)               # exact fp32 values
    exact = lv * s                                          # <= 27 significant bits
    return exact.astype(np.float32), exact


# ---------------------------------------------------------------------------
# GEMMs.  [UFP4] Method: Y^ = Q_G(X H') Q_G(W H')^T; the rotation cancels on
# the shared dimension, so every GEMM contracts the two dequantized rotated
# operands over K.  [2DFP4] root cause: dX = dY W and dW = dY^T X.
# All three are C[p, q] = sum_k A[p, k] B[q, k] (fp64 here).
# ---------------------------------------------------------------------------
def gemm_ref(DA, DB):
    return np.asarray(DA, np.float64) @ np.asarray(DB, np.float64).T


def rel_fro(c, ref):
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(np.asarray(c, np.float64) - ref) / (den if den > 0 else 1.0))
