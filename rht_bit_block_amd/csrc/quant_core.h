// Fused random Hadamard transform + blockwise 4-bit quantizer for gfx950:
// kernels and per-grid launchers (included by quant_e1m2.hip, quant_int4.hip,
// quant_e2m1.hip, one translation unit per codebook so they build in
// parallel).
//
// [UFP4] = "Rethinking Shrinkage Bias in FP4 Pretraining of LLMs ... the UFP4
// Recipe" (hyper.ai summary: formats and blockwise quantization; Method).
// [2DFP4] = "Stable FP4 Training via Transposition-Invariant Block
// Quantization" (agifrontier tutorial: 2D square-block quantization).
//
// Every lane owns W consecutive elements of one row of the logical operand
// A (P x K, K = the GEMM's shared dimension) and runs the whole pipeline on
// them in registers:
//   bf16 -> fp32, random signs S_n (sign-bit XOR on packed bf16 pairs),
//   Walsh-Hadamard butterflies h = 1, 2, ..., n/2 (in-lane for h < W, across
//   lanes with DPP quad permutes for h >= W), one multiply by c_n = RN(n^-1/2),
//   block absmax, scale, RN(y / s) (Markstein's reciprocal correction,
//   falling back to IEEE division when its preconditions fail), RTNE or
//   stochastic rounding (Philox4x32-10 keyed by the element index), nibble
//   encoding, packing, 8/16-byte stores.  E2M1 round-to-nearest and E4M3
//   (MXFP8) codes come from gfx950's FP4 / FP8 conversion instructions,
//   whose rounding is the codebooks' (negative zero cleared afterwards).
// For n = 4^j, c_n is a power of two: multiplying by it commutes exactly with
// the absmax, the scale and the quotient, so it is folded into the stored
// scale (blocks so small that the fold could underflow take the literal path).
// Row-wise calls read A straight from HBM; column-wise calls (A = X^T) stage
// a 128 x 64 tile of X through LDS and read it down the columns.
// All fp32 arithmetic that decides an output bit is explicit RN (no
// contraction; the library is built with -ffp-contract=off).
#pragma once

#include <atomic>

#include "ufp4_internal.h"

namespace ufp4 {
namespace qk {

constexpr int kThreads = 256;

template <int GRID> struct Grid;
template <> struct Grid<0> { static constexpr float qmax = 1.75f, inv_delta = 4.0f; };  // E1M2
template <> struct Grid<1> { static constexpr float qmax = 7.0f, inv_delta = 1.0f; };   // INT4
template <> struct Grid<2> { static constexpr float qmax = 6.0f, inv_delta = 0.0f; };   // E2M1
// MXFP8: OCP E4M3 elements (one byte per code), 1 x 32 power-of-two scales only
template <> struct Grid<3> { static constexpr float qmax = 448.0f, inv_delta = 0.0f; };

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (read once: non-temporal hint).
__device__ __forceinline__ uint4 ld16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint32_t fdiv_u32(uint32_t n, FastDiv f) {
  const uint64_t t = (uint64_t)__umulhi(n, f.m) + n;
  return (uint32_t)(t >> f.l);
}

// Per-pair sign masks: bit 15 flips the low bf16 of a packed pair, bit 31 the
// high one.  Bit j of `pat` is the sign of element j of the lane's segment.
template <int W>
__device__ __forceinline__ void sign_masks(uint32_t pat, uint32_t (&pm)[W / 2]) {
#pragma unroll
  for (int i = 0; i < W / 2; ++i) {
    const uint32_t lo = (pat >> (2 * i)) & 1u;
    const uint32_t hi = (pat >> (2 * i + 1)) & 1u;
    pm[i] = (lo << 15) | (hi << 31);
  }
}

// Sign pattern of the lane's segment: word qpos of the n-bit sign vector when a
// chunk spans several lanes, else the pattern repeated with period n (host).
template <class Q>
__device__ __forceinline__ uint32_t select_pattern(const Q& q, uint32_t qpos) {
  const uint32_t a = (qpos & 1u) ? q.sign_pat[1] : q.sign_pat[0];
  const uint32_t b = (qpos & 1u) ? q.sign_pat[3] : q.sign_pat[2];
  return (qpos & 2u) ? b : a;
}

// bf16 pairs (already sign-flipped) -> fp32.
template <int W>
__device__ __forceinline__ void unpack(const uint32_t (&w)[W / 2], const uint32_t (&pm)[W / 2],
                                       float (&y)[W]) {
#pragma unroll
  for (int i = 0; i < W / 2; ++i) {
    const uint32_t v = w[i] ^ pm[i];
    y[2 * i] = __uint_as_float(v << 16);
    y[2 * i + 1] = __uint_as_float(v & 0xFFFF0000u);
  }
}

// Compile-time facts about the Hadamard size n.
template <int N> struct Rht {
  static constexpr bool fold = (N == 4 || N == 16 || N == 64);   // c_n = 2^-k exactly
  static constexpr float c = N == 4 ? 0.5f : (N == 16 ? 0.25f : (N == 64 ? 0.125f : 1.0f));
};

// In-lane butterflies h = 1, 2, ..., min(n, W)/2 (fixed stage order).
template <int W, int N>
__device__ __forceinline__ void fwht_inlane(float (&y)[W]) {
#pragma unroll
  for (int h = 1; h < (N < W ? N : W); h <<= 1) {
#pragma unroll
    for (int i = 0; i < W; ++i) {
      if ((i & h) == 0) {
        const float a = y[i], b = y[i + h];
        y[i] = __fadd_rn(a, b);
        y[i + h] = __fsub_rn(a, b);
      }
    }
  }
}

// One butterfly stage between lanes L and L ^ m (m = 1 or 2) for every
// element: the lane with the bit clear keeps a + b, the other b - a, where
// a is its own value and b the partner's.  Computed as b + (+-a) so both
// lanes run the same instruction (IEEE: x - y == x + (-y), and a + b == b + a).
// Three instructions per element (DPP move, sign, add); exact in every bit,
// used when the rotated values are written out.
template <int W, int CTRL>
__device__ __forceinline__ void fwht_xlane_exact(float (&y)[W], uint32_t negmask) {
#pragma unroll
  for (int i = 0; i < W; ++i) {
    const float b = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(y[i]), CTRL, 0xF, 0xF, false));
    const float a = __uint_as_float(__float_as_uint(y[i]) ^ negmask);
    y[i] = __fadd_rn(b, a);
  }
}

// The same stage in one v_fmac_f32_dpp per element: y = y[L ^ m] * sgn + y,
// with sgn = +1 in the lane with the bit clear and -1 in the other.  The
// first lane gets a + b, the second -(b - a): the stage's result negated
// (an fma with a factor +-1 rounds once, as the add; x - y == -(y - x) for
// x != y).  If both lanes held their values negated, both results come out
// negated too.  Only the sign of an exact zero can differ from the negated
// result (a - a is +0 in either order), and no quotient, scale or code
// depends on it.  The compiler does not fold a DPP move into an fma, so the
// instruction is written out: sixteen elements per block, behind the two
// wait states a DPP read needs after a VALU write of its source.
#define UFP4_DPP_FMAC(i, ctrl) "v_fmac_f32_dpp %" #i ", %" #i ", %16 " ctrl " row_mask:0xf bank_mask:0xf\n\t"
#define UFP4_DPP_FMAC16(ctrl)                                                               \
  "s_nop 1\n\t" UFP4_DPP_FMAC(0, ctrl) UFP4_DPP_FMAC(1, ctrl) UFP4_DPP_FMAC(2, ctrl)     \
      UFP4_DPP_FMAC(3, ctrl) UFP4_DPP_FMAC(4, ctrl) UFP4_DPP_FMAC(5, ctrl)                \
          UFP4_DPP_FMAC(6, ctrl) UFP4_DPP_FMAC(7, ctrl) UFP4_DPP_FMAC(8, ctrl)            \
              UFP4_DPP_FMAC(9, ctrl) UFP4_DPP_FMAC(10, ctrl) UFP4_DPP_FMAC(11, ctrl)      \
                  UFP4_DPP_FMAC(12, ctrl) UFP4_DPP_FMAC(13, ctrl) UFP4_DPP_FMAC(14, ctrl) \
                      UFP4_DPP_FMAC(15, ctrl)
template <int W, int M>
__device__ __forceinline__ void fwht_xlane(float (&y)[W], uint32_t negmask) {
  static_assert(W % 16 == 0 && (M == 1 || M == 2), "16-element blocks; partner lane ^ 1 or ^ 2");
  const float sgn = __uint_as_float(0x3F800000u | negmask);
#pragma unroll
  for (int b = 0; b < W; b += 16) {
#define UFP4_DPP_OPS                                                                       \
  : "+v"(y[b]), "+v"(y[b + 1]), "+v"(y[b + 2]), "+v"(y[b + 3]), "+v"(y[b + 4]),            \
    "+v"(y[b + 5]), "+v"(y[b + 6]), "+v"(y[b + 7]), "+v"(y[b + 8]), "+v"(y[b + 9]),        \
    "+v"(y[b + 10]), "+v"(y[b + 11]), "+v"(y[b + 12]), "+v"(y[b + 13]), "+v"(y[b + 14]),   \
    "+v"(y[b + 15])                                                                        \
  : "v"(sgn)
    if constexpr (M == 1)
      asm(UFP4_DPP_FMAC16("quad_perm:[1,0,3,2]") UFP4_DPP_OPS);
    else
      asm(UFP4_DPP_FMAC16("quad_perm:[2,3,0,1]") UFP4_DPP_OPS);
#undef UFP4_DPP_OPS
  }
}
#undef UFP4_DPP_FMAC16
#undef UFP4_DPP_FMAC

// Runs f with the butterfly variant as a compile-time constant: exact (the
// rotated values are written out) or fused.  Taken once around a loop, so the
// loop body holds one variant and no merge of the two variants' registers.
template <bool V> struct ExactTag { static constexpr bool value = V; };
template <typename F>
__device__ __forceinline__ void with_exact(bool exact, F&& f) {
  if (exact)
    f(ExactTag<true>{});
  else
    f(ExactTag<false>{});
}

// All butterfly stages of n (lanes of a chunk are adjacent: n / W of them).
// Returns the lane's sign state: 0x80000000 if its values come out negated
// (an odd number of fused cross-lane stages in which its bit was set), else
// 0.  `exact` (uniform across the launch: the rotated values are written
// out) takes the three-instruction stages, whose results are the rotated
// values in every bit, zero signs included (sign state 0).
template <int W, int N>
__device__ __forceinline__ uint32_t fwht(float (&y)[W], uint32_t neg1, uint32_t neg2,
                                         bool exact) {
  fwht_inlane<W, N>(y);
  uint32_t sig = 0u;
  if constexpr (N >= 2 * W) {
    if (exact) {
      fwht_xlane_exact<W, 0xB1>(y, neg1);                             // lane ^ 1
      if constexpr (N >= 4 * W) fwht_xlane_exact<W, 0x4E>(y, neg2);   // lane ^ 2
      return 0u;
    }
    fwht_xlane<W, 1>(y, neg1);
    sig ^= neg1;
    if constexpr (N >= 4 * W) {
      fwht_xlane<W, 2>(y, neg2);
      sig ^= neg2;
    }
  }
  return sig;
}

template <int W>
__device__ __forceinline__ void scale_by(float (&y)[W], float c) {
#pragma unroll
  for (int i = 0; i < W; ++i) y[i] = __fmul_rn(y[i], c);
}

// ---------------------------------------------------------------------------
// Rounding and encoding.  Every path first produces the signed level index k
// (level = k * spacing unit) inside a "magic" float: for an integer-valued or
// rounding fp32 x with |x| < 2^22, RN(x + 1.5 * 2^23 + 8) = 1.5 * 2^23 + 8 +
// rint(x) (ties to even: the offset is even), so for k in [-8, 7] the float's
// bits are 0x4B400000 + (k + 8) -- a constant upper part and the offset-binary
// nibble k + 8 (one rounding, exact).  Eight such words are packed with one
// shift-add each: sum_j word_j << 4j = sum_j 0x4B400000 << 4j + sum_j
// (k_j + 8) << 4j (mod 2^32, no carries between nibbles), so subtracting the
// constant part leaves the offset-binary nibbles.  INT4 codes are their two's-
// complement form (bit 3 flipped); E1M2 / E2M1 codes are sign-magnitude,
// obtained for eight packed nibbles at once (ob_to_sm).
// ---------------------------------------------------------------------------
constexpr float kMagic = 12582912.0f;    // 1.5 * 2^23
constexpr float kMagicOB = 12582920.0f;  // 1.5 * 2^23 + 8
constexpr uint32_t kMagicHi = 0x4B400000u;
constexpr uint32_t kPackBias = kMagicHi + (kMagicHi << 4) + (kMagicHi << 8) + (kMagicHi << 12) +
                               (kMagicHi << 16) + (kMagicHi << 20) + (kMagicHi << 24) +
                               (kMagicHi << 28);

// Two's-complement nibble of a magic word.
__device__ __forceinline__ uint32_t word_nibble(uint32_t f) { return (f & 15u) ^ 8u; }

// Sum of word_j << 4j over a lane's eight elements -> offset-binary nibbles k + 8.
__device__ __forceinline__ uint32_t unbias_words(uint32_t acc) { return acc - kPackBias; }

// Offset-binary nibbles k + 8, k in [-7, 7] -> sign-magnitude (8 | |k| for
// k < 0; zero stays 0).  Per nibble o: k >= 0 iff bit 3, then the code is
// o ^ 8; else it is 16 - o = (o ^ 15) + 1.  t holds 8 in the negative
// nibbles, t - (t >> 3) holds 7 there (no borrows), t >> 3 the +1.
__device__ __forceinline__ uint32_t ob_to_sm(uint32_t o) {
  const uint32_t t = ~o & 0x88888888u;
  const uint32_t one = t >> 3;
  return (o ^ 0x88888888u ^ (t - one)) + one;
}

// E2M1 codes from the hardware FP4 conversion, which rounds to nearest even
// exactly as the E2M1 codebook does (levels 0, 0.5, .. 6 are the FP4 values,
// the even index is the even mantissa; saturating at 6) but keeps the sign
// of a value that rounds to zero.  Codes of magnitude 0 lose their sign bit.
__device__ __forceinline__ uint32_t fp4_clear_negzero(uint32_t w) {
  const uint32_t m = w & 0x77777777u;
  return m | (w & ((m + 0x77777777u) & 0x88888888u));
}

// Codes of (a, b) into byte sel of w (a in the low nibble); sel is a constant
// once the caller's loops are unrolled.
__device__ __forceinline__ uint32_t fp4_pair(uint32_t w, float a, float b, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a, b, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a, b, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a, b, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a, b, 1.0f, 3);
  }
}

// E4M3 bytes of (a, b) into half hi of w from the hardware FP8 conversion
// (scale 1), which rounds to nearest even onto the OCP E4M3 values exactly as
// the codebook rounding does, but keeps the sign of a value that rounds to
// zero; e4m3_clear_negzero drops it.
typedef short short2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t fp8_pair(uint32_t w, float a, float b, int hi) {
  const short2_t o = __builtin_bit_cast(short2_t, w);
  return __builtin_bit_cast(uint32_t, hi ? __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, a, b, 1.0f, true)
                                         : __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, a, b, 1.0f, false));
}
__device__ __forceinline__ uint32_t e4m3_clear_negzero(uint32_t w) {
  const uint32_t m = w & 0x7F7F7F7Fu;
  return m | (w & ((m + 0x7F7F7F7Fu) & 0x80808080u));
}

// RTNE: magic word of k = rint(v / spacing) for the uniform grids (|v| <= qmax,
// or one ulp above, which rounds to the same k); E2M1 by magnitude region.
template <int GRID>
__device__ __forceinline__ uint32_t rtne_word(float v) {
  if constexpr (GRID != 2) {
    return __float_as_uint(__fmaf_rn(v, Grid<GRID>::inv_delta, kMagicOB));
  } else {
    // spacing 0.5 below 2, 1 below 4, 2 above; index = rint(m/spacing) + add
    const float m = fabsf(v);
    const float mul = m < 2.0f ? 2.0f : (m < 4.0f ? 1.0f : 0.5f);
    const float add = m < 2.0f ? 0.0f : (m < 4.0f ? 2.0f : 4.0f);
    const float k = (__fmaf_rn(m, mul, kMagic) - kMagic) + add;   // exact integers
    return __float_as_uint(copysignf(k, v) + kMagicOB);
  }
}

// SR: k = k_lo + [r16 < f 2^16] on the magnitude, sign restored; magic word of k.
// With t = |v| / spacing (exact) and u = r16 2^-16, k_lo + [f > u] =
// ceil(t - u).  The fma below rounds t - u once: it is exact for t >= 1/2
// (t < 8 and u on a 2^-16 grid fit 24 bits at t's ulp), and for smaller t
// the result lies in (-1, 1/2), where rounding keeps its sign, keeps it
// nonzero and keeps it above -1 (-1 + 2^-16 is a float), so the ceiling is
// unchanged.
template <int GRID>
__device__ __forceinline__ uint32_t sr_word(float v, uint32_t r16) {
  const float m = fabsf(v);
  float mul = Grid<GRID>::inv_delta, add = 0.0f;
  if constexpr (GRID == 2) {
    mul = m < 2.0f ? 2.0f : (m < 4.0f ? 1.0f : 0.5f);
    add = m < 2.0f ? 0.0f : (m < 4.0f ? 2.0f : 4.0f);
  }
  const float t = m * mul;                        // exact
  float k = ceilf(__fmaf_rn((float)r16, -0x1p-16f, t));
  if constexpr (GRID == 2) k += add;
  return __float_as_uint(copysignf(k, v) + kMagicOB);
}

// Eight offset-binary nibbles (element j at bits 4j) -> final codes: INT4
// two's complement, E1M2 / E2M1 sign-magnitude.
template <int GRID>
__device__ __forceinline__ uint32_t finish_codes(uint32_t o) {
  return GRID == 1 ? (o ^ 0x88888888u) : ob_to_sm(o);
}

// 16-bit draws of the W elements starting at element index e0 (e0 % 8 == 0).
template <int W>
__device__ __forceinline__ void sr_draws(uint64_t e0, uint64_t seed, uint32_t stream,
                                         uint32_t (&words)[W / 2]) {
#pragma unroll
  for (int t = 0; t < W / 8; ++t) {
    const uint64_t g = (e0 >> 3) + (uint64_t)t;
    uint32_t c[4] = {(uint32_t)g, (uint32_t)(g >> 32), stream, 0u};
    philox4x32_10_dev(c, (uint32_t)seed, (uint32_t)(seed >> 32));
#pragma unroll
    for (int i = 0; i < 4; ++i) words[4 * t + i] = c[i];
  }
}

// Least e in [-127, 127] with M <= qmax * 2^e ([2DFP4] power-of-two scale
// equation; the clamp is the E8M0 range).  M = 0 gives -127.
template <int GRID>
__device__ __forceinline__ int pow2_exponent(float M) {
  constexpr float qmax = Grid<GRID>::qmax;
  int e = -127;
  if (M > 0.0f) {
    // qmax < 2^QE, so M > qmax * 2^(ilogb(M) - QE)
    constexpr int QE = GRID == 3 ? 9 : 3;
    e = ilogbf(M) - QE;
    if (e < -127) e = -127;
    while (e < 127 && M > ldexpf(qmax, e)) ++e;
  }
  return e;
}

// Byte offset of element e0's code: 4-bit codes two per byte, E4M3 one.
template <int GRID>
__device__ __forceinline__ uint8_t* code_ptr(uint8_t* base, uint64_t e0) {
  return base + (GRID == 3 ? e0 : (e0 >> 1));
}

// Quantize the W values of one lane whose blocks are 1 x B; writes codes
// (W/2 bytes) and W/B scales.  RND bit 0: stochastic rounding; RND bit 1:
// power-of-two scales stored as E8M0 bytes (1 x 32 blocks), else fp32
// absmax scales.  With power-of-two scales c is the two-level multiplier
// m_T = RN(1 / s_T) (1 for single-level scaling).  FOLD (fp32 scales only): y holds the
// unnormalized transform x, the rotated values are c * x with c a power of
// two, and RN(c x / s_c) = RN(x / s_x), s_c = c s_x whenever nothing
// underflows; blocks with c * absmax < 2^-100 redo the literal computation.
// Per-thread level statistics of the diagnostics kernel, in LDS: for every
// magnitude level index k, the number of elements rounded to level k and the
// sum over them of rint((L_k - |t|) * 2^28), t the clamped normalized value
// the rounding acts on ([UFP4] Method, bin-asymmetry equation: the mean of
// rho(t) - t per bin; integer sums, so the totals do not depend on order).
struct DiagLds {
  uint32_t cnt[8][kThreads];
  long long sum[8][kThreads];
};

// Magnitude of level index k (0..7) in grid units.
template <int GRID>
__device__ __forceinline__ float level_magnitude(int k) {
  if constexpr (GRID == 0) return 0.25f * (float)k;
  else if constexpr (GRID == 1) return (float)k;
  else return k < 4 ? 0.5f * (float)k : (float)((2 + (k & 1)) << ((k >> 1) - 2));
}

template <int GRID>
__device__ __forceinline__ void diag_accumulate(DiagLds* d, uint32_t nib, float t) {
  const int sk = ((int)(nib << 28)) >> 28;   // signed level index, in [-7, 7]
  const int k = (sk < 0 ? -sk : sk) & 7;     // (the mask only bounds the LDS index)
  const double err = (double)level_magnitude<GRID>(k) - (double)fabsf(t);   // exact
  const int efx = (int)rint(err * 268435456.0);                             // |err| <= 2
  const int tid = threadIdx.x;
  // LDS atomic adds on the thread's own column: no contention, and unlike a
  // read-modify-write they do not serialize consecutive elements of a lane
  // on the LDS latency
  atomicAdd(&d->cnt[k][tid], 1u);
  atomicAdd(reinterpret_cast<unsigned long long*>(&d->sum[k][tid]),
            (unsigned long long)(long long)efx);
}

// `sig` is the lane's sign state from fwht: when set, y holds the negated
// rotated values, and the quotients use the negated divisor (or reciprocal),
// which gives the same RN(y / s): rounding is symmetric.
// s = RN(M / qmax) for the codebook's constant qmax (1.75, 7 or 6): the
// product M * RN(1/qmax) corrected once through its exact fma remainder
// (Markstein's division by a known divisor).  It equals the IEEE quotient for
// every float M in [1, 4) for each of the three divisors (an exhaustive host
// check in the tests); the sequence and the quotient both scale exactly with
// M by powers of two while the remainder stays normal, so this holds for every
// M in [2^-100, FLT_MAX] and for M = 0.  Other M (tiny, inf, NaN) divide.
template <int GRID>
__device__ __forceinline__ float div_qmax(float M) {
  constexpr float qmax = Grid<GRID>::qmax, rq = 1.0f / qmax;
  if (__builtin_expect(!((M >= 0x1p-100f || M == 0.0f) && M <= 0x1.fffffep127f), 0))
    return __fdiv_rn(M, qmax);
  const float q0 = __fmul_rn(M, rq);
  return __fmaf_rn(__fmaf_rn(-q0, qmax, M), rq, q0);
}

template <int W, int B, int GRID, int RND, bool FOLD, bool DIAG = false>
__device__ __forceinline__ void quantize_1d(const float (&y)[W], uint32_t sig, float c, uint64_t e0,
                                            uint64_t seed, uint32_t stream, uint8_t* codes_out,
                                            void* scales_out, DiagLds* diag = nullptr) {
  constexpr float qmax = Grid<GRID>::qmax;
  constexpr int RM = RND & 1;
  constexpr bool POW2 = (RND & 2) != 0;
  static_assert(!(POW2 && FOLD), "power-of-two scales take the normalized values");
  uint32_t rw[W / 2];
  if constexpr (RM == 1) sr_draws<W>(e0, seed, stream, rw);
  uint32_t packed[W / 8];   // sums of magic words (shift-added), see unbias_words
#pragma unroll
  for (int i = 0; i < W / 8; ++i) packed[i] = 0u;
  // E2M1 RTNE: two elements per hardware FP4 conversion (scale 1: v is
  // already in grid units), codes written into byte (idx & 7) / 2 of the word
  constexpr bool kHwFp4 = GRID == 2 && RM == 0 && !DIAG;
  uint32_t bytes[GRID == 3 ? W / 4 : 1];   // E4M3 codes, four per word
#pragma unroll
  for (int i = 0; i < (GRID == 3 ? W / 4 : 1); ++i) bytes[i] = 0u;
#pragma unroll
  for (int blk = 0; blk < W / B; ++blk) {
    float M = 0.0f;
#pragma unroll
    for (int j = 0; j < B; ++j) M = fmaxf(M, fabsf(y[blk * B + j]));
    float v[B];
    if constexpr (POW2) {
      // two-level scaling: c = m_T, the values are u = RN(y m_T) and
      // max |u| = RN(M m_T) since rounding is monotone (m_T = 1: unchanged)
      M = __fmul_rn(M, c);
      const int e = pow2_exponent<GRID>(M);
      const float inv = __uint_as_float(__float_as_uint(ldexpf(1.0f, -e)) ^ sig);   // +-2^-e
#pragma unroll
      for (int j = 0; j < B; ++j) v[j] = __fmul_rn(__fmul_rn(y[blk * B + j], c), inv);
      if (e == 127) {   // only there can |v| exceed qmax
#pragma unroll
        for (int j = 0; j < B; ++j) v[j] = fminf(fmaxf(v[j], -qmax), qmax);
      }
      if constexpr (!DIAG) reinterpret_cast<uint8_t*>(scales_out)[blk] = (uint8_t)(e + 127);
    } else {
    float s = div_qmax<GRID>(M);  // s_B = RN(absmax / qmax)
    {
      // s = 0 (all-zero block, or absmax / qmax below the subnormal range):
      // every v is 0.  Running the quotient below with divisor 1 and
      // reciprocal 0 gives q = +-0, e = y, v = e * 0 + q = +-0 without a branch.
      const bool zero = s == 0.0f;
      const float sd = zero ? 1.0f : s;
      // RN(1/sd); outside [2^-60, 2^60] the quotients below take the IEEE
      // division and r is not used
      const float r = zero ? 0.0f : rcp_rn(sd);
      const float sdn = __uint_as_float(__float_as_uint(sd) ^ sig);   // divisor and
      const float rn = __uint_as_float(__float_as_uint(r) ^ sig);     // reciprocal, signed
      // Markstein: with r = RN(1/s) and q within an ulp of y/s, the fma
      // remainder is exact and RN(q + e r) = RN(y/s).  Preconditions: no
      // underflow of q or of the remainder.
      // An element with |y| < s 2^-39 may break the no-underflow condition;
      // RTNE sends it to level 0 whatever its quotient (every candidate is
      // below 2^-36 in size), so only SR and the diagnostics, which use v
      // itself, take the exact division for it.
      constexpr bool kTinyExact = RM == 1 || DIAG;
      const float thr = sd * 0x1p-39f;
      bool slow = !(sd >= 0x1p-60f && sd <= 0x1p60f);
#pragma unroll
      for (int j = 0; j < B; ++j) {
        const float yy = y[blk * B + j];
        const float q = __fmul_rn(yy, rn);
        const float e = __fmaf_rn(-q, sdn, yy);
        v[j] = __fmaf_rn(e, rn, q);
        if constexpr (kTinyExact) slow |= fabsf(yy) < thr;
      }
      if (__builtin_expect(slow, 0)) {
#pragma unroll
        for (int j = 0; j < B; ++j) v[j] = zero ? 0.0f : __fdiv_rn(y[blk * B + j], sdn);
      }
    }
    if constexpr (FOLD) {
      if (__builtin_expect(M * c < 0x1p-100f, 0)) {
        // literal path: y = RN(c x), s = RN(max|y| / qmax), v = RN(y / s)
        float M2 = 0.0f;
#pragma unroll
        for (int j = 0; j < B; ++j) M2 = fmaxf(M2, fabsf(__fmul_rn(y[blk * B + j], c)));
        s = __fdiv_rn(M2, qmax);
        const float s2 = __uint_as_float(__float_as_uint(s) ^ sig);
#pragma unroll
        for (int j = 0; j < B; ++j)
          v[j] = s == 0.0f ? 0.0f : __fdiv_rn(__fmul_rn(y[blk * B + j], c), s2);
      } else {
        s = __fmul_rn(s, c);   // exact: power of two, no underflow
      }
    }
    if constexpr (!DIAG) reinterpret_cast<float*>(scales_out)[blk] = s;
    }
    if constexpr (GRID == 3) {
      static_assert(RM == 0 && POW2 && !DIAG, "E4M3: RTNE with power-of-two scales");
#pragma unroll
      for (int j = 0; j < B; j += 2) {
        const int idx = blk * B + j;
        bytes[idx >> 2] = fp8_pair(bytes[idx >> 2], v[j], v[j + 1], (idx & 3) >> 1);
      }
      continue;
    }
    if constexpr (kHwFp4) {
#pragma unroll
      for (int j = 0; j < B; j += 2) {
        const int idx = blk * B + j;
        packed[idx >> 3] = fp4_pair(packed[idx >> 3], v[j], v[j + 1], (idx & 7) >> 1);
      }
      continue;
    }
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int idx = blk * B + j;
      uint32_t word;
      if constexpr (RM == 0) {
        word = rtne_word<GRID>(v[j]);   // no clamp needed: qmax + 1 ulp rounds to qmax
      } else {
        const float vc = fminf(fmaxf(v[j], -qmax), qmax);
        const uint32_t r16 = (rw[idx >> 1] >> (16 * (idx & 1))) & 0xFFFFu;
        word = sr_word<GRID>(vc, r16);
      }
      if constexpr (DIAG)
        diag_accumulate<GRID>(diag, word_nibble(word), fminf(fmaxf(v[j], -qmax), qmax));
      packed[idx >> 3] += word << (4 * (idx & 7));
    }
  }
  if constexpr (DIAG) return;
  if constexpr (GRID == 3) {
#pragma unroll
    for (int i = 0; i < W / 16; ++i)
      reinterpret_cast<uint4*>(codes_out)[i] =
          make_uint4(e4m3_clear_negzero(bytes[4 * i]), e4m3_clear_negzero(bytes[4 * i + 1]),
                     e4m3_clear_negzero(bytes[4 * i + 2]), e4m3_clear_negzero(bytes[4 * i + 3]));
    return;
  }
#pragma unroll
  for (int i = 0; i < W / 8; ++i)
    packed[i] = kHwFp4 ? fp4_clear_negzero(packed[i]) : finish_codes<GRID>(unbias_words(packed[i]));
  if constexpr (W == 16) {
    *reinterpret_cast<uint2*>(codes_out) = make_uint2(packed[0], packed[1]);
  } else {
    *reinterpret_cast<uint4*>(codes_out) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  }
}

// The rotated values of a lane (un-negated by its sign state).
template <int W>
__device__ __forceinline__ void store_rotated(float* dst, const float (&y)[W], uint32_t sig) {
  auto f = [&](int i) { return __uint_as_float(__float_as_uint(y[i]) ^ sig); };
#pragma unroll
  for (int i = 0; i < W; i += 4)
    *reinterpret_cast<float4*>(dst + i) = make_float4(f(i), f(i + 1), f(i + 2), f(i + 3));
}

// After the butterflies: normalize (or fold), optionally store the rotated
// values, quantize.  scales_out points at the lane's first scale (fp32 or
// E8M0 byte, by RND bit 1).
template <int W, int B, int N, int GRID, int RND, class Q>
__device__ __forceinline__ void finish_lane(float (&y)[W], uint32_t sig, const Q& q, uint64_t e0,
                                            uint8_t* codes_out, void* scales_out) {
  if constexpr (Rht<N>::fold && (RND & 2) == 0) {
    if (q.rotated == nullptr) {
      quantize_1d<W, B, GRID, RND, true>(y, sig, Rht<N>::c, e0, q.sr_seed, q.sr_stream,
                                         codes_out, scales_out);
      return;
    }
  }
  if constexpr (N > 1) scale_by<W>(y, q.cn);
  if (q.rotated) store_rotated<W>(q.rotated + e0, y, sig);
  quantize_1d<W, B, GRID, RND, false>(y, sig, q.tmul, e0, q.sr_seed, q.sr_stream, codes_out,
                                      scales_out);
}

// Address of scale number i of a 1D quantization (fp32 or E8M0 byte).
template <int RND>
__device__ __forceinline__ void* scale_at(void* base, uint64_t i) {
  if constexpr ((RND & 2) != 0) return reinterpret_cast<uint8_t*>(base) + i;
  else return reinterpret_cast<float*>(base) + i;
}

// ---------------------------------------------------------------------------
// Row-wise, 1 x B blocks: grid-stride over segments of W elements.
// ---------------------------------------------------------------------------
template <int W, int B, int N, int GRID, int RND>
__global__ __launch_bounds__(kThreads) void k_quant_rows(QuantLaunch q, FastDiv segs_per_row,
                                                         uint32_t nseg) {
  constexpr int lpc = N > W ? N / W : 1;
  const uint32_t tid = blockIdx.x * kThreads + threadIdx.x;
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  // Position of this lane inside its chunk of n elements; constant across the
  // grid-stride loop because stride and segs_per_row are multiples of lpc.
  const uint32_t qpos = tid & (uint32_t)(lpc - 1);
  uint32_t pm[W / 2];
  sign_masks<W>(select_pattern(q, qpos), pm);
  const uint32_t neg1 = (qpos & 1u) ? 0x80000000u : 0u;
  const uint32_t neg2 = (qpos & 2u) ? 0x80000000u : 0u;
  const uint32_t K = (uint32_t)q.K;
  with_exact(q.rotated != nullptr, [&](auto ex) {
    for (uint64_t s64 = tid; s64 < nseg; s64 += stride) {   // 64-bit: no wrap near 2^32
      const uint32_t seg = (uint32_t)s64;
      const uint32_t p = fdiv_u32(seg, segs_per_row);
      const uint32_t kseg = seg - p * segs_per_row.d;
      const uint32_t k0 = kseg * W;
      const uint16_t* src = q.x + (int64_t)p * q.ld + k0;
      uint32_t w[W / 2];
#pragma unroll
      for (int i = 0; i < W / 8; ++i) {
        const uint4 v = ld16(reinterpret_cast<const uint4*>(src) + i);
        w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
      }
      float y[W];
      unpack<W>(w, pm, y);
      const uint32_t sig = fwht<W, N>(y, neg1, neg2, decltype(ex)::value);
      const uint64_t e0 = (uint64_t)p * K + k0;
      finish_lane<W, B, N, GRID, RND, QuantLaunch>(y, sig, q, e0, code_ptr<GRID>(q.codes, e0),
                                      scale_at<RND>(q.scales, (uint64_t)p * (K / B) + k0 / B));
    }
  });
}

// ---------------------------------------------------------------------------
// Level statistics of a row-wise 1 x B quantization (diagnostics): the same
// pipeline as k_quant_rows, each element's level index and rounding error
// accumulated in the thread's LDS column instead of being stored; at the end
// the workgroup sums its columns and adds them (64-bit integer atomics) to
// a partial set: counts [0..7], error sums [8..15].
// ---------------------------------------------------------------------------
// Partial statistics of the workgroups live in a device buffer of
// kDiagSlots sets of 16 words (kDiagWorkspaceBytes) that the caller passes:
// the zeroing kernel clears them, workgroup b adds into set b % kDiagSlots,
// and the final kernel sums the sets into the caller's stats.  The three
// launches of one call are ordered by its stream; two calls may overlap only
// with different buffers.

template <int W, int B, int N, int GRID, int RND>
__global__ __launch_bounds__(kThreads) void k_quant_diag(QuantLaunch q, FastDiv segs_per_row,
                                                         uint32_t nseg,
                                                         unsigned long long* partials) {
  __shared__ DiagLds d;
  constexpr int lpc = N > W ? N / W : 1;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    d.cnt[k][threadIdx.x] = 0u;
    d.sum[k][threadIdx.x] = 0;
  }
  const uint32_t tid = blockIdx.x * kThreads + threadIdx.x;
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  const uint32_t qpos = tid & (uint32_t)(lpc - 1);
  uint32_t pm[W / 2];
  sign_masks<W>(select_pattern(q, qpos), pm);
  const uint32_t neg1 = (qpos & 1u) ? 0x80000000u : 0u;
  const uint32_t neg2 = (qpos & 2u) ? 0x80000000u : 0u;
  const uint32_t K = (uint32_t)q.K;
  for (uint64_t s64 = tid; s64 < nseg; s64 += stride) {   // 64-bit: no wrap near 2^32
    const uint32_t seg = (uint32_t)s64;
    const uint32_t p = fdiv_u32(seg, segs_per_row);
    const uint32_t k0 = (seg - p * segs_per_row.d) * W;
    const uint16_t* src = q.x + (int64_t)p * q.ld + k0;
    uint32_t w[W / 2];
#pragma unroll
    for (int i = 0; i < W / 8; ++i) {
      const uint4 v = ld16(reinterpret_cast<const uint4*>(src) + i);
      w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
    }
    float y[W];
    unpack<W>(w, pm, y);
    const uint32_t sig = fwht<W, N>(y, neg1, neg2, false);
    const uint64_t e0 = (uint64_t)p * K + k0;
    if constexpr (Rht<N>::fold && (RND & 2) == 0) {
      quantize_1d<W, B, GRID, RND, true, true>(y, sig, Rht<N>::c, e0, q.sr_seed, q.sr_stream,
                                               nullptr, nullptr, &d);
    } else {
      if constexpr (N > 1) scale_by<W>(y, q.cn);
      quantize_1d<W, B, GRID, RND, false, true>(y, sig, q.tmul, e0, q.sr_seed, q.sr_stream,
                                                nullptr, nullptr, &d);
    }
  }
  __syncthreads();
  // thread t sums level t / 32 over the columns t % 32 + 32 i, then the 32
  // threads of that level (one half of a wave) reduce by butterflies
  const int lev = threadIdx.x >> 5, part = threadIdx.x & 31;
  unsigned long long c = 0;
  long long sm = 0;
#pragma unroll
  for (int i = 0; i < kThreads / 32; ++i) {
    c += d.cnt[lev][part + 32 * i];
    sm += d.sum[lev][part + 32 * i];
  }
#pragma unroll
  for (int off = 16; off > 0; off >>= 1) {
    c += __shfl_xor(c, off);
    sm += __shfl_xor(sm, off);
  }
  if (part == 0) {   // one of kDiagSlots partial sets, so few workgroups share an address
    unsigned long long* slot = partials + (blockIdx.x % kDiagSlots) * 16;
    atomicAdd(slot + lev, c);
    atomicAdd(slot + 8 + lev, (unsigned long long)sm);
  }
}

// ---------------------------------------------------------------------------
// Column-wise (and segmented column-wise), 1 x B blocks.  A = X^T: a work-
// group stages X[k0 : k0+128, p0 : p0+64] in LDS and each lane pulls W
// consecutive k of one column p.  The tile is stored as 32-bit words holding
// rows (2i, 2i+1) of one column -- exactly the packed bf16 pairs the
// quantizer consumes -- so a lane reads W/2 words; the staging thread forms
// the pairs of 8 columns from two 16-byte row loads with 8 byte permutes.
// Words are [pair row][column], columns XOR-swizzled in groups of 4 (bits 2..4
// of the column) by bits 3..5 of the pair row and bits 5..7 of the column: the
// 4-word staging writes stay contiguous; lanes reading pair rows 8 apart (one
// Hadamard chunk spread over adjacent lanes) hit different banks; and the
// 16-byte reads of one pair row's 32-column segments, and the staging writes
// of 8 consecutive 8-column groups, fall on different banks (a pair row is a
// multiple of 32 words, so without the column term every such access of a
// pair row would land on the same four banks).
// ---------------------------------------------------------------------------
constexpr int kTK = 128, kTP = 64;

__device__ __forceinline__ int col_swz(int pr, int col) {
  return col ^ ((((pr >> 3) ^ (col >> 5)) & 7) << 2);
}
// (A lane's column segment starts at pair row kr / 2 = W / 2 * kseg, a multiple of
// 8 for W = 16 and 32: its pair rows come in groups of 8 with one swizzle each.)

template <int W, int B, int N, int GRID, int RND>
__global__ __launch_bounds__(kThreads) void k_quant_cols(QuantLaunch q) {
  static_assert(W % 16 == 0, "column segments of whole 8-pair swizzle groups");
  __shared__ uint32_t tile[(kTK / 2) * kTP];
  constexpr int lpc = N > W ? N / W : 1;
  // which segment / tile
  const int bid = blockIdx.x;
  int g = 0;
  while (g + 1 < q.nseg && q.tile_start[g + 1] <= bid) ++g;
  const int64_t seg0 = q.seg_off[g], seg1 = q.seg_off[g + 1];
  const int64_t L = seg1 - seg0;                       // K of this segment's operand
  const int64_t C = q.cols;                            // P of the operand
  const int tiles_p = (int)((C + kTP - 1) / kTP);
  const int local = bid - q.tile_start[g];
  const int tk = local / tiles_p, tp = local - tk * tiles_p;
  const int64_t k0 = (int64_t)tk * kTK;                // within the segment
  const int64_t p0 = (int64_t)tp * kTP;
  const int krows = (int)min<int64_t>(kTK, L - k0);
  const int pcols = (int)min<int64_t>(kTP, C - p0);

  // Stage: task = (pair row i, group of 8 columns); 64 x 8 tasks, 2 per thread.
  for (int t = threadIdx.x; t < (kTK / 2) * (kTP / 8); t += kThreads) {
    const int i = t / (kTP / 8), c8 = (t % (kTP / 8)) * 8;
    uint4 ra = make_uint4(0, 0, 0, 0), rb = ra;
    const int r = 2 * i;
    const uint16_t* src = q.x + (seg0 + k0 + r) * q.ld + p0 + c8;
    if (c8 + 8 <= pcols) {
      if (r < krows) ra = ld16(src);
      if (r + 1 < krows) rb = ld16(src + q.ld);
    } else {
      // ragged columns: element loads with compile-time indices (a runtime
      // index into a local array would place it in scratch memory)
      uint32_t ta[8], tb[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bool in = c8 + j < pcols;
        ta[j] = (in && r < krows) ? (uint32_t)src[j] : 0u;
        tb[j] = (in && r + 1 < krows) ? (uint32_t)src[q.ld + j] : 0u;
      }
      ra = make_uint4(ta[0] | (ta[1] << 16), ta[2] | (ta[3] << 16), ta[4] | (ta[5] << 16),
                      ta[6] | (ta[7] << 16));
      rb = make_uint4(tb[0] | (tb[1] << 16), tb[2] | (tb[3] << 16), tb[4] | (tb[5] << 16),
                      tb[6] | (tb[7] << 16));
    }
    const uint32_t a4[4] = {ra.x, ra.y, ra.z, ra.w}, b4[4] = {rb.x, rb.y, rb.z, rb.w};
    uint32_t o[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o[2 * j] = __builtin_amdgcn_perm(b4[j], a4[j], 0x05040100u);       // column 2j
      o[2 * j + 1] = __builtin_amdgcn_perm(b4[j], a4[j], 0x07060302u);   // column 2j+1
    }
    uint32_t* d = tile + i * kTP;
    *reinterpret_cast<uint4*>(d + col_swz(i, c8)) = make_uint4(o[0], o[1], o[2], o[3]);
    *reinterpret_cast<uint4*>(d + col_swz(i, c8 + 4)) = make_uint4(o[4], o[5], o[6], o[7]);
  }
  __syncthreads();

  constexpr int kSegsPerCol = kTK / W;
  const uint32_t qpos = threadIdx.x & (uint32_t)(lpc - 1);
  uint32_t pm[W / 2];
  sign_masks<W>(select_pattern(q, qpos), pm);
  const uint32_t neg1 = (qpos & 1u) ? 0x80000000u : 0u;
  const uint32_t neg2 = (qpos & 2u) ? 0x80000000u : 0u;
  with_exact(q.rotated != nullptr, [&](auto ex) {
    for (int u = threadIdx.x; u < kTP * kSegsPerCol; u += kThreads) {
      // consecutive lanes take consecutive W-segments of one column, so a
      // column's codes and scales are written by adjacent lanes (contiguous
      // stores), and the lanes of one Hadamard chunk are adjacent
      const int kseg = u % kSegsPerCol;
      const int col = u / kSegsPerCol;
      const int kr = kseg * W;
      if (kr >= krows || col >= pcols) continue;  // whole chunks drop out together
      // row pairs kr/2 .. kr/2 + W/2 - 1 in groups of 8 that share one swizzle
      uint32_t w[W / 2];
#pragma unroll
      for (int h = 0; h < W / 16; ++h) {
        const int pr = kr / 2 + 8 * h;
        const uint32_t* base = tile + pr * kTP + col_swz(pr, col);
#pragma unroll
        for (int i = 0; i < 8; ++i) w[8 * h + i] = base[i * kTP];
      }
      float y[W];
      unpack<W>(w, pm, y);
      const uint32_t sig = fwht<W, N>(y, neg1, neg2, decltype(ex)::value);
      const int64_t p = p0 + col;
      const int64_t k = k0 + kr;
      const uint64_t e0 = (uint64_t)C * seg0 + (uint64_t)p * L + k;   // global draw index
      finish_lane<W, B, N, GRID, RND, QuantLaunch>(y, sig, q, e0, code_ptr<GRID>(q.codes, e0),
                                      scale_at<RND>(q.scales, e0 / B));
    }
  });
}

// ---------------------------------------------------------------------------
// Both axes from one read of X (1 x B blocks): the column-wise quantization
// of a staged 128 x 64 tile exactly as k_quant_cols, then the row-wise
// quantization of the same tile (A = X, K = the columns) from the staged
// words -- a lane takes W consecutive columns of one row and keeps its row's
// bf16 half of each word.  The row side has its own signs, SR stream and
// outputs.  Hadamard chunks along the row must fit the tile width: tiles are
// 128 x 64 for n <= 64 and 128 x 128 for n = 128 (dual_tile_cols).
//
// A workgroup takes one tile, or two consecutive tiles (dual_tiles_per_wg).
// With two, when both are whole (no ragged rows or columns) the second tile's
// HBM loads are issued together with the first's and are in flight while the
// first is quantized; otherwise each tile is loaded and staged in turn.
// Measured on gfx950: the 128 x 64 tiles of n <= 64 run 17-35 % (RTNE) and
// 0-2 % (SR) faster two to a workgroup, while the 128 x 128 tiles of n = 128
// run 2-9 % faster one to a workgroup, with twice the workgroups and without
// the second tile's registers.
// ---------------------------------------------------------------------------
struct DualTile {
  int64_t seg0, L, k0, p0;
  int krows, pcols;
};

template <int TP>
__device__ __forceinline__ DualTile dual_tile(const QuantLaunch& q, int bid) {
  int g = 0;
  while (g + 1 < q.nseg && q.tile_start[g + 1] <= bid) ++g;
  DualTile d;
  d.seg0 = q.seg_off[g];
  d.L = q.seg_off[g + 1] - d.seg0;
  const int tiles_p = (int)((q.cols + TP - 1) / TP);
  const int local = bid - q.tile_start[g];
  const int tk = local / tiles_p, tp = local - tk * tiles_p;
  d.k0 = (int64_t)tk * kTK;
  d.p0 = (int64_t)tp * TP;
  d.krows = (int)min<int64_t>(kTK, d.L - d.k0);
  d.pcols = (int)min<int64_t>(TP, q.cols - d.p0);
  return d;
}

// Staging task j of this thread: pair row i, columns c8 .. c8+7 (2 tasks per
// thread for 64-column tiles, 4 for 128).
template <int TP> constexpr int stage_tasks() { return (kTK / 2) * (TP / 8) / kThreads; }

// Two bf16 rows (2i, 2i+1) x 8 columns -> 8 paired-row words in LDS.
template <int TP>
__device__ __forceinline__ void stage_pairs(uint32_t* tile, int i, int c8, uint4 ra, uint4 rb) {
  const uint32_t a4[4] = {ra.x, ra.y, ra.z, ra.w}, b4[4] = {rb.x, rb.y, rb.z, rb.w};
  uint32_t o[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    o[2 * j] = __builtin_amdgcn_perm(b4[j], a4[j], 0x05040100u);
    o[2 * j + 1] = __builtin_amdgcn_perm(b4[j], a4[j], 0x07060302u);
  }
  uint32_t* d = tile + i * TP;
  *reinterpret_cast<uint4*>(d + col_swz(i, c8)) = make_uint4(o[0], o[1], o[2], o[3]);
  *reinterpret_cast<uint4*>(d + col_swz(i, c8 + 4)) = make_uint4(o[4], o[5], o[6], o[7]);
}

// The 16-byte row loads of a whole tile (all rows and columns inside X).
template <int TP>
struct DualRegs {
  uint4 a[stage_tasks<TP>()], b[stage_tasks<TP>()];
};

template <int TP>
__device__ __forceinline__ void load_whole(const QuantLaunch& q, const DualTile& d,
                                           DualRegs<TP>& r) {
#pragma unroll
  for (int j = 0; j < stage_tasks<TP>(); ++j) {
    const int t = threadIdx.x + j * kThreads;
    const int i = t / (TP / 8), c8 = (t % (TP / 8)) * 8;
    const uint16_t* src = q.x + (d.seg0 + d.k0 + 2 * i) * q.ld + d.p0 + c8;
    r.a[j] = ld16(src);
    r.b[j] = ld16(src + q.ld);
  }
}

template <int TP>
__device__ __forceinline__ void stage_whole(const DualRegs<TP>& r, uint32_t* tile) {
#pragma unroll
  for (int j = 0; j < stage_tasks<TP>(); ++j) {
    const int t = threadIdx.x + j * kThreads;
    stage_pairs<TP>(tile, t / (TP / 8), (t % (TP / 8)) * 8, r.a[j], r.b[j]);
  }
}

// Any tile, ragged rows and columns read as zeros.
template <int TP>
__device__ __forceinline__ void load_stage_any(const QuantLaunch& q, const DualTile& d,
                                               uint32_t* tile) {
  for (int t = threadIdx.x; t < (kTK / 2) * (TP / 8); t += kThreads) {
    const int i = t / (TP / 8), c8 = (t % (TP / 8)) * 8;
    uint4 ra = make_uint4(0, 0, 0, 0), rb = ra;
    const int r = 2 * i;
    const uint16_t* src = q.x + (d.seg0 + d.k0 + r) * q.ld + d.p0 + c8;
    if (c8 + 8 <= d.pcols) {
      if (r < d.krows) ra = ld16(src);
      if (r + 1 < d.krows) rb = ld16(src + q.ld);
    } else {
      // ragged columns: element loads with compile-time indices (a runtime
      // index into a local array would place it in scratch memory)
      uint32_t ta[8], tb[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bool in = c8 + j < d.pcols;
        ta[j] = (in && r < d.krows) ? (uint32_t)src[j] : 0u;
        tb[j] = (in && r + 1 < d.krows) ? (uint32_t)src[q.ld + j] : 0u;
      }
      ra = make_uint4(ta[0] | (ta[1] << 16), ta[2] | (ta[3] << 16), ta[4] | (ta[5] << 16),
                      ta[6] | (ta[7] << 16));
      rb = make_uint4(tb[0] | (tb[1] << 16), tb[2] | (tb[3] << 16), tb[4] | (tb[5] << 16),
                      tb[6] | (tb[7] << 16));
    }
    stage_pairs<TP>(tile, i, c8, ra, rb);
  }
}

// Both quantizations of one staged tile.
template <int W, int B, int N, int GRID, int RND, int TP>
__device__ __forceinline__ void dual_quantize(const QuantLaunch& q, const RowSide& rside,
                                              const DualTile& d, const uint32_t* tile) {
  constexpr int lpc = N > W ? N / W : 1;
  const int64_t C = q.cols;
  const uint32_t qpos = threadIdx.x & (uint32_t)(lpc - 1);
  const uint32_t neg1 = (qpos & 1u) ? 0x80000000u : 0u;
  const uint32_t neg2 = (qpos & 2u) ? 0x80000000u : 0u;
  // column-wise: A = X^T, K = the segment's rows
  {
    uint32_t pm[W / 2];
    sign_masks<W>(select_pattern(q, qpos), pm);
    constexpr int kSegsPerCol = kTK / W;
    with_exact(q.rotated != nullptr, [&](auto ex) {
      for (int u = threadIdx.x; u < TP * kSegsPerCol; u += kThreads) {
        const int kseg = u % kSegsPerCol;
        const int col = u / kSegsPerCol;
        const int kr = kseg * W;
        if (kr >= d.krows || col >= d.pcols) continue;
        // row pairs kr/2 .. kr/2 + W/2 - 1: kr/2 is a multiple of 8 (W >= 16), so each
        // group of 8 shares one swizzle and the 8 reads are one base plus constants
        uint32_t w[W / 2];
#pragma unroll
        for (int h = 0; h < W / 16; ++h) {
          const int pr = kr / 2 + 8 * h;
          const uint32_t* base = tile + pr * TP + col_swz(pr, col);
#pragma unroll
          for (int i = 0; i < 8; ++i) w[8 * h + i] = base[i * TP];
        }
        float y[W];
        unpack<W>(w, pm, y);
        const uint32_t sig = fwht<W, N>(y, neg1, neg2, decltype(ex)::value);
        const uint64_t e0 = (uint64_t)C * d.seg0 + (uint64_t)(d.p0 + col) * d.L + (d.k0 + kr);
        finish_lane<W, B, N, GRID, RND, QuantLaunch>(y, sig, q, e0, code_ptr<GRID>(q.codes, e0),
                                                     scale_at<RND>(q.scales, e0 / B));
      }
    });
  }
  // row-wise: A = X, K = the columns
  {
    uint32_t pm[W / 2];
    sign_masks<W>(select_pattern(rside, qpos), pm);
    constexpr int kSegsPerRow = TP / W;
    with_exact(rside.rotated != nullptr, [&](auto ex) {
      for (int u = threadIdx.x; u < kTK * kSegsPerRow; u += kThreads) {
        const int seg = u % kSegsPerRow;
        const int row = u / kSegsPerRow;
        const int c0 = seg * W;
        if (row >= d.krows || c0 >= d.pcols) continue;   // whole chunks drop out together
        const int pr = row >> 1;
        const uint32_t sel = (row & 1) ? 0x07060302u : 0x05040100u;
        uint32_t w[W / 2];
#pragma unroll
        for (int j = 0; j < W / 4; ++j) {
          const uint4 v = *reinterpret_cast<const uint4*>(tile + pr * TP + col_swz(pr, c0 + 4 * j));
          w[2 * j] = __builtin_amdgcn_perm(v.y, v.x, sel);
          w[2 * j + 1] = __builtin_amdgcn_perm(v.w, v.z, sel);
        }
        float y[W];
        unpack<W>(w, pm, y);
        const uint32_t sig = fwht<W, N>(y, neg1, neg2, decltype(ex)::value);
        const uint64_t e0 = (uint64_t)(d.seg0 + d.k0 + row) * (uint64_t)C + (uint64_t)(d.p0 + c0);
        finish_lane<W, B, N, GRID, RND, RowSide>(y, sig, rside, e0, code_ptr<GRID>(rside.codes, e0),
                                                 scale_at<RND>(rside.scales, e0 / B));
      }
    });
  }
}

constexpr int dual_tiles_per_wg(int n) { return n == 128 ? 1 : 2; }

template <int W, int B, int N, int GRID, int RND>
__global__ __launch_bounds__(kThreads) void k_quant_dual(QuantLaunch q, RowSide rside) {
  static_assert(W % 16 == 0, "column segments of whole 8-pair swizzle groups");
  constexpr int TP = dual_tile_cols(N);
  __shared__ uint32_t tile[(kTK / 2) * TP];
  static_assert(N <= TP, "row-wise Hadamard chunks must fit the tile width");
  static_assert(stage_tasks<TP>() * kThreads == (kTK / 2) * (TP / 8), "staging tasks per thread");
  const int total = q.tile_start[q.nseg];
  constexpr int kTiles = dual_tiles_per_wg(N);
  const int b0 = kTiles * blockIdx.x;
  const bool two = kTiles == 2 && b0 + 1 < total;
  const DualTile d0 = dual_tile<TP>(q, b0);
  const DualTile d1 = dual_tile<TP>(q, two ? b0 + 1 : b0);
  const bool whole = d0.krows == kTK && d0.pcols == TP && d1.krows == kTK && d1.pcols == TP;
  if (whole) {
    DualRegs<TP> r0;
    load_whole<TP>(q, d0, r0);
    if constexpr (kTiles == 2) {
      DualRegs<TP> r1;
      load_whole<TP>(q, d1, r1);   // (the first tile again when there is no second)
      stage_whole<TP>(r0, tile);
      __syncthreads();
      dual_quantize<W, B, N, GRID, RND, TP>(q, rside, d0, tile);
      if (two) {
        __syncthreads();   // every lane is done reading the first tile
        stage_whole<TP>(r1, tile);
        __syncthreads();
        dual_quantize<W, B, N, GRID, RND, TP>(q, rside, d1, tile);
      }
    } else {
      stage_whole<TP>(r0, tile);
      __syncthreads();
      dual_quantize<W, B, N, GRID, RND, TP>(q, rside, d0, tile);
    }
  } else {
    load_stage_any<TP>(q, d0, tile);
    __syncthreads();
    dual_quantize<W, B, N, GRID, RND, TP>(q, rside, d0, tile);
    if (two) {
      __syncthreads();
      load_stage_any<TP>(q, d1, tile);
      __syncthreads();
      dual_quantize<W, B, N, GRID, RND, TP>(q, rside, d1, tile);
    }
  }
}

// ---------------------------------------------------------------------------
// Row-wise, BS x BS square blocks (BS = 16 or 32) with power-of-two (E8M0)
// scales ([2DFP4] 2D section).  A wave covers BS rows x 64 columns: lane l
// takes row (l % BS) of block column (l / BS); the block absmax is a
// BS-lane reduction.  The scale is the least e with M <= qmax 2^e.
// ---------------------------------------------------------------------------
template <int BS, int N, int GRID, int RND>
__global__ __launch_bounds__(kThreads) void k_quant_rows_2d(QuantLaunch q, uint32_t kgroups,
                                                            uint32_t nwaves) {
  constexpr int W = BS;
  constexpr uint32_t kPerWave = 64 / BS;   // block columns per wave
  constexpr float qmax = Grid<GRID>::qmax;
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  uint32_t pm[W / 2];
  sign_masks<W>(q.sign_pat[0], pm);
  const uint32_t K = (uint32_t)q.K;
  const uint32_t kblocks = K / BS;
  const uint64_t wstride = (uint64_t)gridDim.x * (kThreads / 64);
  for (uint64_t w64 = wave; w64 < nwaves; w64 += wstride) {   // 64-bit: no wrap near 2^32
    const uint32_t wv = (uint32_t)w64;
    const uint32_t pb = wv / kgroups;
    const uint32_t kb = (wv - pb * kgroups) * kPerWave + lane / BS;
    const bool valid = kb < kblocks;
    const uint32_t p = pb * BS + lane % BS;
    const uint32_t k0 = kb * BS;
    float y[W];
    float M = 0.0f;
    if (valid) {
      const uint16_t* src = q.x + (int64_t)p * q.ld + k0;
      uint32_t w[W / 2];
#pragma unroll
      for (int i = 0; i < W / 8; ++i) {
        const uint4 v = ld16(reinterpret_cast<const uint4*>(src) + i);
        w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
      }
      unpack<W>(w, pm, y);
      fwht<W, N>(y, 0u, 0u, true);   // N <= W: no cross-lane stage, sign state 0
      if constexpr (N > 1) scale_by<W>(y, q.cn);
#pragma unroll
      for (int j = 0; j < W; ++j) M = fmaxf(M, fabsf(y[j]));
    }
    // absmax over the BS rows of the block (lanes sharing l / BS)
#pragma unroll
    for (int m = 1; m < BS; m <<= 1) M = fmaxf(M, __shfl_xor(M, m, 64));
    if (!valid) continue;
    M = __fmul_rn(M, q.tmul);            // two-level: max |RN(y m_T)| = RN(M m_T)
    const int e = pow2_exponent<GRID>(M);
    const float inv = ldexpf(1.0f, -e);  // exact power of two (2^-127 is a subnormal)
    const uint64_t e0 = (uint64_t)p * K + k0;
    if (q.rotated) store_rotated<W>(q.rotated + e0, y, 0u);
    uint32_t rw[W / 2];
    if constexpr (RND == 1) sr_draws<W>(e0, q.sr_seed, q.sr_stream, rw);
    uint32_t packed[W / 8];
#pragma unroll
    for (int i = 0; i < W / 8; ++i) packed[i] = 0u;
#pragma unroll
    for (int j = 0; j < W; ++j) {
      // power-of-two scale: |v| <= qmax exactly unless e hit its clamp at 127
      float v = __fmul_rn(__fmul_rn(y[j], q.tmul), inv);
      if (e == 127) v = fminf(fmaxf(v, -qmax), qmax);
      uint32_t word;
      if constexpr (RND == 0) {
        word = rtne_word<GRID>(v);
      } else {
        word = sr_word<GRID>(v, (rw[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
      }
      packed[j >> 3] += word << (4 * (j & 7));
    }
#pragma unroll
    for (int i = 0; i < W / 8; ++i) packed[i] = finish_codes<GRID>(unbias_words(packed[i]));
    if constexpr (BS == 32)
      *reinterpret_cast<uint4*>(q.codes + (e0 >> 1)) =
          make_uint4(packed[0], packed[1], packed[2], packed[3]);
    else
      *reinterpret_cast<uint2*>(q.codes + (e0 >> 1)) = make_uint2(packed[0], packed[1]);
    if (lane % BS == 0u)
      reinterpret_cast<uint8_t*>(q.scales)[(uint64_t)pb * kblocks + kb] = (uint8_t)(e + 127);
  }
}

inline int device_grid_limit() {
  static int cus = 0;
  if (!cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = 256;
  }
  return cus;
}

inline int lane_width(int n, int bc) { return (bc == 32 || n >= 32) ? 32 : 16; }

template <int W, int B, int N, int G, int R>
hipError_t run_rows(const QuantLaunch& q, hipStream_t s) {
  const uint32_t segs_per_row = (uint32_t)(q.K / W);
  const uint64_t nseg = (uint64_t)q.P * segs_per_row;
  if (nseg == 0) return hipSuccess;
  // One segment per thread over a grid that covers the tensor (a grid-stride
  // loop only past 2^24 workgroups): on gfx950 this moved n = 16 RTNE from 5.15
  // to 6.17 TB/s against as many workgroups as fit on the chip at once.
  const uint64_t blocks_needed = (nseg + kThreads - 1) / kThreads;
  const uint64_t cap = (uint64_t)1 << 24;
  const uint32_t blocks = (uint32_t)(blocks_needed < cap ? blocks_needed : cap);
  hipLaunchKernelGGL((k_quant_rows<W, B, N, G, R>), dim3(blocks), dim3(kThreads), 0, s, q,
                     make_fastdiv(segs_per_row), (uint32_t)nseg);
  return hipGetLastError();
}

template <int G>
__global__ void k_diag_zero(unsigned long long* partials) {
  for (int i = threadIdx.x; i < kDiagSlots * 16; i += blockDim.x) partials[i] = 0ull;
}

template <int G>
__global__ void k_diag_final(const unsigned long long* partials, unsigned long long* stats) {
  if (threadIdx.x >= 16) return;
  unsigned long long t = 0;
  for (int s = 0; s < kDiagSlots; ++s) t += partials[s * 16 + threadIdx.x];
  stats[threadIdx.x] = t;
}

template <int W, int B, int N, int G, int R>
hipError_t run_diag(const QuantLaunch& q, unsigned long long* stats,
                    unsigned long long* partials, hipStream_t s) {
  hipLaunchKernelGGL(k_diag_zero<G>, dim3(1), dim3(256), 0, s, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint32_t segs_per_row = (uint32_t)(q.K / W);
  const uint64_t nseg = (uint64_t)q.P * segs_per_row;
  if (nseg > 0) {
    const uint64_t blocks_needed = (nseg + kThreads - 1) / kThreads;
    const uint64_t cap = (uint64_t)device_grid_limit() * 8;
    const uint32_t blocks = (uint32_t)(blocks_needed < cap ? blocks_needed : cap);
    hipLaunchKernelGGL((k_quant_diag<W, B, N, G, R>), dim3(blocks), dim3(kThreads), 0, s, q,
                       make_fastdiv(segs_per_row), (uint32_t)nseg, partials);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_diag_final<G>, dim3(1), dim3(64), 0, s, partials, stats);
  return hipGetLastError();
}

template <int G>
hipError_t run_diag_1d(const QuantLaunch& q, unsigned long long* stats,
                       unsigned long long* partials, hipStream_t s) {
#define UFP4_RUN(B_, N_)                                                                \
  if (q.bc == B_ && q.n == N_) {                                                       \
    constexpr int W_ = (B_ == 32 || N_ >= 32) ? 32 : 16;                               \
    if (B_ == 32 && q.scale_mode == 1) {                                                \
      if (q.rounding == 0) return run_diag<W_, B_, N_, G, 2>(q, stats, partials, s);    \
      return run_diag<W_, B_, N_, G, 3>(q, stats, partials, s);                         \
    }                                                                                   \
    if (q.rounding == 0) return run_diag<W_, B_, N_, G, 0>(q, stats, partials, s);      \
    return run_diag<W_, B_, N_, G, 1>(q, stats, partials, s);                           \
  }
#define UFP4_RUN_B(B_) \
  UFP4_RUN(B_, 1) UFP4_RUN(B_, 2) UFP4_RUN(B_, 4) UFP4_RUN(B_, 8) UFP4_RUN(B_, 16) \
  UFP4_RUN(B_, 32) UFP4_RUN(B_, 64) UFP4_RUN(B_, 128)
  UFP4_RUN_B(16)
  UFP4_RUN_B(32)
#undef UFP4_RUN_B
#undef UFP4_RUN
  return hipErrorInvalidValue;
}

template <int W, int B, int N, int G, int R>
hipError_t run_cols(const QuantLaunch& q, hipStream_t s) {
  const int total = q.tile_start[q.nseg];
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL((k_quant_cols<W, B, N, G, R>), dim3(total), dim3(kThreads), 0, s, q);
  return hipGetLastError();
}

template <int W, int B, int N, int G, int R>
hipError_t run_dual(const QuantLaunch& q, const RowSide& r, hipStream_t s) {
  const int total = q.tile_start[q.nseg];
  if (total == 0) return hipSuccess;
  constexpr int kTiles = dual_tiles_per_wg(N);
  hipLaunchKernelGGL((k_quant_dual<W, B, N, G, R>), dim3((total + kTiles - 1) / kTiles),
                     dim3(kThreads), 0, s,
                     q, r);
  return hipGetLastError();
}

template <int G>
hipError_t run_dual_1d(const QuantLaunch& q, const RowSide& r, hipStream_t s) {
#define UFP4_RUN(B_, N_)                                                       \
  if (q.bc == B_ && q.n == N_) {                                              \
    constexpr int W_ = (B_ == 32 || N_ >= 32) ? 32 : 16;                      \
    if (B_ == 32 && q.scale_mode == 1) {                                       \
      if (q.rounding == 0) return run_dual<W_, B_, N_, G, 2>(q, r, s);         \
      return run_dual<W_, B_, N_, G, 3>(q, r, s);                              \
    }                                                                          \
    if (q.rounding == 0) return run_dual<W_, B_, N_, G, 0>(q, r, s);           \
    return run_dual<W_, B_, N_, G, 1>(q, r, s);                                \
  }
#define UFP4_RUN_B(B_) \
  UFP4_RUN(B_, 1) UFP4_RUN(B_, 2) UFP4_RUN(B_, 4) UFP4_RUN(B_, 8) UFP4_RUN(B_, 16) \
  UFP4_RUN(B_, 32) UFP4_RUN(B_, 64) UFP4_RUN(B_, 128)
  UFP4_RUN_B(16)
  UFP4_RUN_B(32)
#undef UFP4_RUN_B
#undef UFP4_RUN
  return hipErrorInvalidValue;
}

// Dispatch over (n, block, rounding) for one codebook; W follows from n, b.
template <int G, bool COLS>
hipError_t run_1d(const QuantLaunch& q, hipStream_t s) {
#define UFP4_RUN(B_, N_)                                                                    \
  if (q.bc == B_ && q.n == N_) {                                                           \
    constexpr int W_ = (B_ == 32 || N_ >= 32) ? 32 : 16;                                   \
    if (B_ == 32 && q.scale_mode == 1) {                                                   \
      if (q.rounding == 0)                                                                 \
        return COLS ? run_cols<W_, B_, N_, G, 2>(q, s) : run_rows<W_, B_, N_, G, 2>(q, s); \
      return COLS ? run_cols<W_, B_, N_, G, 3>(q, s) : run_rows<W_, B_, N_, G, 3>(q, s);   \
    }                                                                                      \
    if (q.rounding == 0)                                                                   \
      return COLS ? run_cols<W_, B_, N_, G, 0>(q, s) : run_rows<W_, B_, N_, G, 0>(q, s);   \
    return COLS ? run_cols<W_, B_, N_, G, 1>(q, s) : run_rows<W_, B_, N_, G, 1>(q, s);     \
  }
#define UFP4_RUN_B(B_) \
  UFP4_RUN(B_, 1) UFP4_RUN(B_, 2) UFP4_RUN(B_, 4) UFP4_RUN(B_, 8) UFP4_RUN(B_, 16) \
  UFP4_RUN(B_, 32) UFP4_RUN(B_, 64) UFP4_RUN(B_, 128)
  UFP4_RUN_B(16)
  UFP4_RUN_B(32)
#undef UFP4_RUN_B
#undef UFP4_RUN
  return hipErrorInvalidValue;
}

template <int BS, int G>
hipError_t run_2d_bs(const QuantLaunch& q, hipStream_t s) {
  constexpr uint32_t kPerWave = 64 / BS;
  const uint32_t kblocks = (uint32_t)(q.K / BS);
  const uint32_t kgroups = (kblocks + kPerWave - 1) / kPerWave;
  const uint64_t nwaves = (uint64_t)(q.P / BS) * kgroups;
  if (nwaves == 0) return hipSuccess;
  const uint64_t blocks_needed = (nwaves + 3) / 4;
  // 16 workgroups per CU: a grid covering the tensor measured within -6 .. +4 %
  const uint64_t cap = (uint64_t)device_grid_limit() * 16;
  const uint32_t blocks = (uint32_t)(blocks_needed < cap ? blocks_needed : cap);
#define UFP4_2D(N_)                                                                             \
  if constexpr (N_ <= BS) {                                                                     \
    if (q.n == N_) {                                                                            \
      if (q.rounding == 0)                                                                      \
        hipLaunchKernelGGL((k_quant_rows_2d<BS, N_, G, 0>), dim3(blocks), dim3(kThreads), 0, s, \
                           q, kgroups, (uint32_t)nwaves);                                       \
      else                                                                                      \
        hipLaunchKernelGGL((k_quant_rows_2d<BS, N_, G, 1>), dim3(blocks), dim3(kThreads), 0, s, \
                           q, kgroups, (uint32_t)nwaves);                                       \
      return hipGetLastError();                                                                 \
    }                                                                                           \
  }
  UFP4_2D(1) UFP4_2D(2) UFP4_2D(4) UFP4_2D(8) UFP4_2D(16) UFP4_2D(32)
#undef UFP4_2D
  return hipErrorInvalidValue;
}

template <int G>
hipError_t run_2d(const QuantLaunch& q, hipStream_t s) {
  return q.br == 16 ? run_2d_bs<16, G>(q, s) : run_2d_bs<32, G>(q, s);
}

}  // namespace qk

// Per-codebook entry points (defined in quant_e1m2.hip / quant_int4.hip /
// quant_e2m1.hip).
template <int G> hipError_t quant_rows_grid(const QuantLaunch& q, hipStream_t s);
template <int G> hipError_t quant_cols_grid(const QuantLaunch& q, hipStream_t s);
template <int G> hipError_t quant_rows_2d_grid(const QuantLaunch& q, hipStream_t s);
template <int G> hipError_t quant_dual_grid(const QuantLaunch& q, const RowSide& r, hipStream_t s);
template <int G> hipError_t quant_diag_grid(const QuantLaunch& q, unsigned long long* stats,
                                           unsigned long long* partials, hipStream_t s);

}  // namespace ufp4
