// Block-scaled 4-bit GEMMs C[p][q] = sum_k A[p][k] * B[q][k] on gfx950 MFMA.
//
// [UFP4] = "Rethinking Shrinkage Bias in FP4 Pretraining of LLMs ... the UFP4
// Recipe" (hyper.ai summary, Method: Y^ = Q(X H') Q(W H')^T -- both operands
// are quantized in the rotated basis, so the GEMM contracts them directly).
// [2DFP4] = "Stable FP4 Training via Transposition-Invariant Block
// Quantization" (root cause: dX = dY W, dW = dY^T X).
//
// Scheme of this general kernel ("split-bf16"): every operand element is
// dequantized on the fly to d = RN(level * s) (the oracle's fp32 dequant
// value) and split into bf16 hi + lo (d - hi - lo = O(2^-17 d)); the product
// is accumulated as hi*hi + hi*lo + lo*hi with v_mfma_f32_32x32x16_bf16 (fp32
// accumulate), so the whole K loop stays on the matrix cores and any pair of
// block shapes works.  1 x 16 and 1 x 32 fp32-scale operands go to the
// scale-product kernel instead (exact level products, fp32 scale epilogue).
//
// This file holds the general kernel, used for every case the specialised
// kernels do not take (mixed block shapes between the operands, fp32 scales on
// 32 x 32 blocks, power-of-two scales with K % 128 != 0 or in grouped GEMMs):
// 256 x 256 output tile per 512-thread workgroup, two waves per SIMD (8 waves
// of 128 x 64 = 4 x 2 MFMA tiles, 128 accumulators each), K step 32.  Each
// thread owns one row of one operand per step (waves 0-3: A, 4-7: B): the
// packed codes and scales of step i+2 are fetched into registers, step i+1 is
// decoded into the other LDS buffer between the two k-halves of step i, one
// barrier per step.  The LDS tile is laid out [part][k-chunk of 8][row] x
// 16 B, so a fragment read is 16 B per lane with consecutive lanes on
// consecutive rows.
#include "ufp4_internal.h"
#include "gemm_epilogue.h"

namespace ufp4 {

namespace {

constexpr int TM = 256, TN = 256, TK = 32;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// LDS: [stage][part: A_hi, A_lo, B_hi, B_lo][k-chunk 0..3][row 0..255] x 16 B
constexpr int kParts = 4, kChunks = TK / 8;
constexpr int kLdsBytes = 2 * kParts * kChunks * TM * 16;  // 128 KiB

struct Problem {
  const uint8_t* a_codes;
  const uint8_t* b_codes;
  const void* a_scales;
  const void* b_scales;
  float* c;
  int64_t a_rows, b_rows, K;      // this group's extents
  int64_t a_row0, b_row0;         // first row inside the (shared) operand arrays
};

// Resolve which group a tile belongs to and the group's operand views.
__device__ __forceinline__ Problem resolve(const GemmLaunch& g, int b, int& tm, int& tn) {
  int grp, local;
  slot_tile(g, b, grp, local);
  Problem pr;
  if (g.mode == 0) {
    pr.a_codes = g.a_codes; pr.b_codes = g.b_codes;
    pr.a_scales = g.a_scales; pr.b_scales = g.b_scales;
    pr.c = g.c;
    pr.a_rows = g.PA; pr.b_rows = g.PB; pr.K = g.K;
    pr.a_row0 = 0; pr.b_row0 = 0;
  } else if (g.mode == 1) {
    // rows [off[grp], off[grp+1]) of A; rows grp*R .. of B; C rows as A
    pr.a_codes = g.a_codes; pr.b_codes = g.b_codes;
    pr.a_scales = g.a_scales; pr.b_scales = g.b_scales;
    pr.a_row0 = g.off[grp];
    pr.b_row0 = (int64_t)grp * g.b_rows_per_group;
    pr.a_rows = g.off[grp + 1] - g.off[grp];
    pr.b_rows = g.b_rows_per_group;
    pr.K = g.K;
    pr.c = g.c + pr.a_row0 * g.ldc;
  } else {
    // segment grp of both operands: K = segment length, operands stored
    // [P][L] at element offset P * off[grp]
    const int64_t o = g.off[grp], L = g.off[grp + 1] - g.off[grp];
    pr.a_codes = g.a_codes + (g.PA * o) / 2;
    pr.b_codes = g.b_codes + (g.PB * o) / 2;
    pr.a_scales = reinterpret_cast<const float*>(g.a_scales) + (g.PA * o) / g.a_bc;
    pr.b_scales = reinterpret_cast<const float*>(g.b_scales) + (g.PB * o) / g.b_bc;
    pr.a_rows = g.PA; pr.b_rows = g.PB; pr.K = L;
    pr.a_row0 = 0; pr.b_row0 = 0;
    pr.c = g.c + (int64_t)grp * g.PA * g.ldc;
  }
  const int tiles_n = (int)((pr.b_rows + TN - 1) / TN);
  grouped_order(local, (int)((pr.a_rows + TM - 1) / TM), max(tiles_n, 1), tm, tn);
  return pr;
}

// Decode of packed codes to MFMA operands.  Codes become offset-binary level
// bytes u (level / unit = u - bias, bias a power of two so bias * s is exact):
//   INT4 (two's complement nibble):  u = c ^ 8                    (bias 8)
//   E1M2 (sign-magnitude, unit 1/4): u = 8 + k or 8 - k           (bias 8)
//   E2M1 (sign-magnitude, unit 1/2): u = 16 +- {0,1,2,3,4,6,8,12} (bias 16)
// d = fma(u, s*unit, -bias*s*unit) = RN(level * s), the fp32 dequant value;
// it is split into hi = RN_bf16(d) and lo = RN_bf16(d - hi), the residual
// d - hi being exact (v_dot2 of hi with (-1, 0) added to d).
template <int GRID> struct Dec;
template <> struct Dec<0> { static constexpr float unit = 0.25f, bias = 8.0f; };
template <> struct Dec<1> { static constexpr float unit = 1.0f, bias = 8.0f; };
template <> struct Dec<2> { static constexpr float unit = 0.5f, bias = 16.0f; };

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// 8 code nibbles (one dword, element j at bits 4j) -> offset-binary bytes of
// elements 0,2,4,6 (ev) and 1,3,5,7 (od).
template <int GRID>
__device__ __forceinline__ void decode8(uint32_t w, uint32_t& ev, uint32_t& od) {
  if constexpr (GRID == 1) {
    const uint32_t x = w ^ 0x88888888u;
    ev = x & 0x0F0F0F0Fu;
    od = (x >> 4) & 0x0F0F0F0Fu;
  } else if constexpr (GRID == 0) {
    // per nibble: u = s ? (m ^ 7) + 1 : m + 8, done as (m ^ 7s) + 8 - 7s
    const uint32_t sgn = w & 0x88888888u;
    const uint32_t neg7 = sgn - (sgn >> 3);                 // 7 in negative nibbles
    const uint32_t x = ((w & 0x77777777u) ^ neg7) + (0x88888888u - neg7);
    ev = x & 0x0F0F0F0Fu;
    od = (x >> 4) & 0x0F0F0F0Fu;
  } else {
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    auto map = [](uint32_t v) {
      const uint32_t idx = v & 0x07070707u;
      const uint32_t pos = __builtin_amdgcn_perm(0x1C181614u, 0x13121110u, idx);
      const uint32_t neg = __builtin_amdgcn_perm(0x04080A0Cu, 0x0D0E0F10u, idx);
      const uint32_t b = (v >> 3) & 0x01010101u;
      const uint32_t m = (b << 8) - b;                      // 0xFF in negative bytes
      return (neg & m) | (pos & ~m);
    };
    ev = map(lo);
    od = map(hi);
  }
}

__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};  // round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

// Selector pairs (-1, 0) and (0, -1) for the residual dot products, held in
// registers: the packed-bf16 operand must not be folded into an inline
// constant, whose 32-bit reading would not be the intended pair.
struct ResidualMasks {
  bf16x2 m0, m1;
};
__device__ __forceinline__ ResidualMasks make_masks() {
  uint32_t a = 0x0000BF80u, b = 0xBF800000u;   // low half = element 0
  asm volatile("" : "+s"(a), "+s"(b));
  return {__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b)};
}

// Elements 2i and 2i+1 of a decoded dword -> packed bf16 hi and lo pairs.
__device__ __forceinline__ void decode_pair(uint32_t ev, uint32_t od, int i, float su, float nb,
                                            const ResidualMasks& rm, uint32_t& hi,
                                            uint32_t& lo) {
  const float u0 = (float)((ev >> (8 * i)) & 0xFFu);
  const float u1 = (float)((od >> (8 * i)) & 0xFFu);
  const float d0 = __fmaf_rn(u0, su, nb);
  const float d1 = __fmaf_rn(u1, su, nb);
  hi = pk_bf16(d0, d1);
  const bf16x2 h = __builtin_bit_cast(bf16x2, hi);
  const float r0 = __builtin_amdgcn_fdot2_f32_bf16(h, rm.m0, d0, false);  // d0 - hi0, exact
  const float r1 = __builtin_amdgcn_fdot2_f32_bf16(h, rm.m1, d1, false);  // d1 - hi1, exact
  lo = pk_bf16(r0, r1);
}

// Per-thread view of one operand inside the K loop: this thread owns row
// `row` of the tile and the 32 codes of each K step.  Index arithmetic is done
// once; the loop only advances pointers.  Rows past the operand re-read a
// valid row with a zero scale, and steps past K re-read the last valid step
// with a zero scale, so the loop body has no data-dependent branches.
struct OperandCursor {
  const uint8_t* codes;     // start of this thread's row
  const uint8_t* scales;    // first scale of the row (fp32 or E8M0 bytes)
  int32_t pow2;             // 1: E8M0 bytes, 0: fp32
  int32_t per_step;         // fp32 scales per K step (2 for 1x16 blocks, 1 for 1x32)
  int32_t last;             // last step with any k < K
  int32_t half_last;        // 1 when the last step holds only 16 codes
  float valid;              // 1 for rows inside the operand, else 0
};

__device__ __forceinline__ OperandCursor make_cursor(const uint8_t* codes, const void* scales,
                                                     int smode, int br, int bc, int64_t row,
                                                     int64_t row_end, int64_t row_begin,
                                                     int64_t K) {
  OperandCursor c;
  c.valid = (row < row_end && K > 0) ? 1.0f : 0.0f;
  if (row >= row_end) row = row_begin;  // an in-range row (the operand has >= 1 row)
  c.last = (int32_t)((K + TK - 1) / TK) - 1;
  c.half_last = (K % TK) != 0;
  if (c.last < 0) { c.last = 0; c.valid = 0.0f; }
  c.codes = codes + row * (K >> 1);
  const int64_t nb = K / bc;
  if (smode == 0) {
    c.scales = reinterpret_cast<const uint8_t*>(scales) + 4 * row * nb;
    c.pow2 = 0;
    c.per_step = TK / bc;
  } else {
    c.scales = reinterpret_cast<const uint8_t*>(scales) + (row / br) * nb;
    c.pow2 = 1;
    c.per_step = TK / bc;
  }
  return c;
}

// Raw loads of one K step.  Nothing is computed from them at fetch time:
// using a loaded value right away would make the wave wait for the memory
// latency; they are finalized when decoded, one step later.
struct Fetched {
  uint2 c0, c1;       // codes 0..15 and 16..31 (c1 re-reads c0 on a half step)
  uint32_t s0, s1;    // raw scale bits (fp32 bits, or the E8M0 byte)
  float v0, v1;       // 1 or 0: row inside the operand and k < K
};

template <int SMODE>
__device__ __forceinline__ Fetched fetch(const OperandCursor& c, int step) {
  Fetched f;
  const int st = step <= c.last ? step : c.last;
  const float v = step <= c.last ? c.valid : 0.0f;
  const bool half = c.half_last && st == c.last;
  const uint8_t* p = c.codes + 16 * st;
  f.c0 = *reinterpret_cast<const uint2*>(p);
  f.c1 = *reinterpret_cast<const uint2*>(p + (half ? 0 : 8));
  if constexpr (SMODE == 1) {
    // E8M0 bytes of 32-element blocks: one per 32-wide step
    f.s0 = f.s1 = c.scales[st];
  } else if constexpr (SMODE == 2) {
    // E8M0 bytes, 16- or 32-element blocks: one or two per 32-wide step
    const int i0 = st * c.per_step;
    f.s0 = c.scales[i0];
    f.s1 = c.scales[i0 + ((c.per_step == 2 && !half) ? 1 : 0)];
  } else {
    // branch-free: 1x16 blocks -> scales 2st, 2st+1; 1x32 -> scale st twice
    const uint32_t* q = reinterpret_cast<const uint32_t*>(c.scales);
    const int i0 = st * c.per_step;
    const int i1 = i0 + ((c.per_step == 2 && !half) ? 1 : 0);
    f.s0 = q[i0];
    f.s1 = q[i1];
  }
  f.v0 = v;
  f.v1 = half ? 0.0f : v;
  return f;
}

template <int SMODE>
__device__ __forceinline__ float finalize_scale(uint32_t raw, float v) {
  float s;
  if constexpr (SMODE != 0) {
    // 2^(e - 127): e >= 1 -> exponent field e; e == 0 -> subnormal 2^-127
    s = __uint_as_float(raw ? (raw << 23) : 0x00400000u);
  } else {
    s = __uint_as_float(raw);
  }
  return s * v;
}

// ---------------------------------------------------------------------------
// The kernel.  With two waves resident on every SIMD the hardware issues one
// wave's decode VALU while the other wave's MFMAs run.
// ---------------------------------------------------------------------------
constexpr int kThreads8 = 512;

template <int GRID, int SMODE>
__device__ __forceinline__ void decode_row(const Fetched& f, const ResidualMasks& rm, uint4* buf,
                                           int part, int row) {
  const float s0 = finalize_scale<SMODE>(f.s0, f.v0);
  const float s1 = finalize_scale<SMODE>(f.s1, f.v1);
#pragma unroll
  for (int cw = 0; cw < 4; ++cw) {
    const uint32_t word = cw == 0 ? f.c0.x : (cw == 1 ? f.c0.y : (cw == 2 ? f.c1.x : f.c1.y));
    const float su = (cw < 2 ? s0 : s1) * Dec<GRID>::unit;
    const float nb = -Dec<GRID>::bias * su;
    uint32_t ev, od, h[4], l[4];
    decode8<GRID>(word, ev, od);
#pragma unroll
    for (int i = 0; i < 4; ++i) decode_pair(ev, od, i, su, nb, rm, h[i], l[i]);
    buf[(part * kChunks + cw) * TM + row] = make_uint4(h[0], h[1], h[2], h[3]);
    buf[((part + 1) * kChunks + cw) * TM + row] = make_uint4(l[0], l[1], l[2], l[3]);
  }
}

struct Frags8 {
  bf16x8 ah[4], al[4], bh[2], bl[2];
};

__device__ __forceinline__ void load_frags8(const uint4* buf, int kh, int lane, int wm, int wn,
                                            Frags8& f) {
  const int chunk = 2 * kh + (lane >> 5);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ra = wm * 128 + i * 32 + (lane & 31);
    f.ah[i] = __builtin_bit_cast(bf16x8, buf[(0 * kChunks + chunk) * TM + ra]);
    f.al[i] = __builtin_bit_cast(bf16x8, buf[(1 * kChunks + chunk) * TM + ra]);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int rb = wn * 64 + j * 32 + (lane & 31);
    f.bh[j] = __builtin_bit_cast(bf16x8, buf[(2 * kChunks + chunk) * TM + rb]);
    f.bl[j] = __builtin_bit_cast(bf16x8, buf[(3 * kChunks + chunk) * TM + rb]);
  }
}

__device__ __forceinline__ void mfma_khalf8(floatx16 (&acc)[4][2], const Frags8& f) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.ah[i], f.bh[j], acc[i][j], 0, 0, 0);
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.ah[i], f.bl[j], acc[i][j], 0, 0, 0);
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.al[i], f.bh[j], acc[i][j], 0, 0, 0);
    }
}

template <int GRID, int SMODE>
__global__ __launch_bounds__(kThreads8) void k_gemm8(GemmLaunch g) {
  extern __shared__ uint4 lds[];
  int tm, tn;
  const Problem pr = resolve(g, blockIdx.x, tm, tn);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;   // 2 x 4 waves of 128 x 64
  const int op = tid >> 8, row = tid & 255;  // the operand row this thread decodes
  const ResidualMasks rm = make_masks();

  const OperandCursor cur = op == 0
      ? make_cursor(pr.a_codes, pr.a_scales, g.scale_mode, g.a_br, g.a_bc,
                    pr.a_row0 + (int64_t)tm * TM + row, pr.a_row0 + pr.a_rows, pr.a_row0, pr.K)
      : make_cursor(pr.b_codes, pr.b_scales, g.scale_mode, g.b_br, g.b_bc,
                    pr.b_row0 + (int64_t)tn * TN + row, pr.b_row0 + pr.b_rows, pr.b_row0, pr.K);
  const int part = 2 * op;
  const int nsteps = (int)((pr.K + TK - 1) / TK);
  constexpr int kStage = kParts * kChunks * TM;

  floatx16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = floatx16{};

  // K == 0 (an empty expert, or an empty operand whose storage may be null):
  // no code or scale is read and the tile stores zeros.
  if (nsteps > 0) {
    decode_row<GRID, SMODE>(fetch<SMODE>(cur, 0), rm, lds, part, row);
    Fetched x = fetch<SMODE>(cur, 1), y;
    __syncthreads();

    auto body = [&](int step, const Fetched& d, Fetched& l) {
      const uint4* cb = lds + (step & 1) * kStage;
      uint4* nb = lds + ((step + 1) & 1) * kStage;
      l = fetch<SMODE>(cur, step + 2);
      Frags8 f;
      load_frags8(cb, 0, lane, wm, wn, f);
      mfma_khalf8(acc, f);
      decode_row<GRID, SMODE>(d, rm, nb, part, row);
      load_frags8(cb, 1, lane, wm, wn, f);
      mfma_khalf8(acc, f);
      __syncthreads();
    };
    int step = 0;
    for (; step + 1 < nsteps; step += 2) {
      body(step, x, y);
      body(step + 1, y, x);
    }
    if (step < nsteps) body(step, x, y);
  }

  {
    const int64_t row0 = (int64_t)tm * TM, col0 = (int64_t)tn * TN;
    const int rv = (int)(pr.a_rows - row0 < TM ? pr.a_rows - row0 : TM);
    const int cv = (int)(pr.b_rows - col0 < TN ? pr.b_rows - col0 : TN);
    store_c<4, 2>(pr.c + row0 * g.ldc + col0, g.ldc, rv, cv, wm * 128, wn * 64, lane, acc,
                  g.c_mul);
  }
}

}  // namespace

template <int GRID, int SMODE>
hipError_t launch_one(const GemmLaunch& g, hipStream_t s) {
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t e = set_lds_limit((const void*)k_gemm8<GRID, SMODE>, kLdsBytes, lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_gemm8<GRID, SMODE>), dim3(g.total_tiles), dim3(kThreads8), kLdsBytes, s, g);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmLaunch& g, hipStream_t s) {
  if (g.total_tiles == 0) return hipSuccess;
  if (gemm_rd_supported(g)) return launch_gemm_rd(g, s);
  // scale modes: 0 fp32; 1 E8M0 with 32-element blocks on both operands; 2 E8M0
  // with a 16-element block on either
  const int sm = g.scale_mode == 0 ? 0 : (g.a_bc == 32 && g.b_bc == 32 ? 1 : 2);
  switch (g.grid * 3 + sm) {
    case 0: return launch_one<0, 0>(g, s);
    case 1: return launch_one<0, 1>(g, s);
    case 2: return launch_one<0, 2>(g, s);
    case 3: return launch_one<1, 0>(g, s);
    case 4: return launch_one<1, 1>(g, s);
    case 5: return launch_one<1, 2>(g, s);
    case 6: return launch_one<2, 0>(g, s);
    case 7: return launch_one<2, 1>(g, s);
    default: return launch_one<2, 2>(g, s);
  }
}

}  // namespace ufp4
