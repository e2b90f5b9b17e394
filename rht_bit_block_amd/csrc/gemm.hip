// Block-scaled 4-bit GEMMs C[p][q] = sum_k A[p][k] * B[q][k] on gfx950 MFMA.
//
// [UFP4] = "Rethinking Shrinkage Bias in FP4 Pretraining of LLMs ... the UFP4
// Recipe" (hyper.ai summary, Method: Y^ = Q(X H') Q(W H')^T -- both operands
// are quantized in the rotated basis, so the GEMM contracts them directly).
// [2DFP4] = "Stable FP4 Training via Transposition-Invariant Block
// Quantization" (root cause: dX = dY W, dW = dY^T X).
//
// Scheme ("split-bf16"): the fp32 block scales are not powers of two, so the
// matrix cores cannot apply them and a per-block fp32 epilogue would leave the
// VALU as the bottleneck.  Instead every operand element is dequantized on the
// fly to d = RN(level * s) (the oracle's fp32 dequant value) and split into
// bf16 hi + lo (d - hi - lo = O(2^-17 d)); the product is accumulated as
// hi*hi + hi*lo + lo*hi with v_mfma_f32_32x32x16_bf16 (fp32 accumulate), so
// the whole K loop stays on the matrix cores and any block shape works.
//
// Tiling: 256 x 256 output tile per 512-thread workgroup (8 waves as 2 x 4,
// each wave 128 x 64 = 4 x 2 MFMA tiles of 32 x 32), K step 32.  The packed
// codes and scales of step i+1 are fetched into registers while step i runs
// its MFMAs; they are then decoded into the other half of a double-buffered
// LDS tile laid out [k-chunk of 8][row] so every fragment read is 16 B per
// lane with consecutive lanes on consecutive rows.
#include "ufp4_internal.h"

namespace ufp4 {

namespace {

constexpr int TM = 256, TN = 256, TK = 32;
constexpr int kThreads = 512;

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
__device__ __forceinline__ Problem resolve(const GemmLaunch& g, int tile, int& tm, int& tn) {
  int grp = 0;
  while (grp + 1 < g.ngroups && g.tile_start[grp + 1] <= tile) ++grp;
  const int local = tile - g.tile_start[grp];
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
  tm = local / max(tiles_n, 1);
  tn = local - tm * tiles_n;
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

// Whole-chunk decode used outside the K loop (prologue).
template <int GRID>
__device__ __forceinline__ void decode16(uint32_t w0, uint32_t w1, float s, const ResidualMasks& rm,
                                         uint4 (&hi)[2], uint4 (&lo)[2]) {
  const float su = s * Dec<GRID>::unit;
  const float nb = -Dec<GRID>::bias * su;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    uint32_t ev, od, h[4], l[4];
    decode8<GRID>(c ? w1 : w0, ev, od);
#pragma unroll
    for (int i = 0; i < 4; ++i) decode_pair(ev, od, i, su, nb, rm, h[i], l[i]);
    hi[c] = make_uint4(h[0], h[1], h[2], h[3]);
    lo[c] = make_uint4(l[0], l[1], l[2], l[3]);
  }
}

// Per-thread view of one operand inside the K loop: this thread owns row
// `row` of the tile and the 16 codes at k = 32*step + 16*half.  All index
// arithmetic is done once; the loop only advances pointers.  Rows past the
// operand read row 0 with a zero scale, and steps past K re-read the last
// valid step with a zero scale, so the loop body has no branches.
struct OperandCursor {
  const uint8_t* codes;     // row start + 8*half bytes
  const uint8_t* scales;    // fp32 or E8M0 scale of this thread's first block
  int32_t sstep;            // scale bytes per K step
  int32_t pow2;             // 1: E8M0 bytes, 0: fp32
  int32_t last;             // last step whose k < K
  float valid;              // 1 for rows inside the operand, else 0
};

__device__ __forceinline__ OperandCursor make_cursor(const uint8_t* codes, const void* scales,
                                                     int smode, int br, int bc, int64_t row,
                                                     int64_t row_end, int64_t row_begin,
                                                     int64_t K, int half) {
  OperandCursor c;
  c.valid = (row < row_end && K > 0) ? 1.0f : 0.0f;
  if (row >= row_end) row = row_begin;      // any in-range row (operand has >= 1 row)
  c.last = (int32_t)((K - 16 * half + 31) / 32) - 1;
  if (c.last < 0) { c.last = 0; c.valid = 0.0f; }
  const int h = (K > 16 * half) ? half : 0;  // keep the address inside the row
  c.codes = codes + row * (K >> 1) + 8 * h;
  const int64_t nb = K / bc;
  if (smode == 0) {
    c.scales = reinterpret_cast<const uint8_t*>(scales) + 4 * (row * nb + (16 * h) / bc);
    c.sstep = 4 * (32 / bc);
    c.pow2 = 0;
  } else {
    c.scales = reinterpret_cast<const uint8_t*>(scales) + (row / br) * nb;
    c.sstep = 1;
    c.pow2 = 1;
  }
  return c;
}

__device__ __forceinline__ void fetch(const OperandCursor& c, int step, uint2& codes, float& s) {
  const int st = step <= c.last ? step : c.last;
  const float v = step <= c.last ? c.valid : 0.0f;
  codes = *reinterpret_cast<const uint2*>(c.codes + 16 * st);
  float sc;
  if (c.pow2) {
    // 2^(e - 127): e >= 1 -> exponent field e; e == 0 -> subnormal 2^-127
    const uint32_t e = c.scales[st];
    sc = __uint_as_float(e ? (e << 23) : 0x00400000u);
  } else {
    sc = *reinterpret_cast<const float*>(c.scales + c.sstep * st);
  }
  s = sc * v;
}

template <int GRID>
__device__ __forceinline__ void stage(uint4* lds, int st, int row, int half, uint2 a, float sa,
                                      uint2 b, float sb, const ResidualMasks& rm) {
  uint4 hi[2], lo[2];
  uint4* base = lds + st * (kParts * kChunks * TM);
  decode16<GRID>(a.x, a.y, sa, rm, hi, lo);
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    base[(0 * kChunks + 2 * half + c) * TM + row] = hi[c];
    base[(1 * kChunks + 2 * half + c) * TM + row] = lo[c];
  }
  decode16<GRID>(b.x, b.y, sb, rm, hi, lo);
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    base[(2 * kChunks + 2 * half + c) * TM + row] = hi[c];
    base[(3 * kChunks + 2 * half + c) * TM + row] = lo[c];
  }
}

// Scheduling groups (mask bits of __builtin_amdgcn_sched_group_barrier).
constexpr int kSgMfma = 0x008, kSgValu = 0x002, kSgDsRead = 0x100, kSgDsWrite = 0x200,
              kSgVmemRead = 0x020;

template <int GRID>
__global__ __launch_bounds__(kThreads) void k_gemm(GemmLaunch g) {
  extern __shared__ uint4 lds[];
  int tm, tn;
  const Problem pr = resolve(g, blockIdx.x, tm, tn);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;   // 2 x 4 waves

  const int frow = tid >> 1, fhalf = tid & 1;
  const OperandCursor ca = make_cursor(pr.a_codes, pr.a_scales, g.scale_mode, g.a_br, g.a_bc,
                                       pr.a_row0 + (int64_t)tm * TM + frow,
                                       pr.a_row0 + pr.a_rows, pr.a_row0, pr.K, fhalf);
  const OperandCursor cb = make_cursor(pr.b_codes, pr.b_scales, g.scale_mode, g.b_br, g.b_bc,
                                       pr.b_row0 + (int64_t)tn * TN + frow,
                                       pr.b_row0 + pr.b_rows, pr.b_row0, pr.K, fhalf);
  const int nsteps = (int)((pr.K + TK - 1) / TK);

  floatx16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = floatx16{};

  // Software pipeline: step i's MFMAs read LDS buffer i&1 while the codes of
  // step i+1 (fetched during step i-1) are decoded into the other buffer and
  // the codes of step i+2 are in flight.
  uint2 fa, fb, na, nb;
  float sa, sb, nsa, nsb;
  fetch(ca, 0, fa, sa);
  fetch(cb, 0, fb, sb);
  const ResidualMasks rm = make_masks();
  stage<GRID>(lds, 0, frow, fhalf, fa, sa, fb, sb, rm);
  fetch(ca, 1, fa, sa);
  fetch(cb, 1, fb, sb);
  __syncthreads();

  for (int step = 0; step < nsteps; ++step) {
    const int st = step & 1;
    fetch(ca, step + 2, na, nsa);     // re-reads the last step past the end (scale 0)
    fetch(cb, step + 2, nb, nsb);

    const uint4* base = lds + st * (kParts * kChunks * TM);
    uint4* nxt = lds + (st ^ 1) * (kParts * kChunks * TM);
    // Decode state of the next step: 4 dwords of codes (A w0, A w1, B w0,
    // B w1), each expanded to even/odd level bytes, then 4 pairs each.
    const uint32_t words[4] = {fa.x, fa.y, fb.x, fb.y};
    const float su[2] = {sa * Dec<GRID>::unit, sb * Dec<GRID>::unit};
    const float nbias[2] = {-Dec<GRID>::bias * su[0], -Dec<GRID>::bias * su[1]};
    uint32_t ev[4], od[4];
    uint32_t hreg[4][4], lreg[4][4];
    // MFMA sequence: 2 k-halves x 3 products x 8 tiles = 48.  After every
    // third MFMA one decode piece runs (16 pieces = 4 dwords x 4 pairs),
    // and the byte expansion of dword w runs before its first pair.
    bf16x8 ah[4], al[4], bh[2], bl[2];
    // fragment loads of k-half kh for part p (0 A_hi, 1 A_lo, 2 B_hi, 3 B_lo)
    auto load_part = [&](int kh, int p) {
      const int chunk = 2 * kh + (lane >> 5);
      if (p < 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = wm * 128 + i * 32 + (lane & 31);
          const bf16x8 v = __builtin_bit_cast(bf16x8, base[(p * kChunks + chunk) * TM + r]);
          if (p == 0) ah[i] = v; else al[i] = v;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int r = wn * 64 + j * 32 + (lane & 31);
          const bf16x8 v = __builtin_bit_cast(bf16x8, base[(p * kChunks + chunk) * TM + r]);
          if (p == 2) bh[j] = v; else bl[j] = v;
        }
      }
    };
    // Product order per k-half: kh0 = hh, hl, lh; kh1 = hl, hh, lh.  A_hi and
    // B_lo of kh1 are fetched at MFMA 16 (their kh0 copies are dead after
    // hl), A_lo and B_hi of kh1 at MFMA 24.
    load_part(0, 0); load_part(0, 2); load_part(0, 3); load_part(0, 1);
#pragma unroll
    for (int m = 0; m < 48; ++m) {
      const int kh = m / 24, t = m % 8, i = t >> 1, j = t & 1;
      const int slot = (m % 24) / 8;                        // 0, 1, 2 within the k-half
      const int prod = kh == 0 ? slot : (slot == 0 ? 1 : (slot == 1 ? 0 : 2));  // 0 hh 1 hl 2 lh
      if (m == 16) { load_part(1, 0); load_part(1, 3); }
      if (m == 24) { load_part(1, 2); load_part(1, 1); }
      const bf16x8 av = prod == 2 ? al[i] : ah[i];
      const bf16x8 bv = prod == 1 ? bl[j] : bh[j];
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[i][j], 0, 0, 0);
      if (m % 3 == 2) {
        const int piece = m / 3;          // 0..15
        const int w = piece >> 2, pr2 = piece & 3;
        if (pr2 == 0) decode8<GRID>(words[w], ev[w], od[w]);
        decode_pair(ev[w], od[w], pr2, su[w >> 1], nbias[w >> 1], rm, hreg[w][pr2], lreg[w][pr2]);
        if (pr2 == 3) {
          // dword w of the codes = chunk (2*half + (w & 1)) of operand (w >> 1)
          const int opnd = w >> 1, c = 2 * fhalf + (w & 1);
          nxt[((2 * opnd + 0) * kChunks + c) * TM + frow] =
              make_uint4(hreg[w][0], hreg[w][1], hreg[w][2], hreg[w][3]);
          nxt[((2 * opnd + 1) * kChunks + c) * TM + frow] =
              make_uint4(lreg[w][0], lreg[w][1], lreg[w][2], lreg[w][3]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    fa = na; fb = nb; sa = nsa; sb = nsb;
  }

  // Epilogue: lane holds column (lane & 31) and rows 8*(r/4) + 4*(lane/32) + r%4.
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = (int64_t)tn * TN + wn * 64 + j * 32 + (lane & 31);
      if (col >= pr.b_rows) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = (int64_t)tm * TM + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < pr.a_rows) pr.c[row * g.ldc + col] = acc[i][j][r];
      }
    }
}

}  // namespace

hipError_t launch_gemm(const GemmLaunch& g, hipStream_t s) {
  if (g.total_tiles == 0) return hipSuccess;
  static bool attr_set = false;
  if (!attr_set) {
    const void* fns[3] = {(const void*)k_gemm<0>, (const void*)k_gemm<1>, (const void*)k_gemm<2>};
    for (const void* f : fns) {
      hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
      if (e != hipSuccess) return e;
    }
    attr_set = true;
  }
  switch (g.grid) {
    case 0: hipLaunchKernelGGL(k_gemm<0>, dim3(g.total_tiles), dim3(kThreads), kLdsBytes, s, g); break;
    case 1: hipLaunchKernelGGL(k_gemm<1>, dim3(g.total_tiles), dim3(kThreads), kLdsBytes, s, g); break;
    default: hipLaunchKernelGGL(k_gemm<2>, dim3(g.total_tiles), dim3(kThreads), kLdsBytes, s, g); break;
  }
  return hipGetLastError();
}

}  // namespace ufp4
