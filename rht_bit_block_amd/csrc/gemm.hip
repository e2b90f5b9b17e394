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

// Signed level LUTs (16 entries, bytes) indexed by the code nibble, in units
// of the grid's spacing unit u: E1M2 u = 1/4 (levels k/4 -> k), INT4 u = 1,
// E2M1 u = 1/2 (levels {0,.5,1,1.5,2,3,4,6} -> {0,1,2,3,4,6,8,12}).
// lo0/lo1: codes 0..7, hi0/hi1: codes 8..15, little-endian bytes.
struct Lut {
  uint32_t lo0, lo1, hi0, hi1;
  float unit;
};
__device__ __forceinline__ Lut make_lut(int grid) {
  if (grid == 0) return {0x03020100u, 0x07060504u, 0xFDFEFF00u, 0xF9FAFBFCu, 0.25f};  // +k, -(c&7)
  if (grid == 1) return {0x03020100u, 0x07060504u, 0xFBFAF9F8u, 0xFFFEFDFCu, 1.0f};   // two's compl.
  return {0x03020100u, 0x0C080604u, 0xFDFEFF00u, 0xF4F8FAFCu, 0.5f};                  // E2M1 x2
}

// 8 code nibbles (one dword) -> 8 signed level bytes (two dwords: elements
// 0,2,4,6 and 1,3,5,7).
__device__ __forceinline__ void decode_bytes(uint32_t w, const Lut& L, uint32_t& even,
                                             uint32_t& odd) {
  const uint32_t lo = w & 0x0F0F0F0Fu;          // nibbles 0,2,4,6 -> bytes
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;   // nibbles 1,3,5,7 -> bytes
  const uint32_t sl = lo & 0x07070707u, sh = hi & 0x07070707u;
  const uint32_t pl = __builtin_amdgcn_perm(L.lo1, L.lo0, sl);
  const uint32_t nl = __builtin_amdgcn_perm(L.hi1, L.hi0, sl);
  const uint32_t ph = __builtin_amdgcn_perm(L.lo1, L.lo0, sh);
  const uint32_t nh = __builtin_amdgcn_perm(L.hi1, L.hi0, sh);
  const uint32_t ml = ((lo >> 3) & 0x01010101u) * 0xFFu;  // 0xFF where the code is >= 8
  const uint32_t mh = ((hi >> 3) & 0x01010101u) * 0xFFu;
  even = (nl & ml) | (pl & ~ml);
  odd = (nh & mh) | (ph & ~mh);
}

__device__ __forceinline__ float sbyte(uint32_t w, int i) {
  return (float)(int)(int8_t)(uint8_t)(w >> (8 * i));
}

__device__ __forceinline__ uint32_t bf16_bits(float x) {
  const __bf16 h = (__bf16)x;  // round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

// Decode 16 codes (two dwords) with scale s into 2 chunks of 8 bf16 (hi, lo).
__device__ __forceinline__ void decode16(uint32_t w0, uint32_t w1, float s, const Lut& L,
                                         uint4 (&hi)[2], uint4 (&lo)[2]) {
  const float su = s * L.unit;
  float d[16];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t ev, od;
    decode_bytes(h ? w1 : w0, L, ev, od);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      d[8 * h + 2 * i] = sbyte(ev, i) * su;
      d[8 * h + 2 * i + 1] = sbyte(od, i) * su;
    }
  }
  uint32_t hb[16], lb[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    hb[i] = bf16_bits(d[i]);
    lb[i] = bf16_bits(d[i] - __uint_as_float(hb[i] << 16));
  }
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    hi[c] = make_uint4(hb[8 * c] | (hb[8 * c + 1] << 16), hb[8 * c + 2] | (hb[8 * c + 3] << 16),
                       hb[8 * c + 4] | (hb[8 * c + 5] << 16), hb[8 * c + 6] | (hb[8 * c + 7] << 16));
    lo[c] = make_uint4(lb[8 * c] | (lb[8 * c + 1] << 16), lb[8 * c + 2] | (lb[8 * c + 3] << 16),
                       lb[8 * c + 4] | (lb[8 * c + 5] << 16), lb[8 * c + 6] | (lb[8 * c + 7] << 16));
  }
}

struct Fetch {
  uint2 a, b;
  float sa, sb;
};

__device__ __forceinline__ float load_scale(const void* scales, int smode, int br, int bc,
                                            int64_t row, int64_t k, int64_t K) {
  if (smode == 0) {
    return reinterpret_cast<const float*>(scales)[row * (K / bc) + k / bc];
  }
  const uint8_t e = reinterpret_cast<const uint8_t*>(scales)[(row / br) * (K / bc) + k / bc];
  return ldexpf(1.0f, (int)e - 127);
}

// This thread's share of one K step: row = tid/2 of the tile, 16 codes at
// k = k0 + 16*(tid&1).
__device__ __forceinline__ void fetch(const GemmLaunch& g, const Problem& pr, int64_t rowA,
                                      int64_t rowB, int64_t k, Fetch& f) {
  f.a = make_uint2(0, 0); f.b = make_uint2(0, 0); f.sa = 0.0f; f.sb = 0.0f;
  if (k < pr.K) {
    if (rowA < pr.a_rows) {
      const int64_t r = pr.a_row0 + rowA;
      f.a = *reinterpret_cast<const uint2*>(pr.a_codes + r * (pr.K / 2) + k / 2);
      f.sa = load_scale(pr.a_scales, g.scale_mode, g.a_br, g.a_bc, r, k, pr.K);
    }
    if (rowB < pr.b_rows) {
      const int64_t r = pr.b_row0 + rowB;
      f.b = *reinterpret_cast<const uint2*>(pr.b_codes + r * (pr.K / 2) + k / 2);
      f.sb = load_scale(pr.b_scales, g.scale_mode, g.b_br, g.b_bc, r, k, pr.K);
    }
  }
}

__device__ __forceinline__ void stage(uint4* lds, int st, int row, int half, const Fetch& f,
                                      const Lut& L) {
  uint4 hi[2], lo[2];
  uint4* base = lds + st * (kParts * kChunks * TM);
  decode16(f.a.x, f.a.y, f.sa, L, hi, lo);
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    base[(0 * kChunks + 2 * half + c) * TM + row] = hi[c];
    base[(1 * kChunks + 2 * half + c) * TM + row] = lo[c];
  }
  decode16(f.b.x, f.b.y, f.sb, L, hi, lo);
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    base[(2 * kChunks + 2 * half + c) * TM + row] = hi[c];
    base[(3 * kChunks + 2 * half + c) * TM + row] = lo[c];
  }
}

__global__ __launch_bounds__(kThreads) void k_gemm(GemmLaunch g) {
  extern __shared__ uint4 lds[];
  int tm, tn;
  const Problem pr = resolve(g, blockIdx.x, tm, tn);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;   // 2 x 4 waves
  const Lut L = make_lut(g.grid);

  const int frow = tid >> 1, fhalf = tid & 1;
  const int64_t rowA = (int64_t)tm * TM + frow;
  const int64_t rowB = (int64_t)tn * TN + frow;
  const int nsteps = (int)((pr.K + TK - 1) / TK);

  floatx16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = floatx16{};

  Fetch f;
  fetch(g, pr, rowA, rowB, (int64_t)fhalf * 16, f);
  stage(lds, 0, frow, fhalf, f, L);
  __syncthreads();

  for (int step = 0; step < nsteps; ++step) {
    const int st = step & 1;
    const bool more = step + 1 < nsteps;
    if (more) fetch(g, pr, rowA, rowB, (int64_t)(step + 1) * TK + fhalf * 16, f);

    const uint4* base = lds + st * (kParts * kChunks * TM);
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const int chunk = 2 * kh + (lane >> 5);
      bf16x8 ah[4], al[4], bh[2], bl[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wm * 128 + i * 32 + (lane & 31);
        ah[i] = __builtin_bit_cast(bf16x8, base[(0 * kChunks + chunk) * TM + r]);
        al[i] = __builtin_bit_cast(bf16x8, base[(1 * kChunks + chunk) * TM + r]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = wn * 64 + j * 32 + (lane & 31);
        bh[j] = __builtin_bit_cast(bf16x8, base[(2 * kChunks + chunk) * TM + r]);
        bl[j] = __builtin_bit_cast(bf16x8, base[(3 * kChunks + chunk) * TM + r]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], bh[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], bl[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[i], bh[j], acc[i][j], 0, 0, 0);
        }
    }
    if (more) stage(lds, st ^ 1, frow, fhalf, f, L);
    __syncthreads();
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
    hipError_t e = hipFuncSetAttribute((const void*)k_gemm,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(k_gemm, dim3(g.total_tiles), dim3(kThreads), kLdsBytes, s, g);
  return hipGetLastError();
}

}  // namespace ufp4
