// Block-scaled 4-bit GEMM with fp32 block scales (1 x 16 or 1 x 32 blocks):
// C[p][q] = sum_k A[p][k] * B[q][k], the products of the dequantized
// operands accumulated in fp32 on the bf16 matrix cores.
//
// [UFP4] = "Rethinking Shrinkage Bias in FP4 Pretraining of LLMs ... the UFP4
// Recipe" (hyper.ai summary: formats and blockwise quantization -- a block's
// elements are its scale times a codebook level; Method: both GEMM operands
// are quantized in the rotated basis and contracted directly).
//
// Arithmetic ("split-bf16"): every operand element is dequantized to the
// oracle's fp32 value d = RN(level * s), split into bf16 hi = RN(d) and
// lo = RN(d - hi) (the residual d - hi is exact), and C accumulates
// hi*hi + hi*lo + lo*hi with v_mfma_f32_32x32x16_bf16.  The dropped lo*lo term
// and the rounding of lo leave about 2^-16 relative error per product.
//
// Data flow (this kernel, 1 x 16 or 1 x 32 fp32-scale blocks): the packed
// codes and the fp32 scales are copied HBM -> LDS untouched by buffer_load ...
// lds (M0-based direct loads; four lanes per 64-byte code row, chunks
// XOR-swizzled), two raw stages of 128 K elements.  Each thread decodes one A
// row and one B row per 16-wide K step into a decoded double buffer
// [A_hi, A_lo, B_hi, B_lo][8-element half][row] x 16 B (32 KiB each), so
// every element is decoded once per tile; the waves read their MFMA fragments
// from it.  Step i: 24 MFMAs with the decode of step i+1 interleaved (one
// MFMA, then up to 8 VALU), one barrier, the fragment reads of step i+1, the
// other 24 MFMAs.
//
// Tiling: 256 x 256 output tile per 256-thread workgroup, 2 x 2 waves of
// 128 x 128 (4 x 4 tiles of 32 x 32, accumulators in AGPRs).  Dense launches
// order tiles so that the tiles resident at once on an XCD share operand
// strips in its L2.  K need only be a multiple of 16: k-blocks past K get a
// zero scale, and rows past the operand read as zeros (buffer bound).
#include "ufp4_internal.h"
#include "gemm_epilogue.h"

namespace ufp4 {

namespace {

constexpr int TM = 256, TN = 256, KST = 128;   // tile, K elements per LDS stage
constexpr int kThreads = 256, NRAW = 2;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int sgpr4 __attribute__((ext_vector_type(4)));

// --- codebook decode -------------------------------------------------------
// Codes become offset-binary bytes u with level = (u - bias) * unit, bias a
// power of two so that -bias * s * unit is exact:
//   INT4 (two's complement nibble):  u = c ^ 8                    (bias 8)
//   E1M2 (sign-magnitude, unit 1/4): u = 8 + k or 8 - k           (bias 8)
//   E2M1 (sign-magnitude, unit 1/2): u = 16 +- {0,1,2,3,4,6,8,12} (bias 16)
// and d = fma(u, s*unit, -bias*s*unit) = RN(level * s).
template <int GRID> struct Dec;
template <> struct Dec<0> { static constexpr float unit = 0.25f, bias = 8.0f; };
template <> struct Dec<1> { static constexpr float unit = 1.0f, bias = 8.0f; };
template <> struct Dec<2> { static constexpr float unit = 0.5f, bias = 16.0f; };

// 8 code nibbles (element j at bits 4j) -> offset-binary bytes of elements
// 0, 2, 4, 6 (ev) and 1, 3, 5, 7 (od).
template <int GRID>
__device__ __forceinline__ void decode8(uint32_t w, uint32_t& ev, uint32_t& od) {
  if constexpr (GRID == 1) {
    const uint32_t x = w ^ 0x88888888u;
    ev = x & 0x0F0F0F0Fu;
    od = (x >> 4) & 0x0F0F0F0Fu;
  } else if constexpr (GRID == 0) {
    const uint32_t sgn = w & 0x88888888u;
    const uint32_t neg7 = sgn - (sgn >> 3);   // 7 in the negative nibbles
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
      const uint32_t m = (b << 8) - b;   // 0xFF in negative bytes
      return (neg & m) | (pos & ~m);
    };
    ev = map(lo);
    od = map(hi);
  }
}

__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};   // round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

// Selector pairs (-1, 0) and (0, -1) for the exact residual dot products,
// kept in registers (as packed bf16 they must not become inline constants).
struct ResidualMasks {
  bf16x2 m0, m1;
};
__device__ __forceinline__ ResidualMasks make_masks() {
  uint32_t a = 0x0000BF80u, b = 0xBF800000u;
  asm volatile("" : "+s"(a), "+s"(b));
  return {__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b)};
}

// One MFMA fragment: 8 consecutive elements (one code dword) with scale s
// -> bf16 hi and lo.
template <int GRID>
__device__ __forceinline__ void decode_frag(uint32_t w, float s, const ResidualMasks& rm,
                                            bf16x8& hi, bf16x8& lo) {
  const float su = s * Dec<GRID>::unit;
  const float nb = -Dec<GRID>::bias * su;
  uint32_t ev, od, h[4], l[4];
  decode8<GRID>(w, ev, od);
  // opaque to the compiler, so each byte converts with one v_cvt_f32_ubyteN
  // instead of a bit-field extract plus a conversion
  asm("" : "+v"(ev), "+v"(od));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float d0 = __fmaf_rn((float)((ev >> (8 * i)) & 0xFFu), su, nb);
    const float d1 = __fmaf_rn((float)((od >> (8 * i)) & 0xFFu), su, nb);
    h[i] = pk_bf16(d0, d1);
    const bf16x2 hh = __builtin_bit_cast(bf16x2, h[i]);
    const float r0 = __builtin_amdgcn_fdot2_f32_bf16(hh, rm.m0, d0, false);   // d0 - hi0
    const float r1 = __builtin_amdgcn_fdot2_f32_bf16(hh, rm.m1, d1, false);   // d1 - hi1
    l[i] = pk_bf16(r0, r1);
  }
  hi = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
  lo = __builtin_bit_cast(bf16x8, make_uint4(l[0], l[1], l[2], l[3]));
}

// --- direct HBM -> LDS loads -----------------------------------------------
__device__ __forceinline__ sgpr4 rsrc4(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  sgpr4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xFFFF);   // stride 0
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}

// Lane i's 16 bytes land at LDS address lds_addr + 16 i (M0 holds the base).
__device__ __forceinline__ void lds_load16(uint32_t lds_addr, const sgpr4& r, uint32_t voff,
                                           uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(r),
                 "s"(__builtin_amdgcn_readfirstlane(soff))
               : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Codes: [row][64 B] per operand and stage, 16-byte chunks XOR-swizzled by
// (row >> 1) & 3.  Scales: [row][SB bytes] (SB = 32 for 1 x 16 blocks, 16 for
// 1 x 32), unswizzled.
__device__ __forceinline__ uint32_t code_off(int row, int c) {
  return (uint32_t)(row * 64 + 16 * (c ^ ((row >> 1) & 3)));
}

template <int BC> struct Layout {
  static constexpr int SB = (KST / BC) * 4;                // scale bytes per row per stage
  static constexpr int CODES = 2 * TM * 64;                // A then B
  static constexpr int SCALES = 2 * TM * SB;
  static constexpr int RAW = CODES + SCALES;               // one raw stage
  static constexpr int SCALE_LOADS = TM * SB / 1024;       // wave loads per operand
  static constexpr int VMEM = 2 * 4 + 2 * SCALE_LOADS / 4;  // loads per wave per raw stage
  // decoded buffer: [A_hi, A_lo, B_hi, B_lo][8-element half][row] x 16 B
  static constexpr int HL = 4 * 2 * TM * 16;               // 32 KiB
  static constexpr int TOTAL = NRAW * RAW + 2 * HL;
};

struct RdCtx {
  sgpr4 ra, rb, rsa, rsb;
  uint32_t lds0;
  uint32_t code_voff[4];     // wave load q: row * (K/2) + 16 * chunk
  uint32_t scale_voff[2];    // wave load q of the scales
  int wave, nst;
};

template <int BC>
__device__ __forceinline__ void issue_stage(const RdCtx& c, int stage, int slot) {
  using L = Layout<BC>;
  const int s = stage < c.nst ? stage : c.nst - 1;   // past the end: re-read, unused
  const uint32_t base = c.lds0 + (uint32_t)slot * L::RAW;
  const uint32_t koff = (uint32_t)s * 64u;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t blk = (uint32_t)(c.wave * 4 + q) * 1024u;   // 16 rows x 64 B
    lds_load16(base + blk, c.ra, c.code_voff[q], koff);
    lds_load16(base + TM * 64 + blk, c.rb, c.code_voff[q], koff);
  }
  const uint32_t soff = (uint32_t)s * L::SB;
#pragma unroll
  for (int q = 0; q < L::SCALE_LOADS / 4; ++q) {
    const uint32_t blk = (uint32_t)(c.wave * (L::SCALE_LOADS / 4) + q) * 1024u;
    lds_load16(base + L::CODES + blk, c.rsa, c.scale_voff[q], soff);
    lds_load16(base + L::CODES + TM * L::SB + blk, c.rsb, c.scale_voff[q], soff);
  }
}

// Raw inputs of one row of operand `op` (0 A, 1 B) for 16-wide K step j
// (0..7) of the raw stage at `raw`: two code dwords (elements 16 j .. +15)
// and the block scale (zero past K).
struct RawRow {
  uint2 w;
  float s;
};

template <int BC>
__device__ __forceinline__ RawRow read_row(const uint8_t* raw, int op, int row, int j,
                                           bool valid) {
  using L = Layout<BC>;
  RawRow r;
  r.w = *reinterpret_cast<const uint2*>(raw + op * TM * 64 + code_off(row, j >> 1) + 8 * (j & 1));
  const float sc = *reinterpret_cast<const float*>(raw + L::CODES + op * TM * L::SB + row * L::SB +
                                                   4 * ((j * 16) / BC));
  r.s = valid ? sc : 0.0f;
  return r;
}

// Decode half `hf` (8 elements) of a raw row into the decoded buffer `hl`.
template <int GRID>
__device__ __forceinline__ void decode_half(const RawRow& r, uint8_t* hl, int op, int row, int hf,
                                            const ResidualMasks& rm) {
  bf16x8 hi, lo;
  decode_frag<GRID>(hf ? r.w.y : r.w.x, r.s, rm, hi, lo);
  uint8_t* base = hl + op * 2 * (2 * TM * 16);
  *reinterpret_cast<bf16x8*>(base + (hf * TM + row) * 16) = hi;
  *reinterpret_cast<bf16x8*>(base + ((2 + hf) * TM + row) * 16) = lo;
}

template <int GRID, int BC>
__device__ __forceinline__ void decode_row(const uint8_t* raw, uint8_t* hl, int op, int row,
                                           int j, bool valid, const ResidualMasks& rm) {
  const RawRow r = read_row<BC>(raw, op, row, j, valid);
  decode_half<GRID>(r, hl, op, row, 0, rm);
  decode_half<GRID>(r, hl, op, row, 1, rm);
}

struct Frags {
  bf16x8 ah[4], al[4], bh[4], bl[4];
};

__device__ __forceinline__ void load_frags(const uint8_t* hl, int lane, int wm, int wn, Frags& f) {
  const int h = lane >> 5;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int ra = wm * 128 + t * 32 + (lane & 31);
    const int rb = wn * 128 + t * 32 + (lane & 31);
    f.ah[t] = *reinterpret_cast<const bf16x8*>(hl + ((0 + h) * TM + ra) * 16);
    f.al[t] = *reinterpret_cast<const bf16x8*>(hl + ((2 + h) * TM + ra) * 16);
    f.bh[t] = *reinterpret_cast<const bf16x8*>(hl + 4 * TM * 16 + ((0 + h) * TM + rb) * 16);
    f.bl[t] = *reinterpret_cast<const bf16x8*>(hl + 4 * TM * 16 + ((2 + h) * TM + rb) * 16);
  }
}

__device__ __forceinline__ void mfma_step(floatx16 (&acc)[4][4], const Frags& f, int m) {
  const int prod = m >> 4, i = (m >> 2) & 3, j = m & 3;   // hh, hl, lh
  const bf16x8 a = prod == 2 ? f.al[i] : f.ah[i];
  const bf16x8 b = prod == 1 ? f.bl[j] : f.bh[j];
  acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i][j], 0, 0, 0);
}

struct Operands {
  const uint8_t* a_codes;
  const uint8_t* b_codes;
  const float* a_scales;
  const float* b_scales;
  float* c;
  int64_t a_rows, b_rows, K;   // this problem's extents
};

// The problem a tile belongs to (dense, grouped along A's rows, or grouped
// along K) and the tile's coordinates inside it.
__device__ __forceinline__ Operands resolve(const GemmLaunch& g, int tile, int& tm, int& tn) {
  int grp = 0;
  while (grp + 1 < g.ngroups && g.tile_start[grp + 1] <= tile) ++grp;
  const int local = tile - g.tile_start[grp];
  Operands o;
  const float* sa = reinterpret_cast<const float*>(g.a_scales);
  const float* sb = reinterpret_cast<const float*>(g.b_scales);
  if (g.mode == 0) {
    o.a_codes = g.a_codes; o.b_codes = g.b_codes; o.a_scales = sa; o.b_scales = sb;
    o.a_rows = g.PA; o.b_rows = g.PB; o.K = g.K; o.c = g.c;
  } else if (g.mode == 1) {
    // rows [off[grp], off[grp+1]) of A against rows grp*R .. of B
    const int64_t r0 = g.off[grp], rb0 = (int64_t)grp * g.b_rows_per_group;
    o.a_codes = g.a_codes + r0 * (g.K / 2);
    o.b_codes = g.b_codes + rb0 * (g.K / 2);
    o.a_scales = sa + r0 * (g.K / g.a_bc);
    o.b_scales = sb + rb0 * (g.K / g.b_bc);
    o.a_rows = g.off[grp + 1] - r0; o.b_rows = g.b_rows_per_group; o.K = g.K;
    o.c = g.c + r0 * g.ldc;
  } else {
    // segment grp of both operands: K = segment length, stored [P][L] at
    // element offset P * off[grp]
    const int64_t e = g.off[grp], L = g.off[grp + 1] - g.off[grp];
    o.a_codes = g.a_codes + (g.PA * e) / 2;
    o.b_codes = g.b_codes + (g.PB * e) / 2;
    o.a_scales = sa + (g.PA * e) / g.a_bc;
    o.b_scales = sb + (g.PB * e) / g.b_bc;
    o.a_rows = g.PA; o.b_rows = g.PB; o.K = L;
    o.c = g.c + (int64_t)grp * g.PA * g.ldc;
  }
  const int tiles_n = (int)((o.b_rows + TN - 1) / TN);
  tm = local / (tiles_n > 0 ? tiles_n : 1);
  tn = local - tm * tiles_n;
  return o;
}

template <int GRID, int BC>
__global__ __launch_bounds__(kThreads) void k_gemm_rd(GemmLaunch g) {
  using L = Layout<BC>;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

  int tm, tn;
  const Operands o = resolve(g, blockIdx.x, tm, tn);
  if (g.mode == 0)   // one dense problem: XCD-aware grouped order
    tile_order(blockIdx.x, g.total_tiles, (int)((o.a_rows + TM - 1) / TM),
               (int)((o.b_rows + TN - 1) / TN), tm, tn);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t K = o.K;
  const int64_t row0 = (int64_t)tm * TM, col0 = (int64_t)tn * TN;
  const int64_t rows_a = o.a_rows - row0 < TM ? o.a_rows - row0 : TM;
  const int64_t rows_b = o.b_rows - col0 < TN ? o.b_rows - col0 : TN;
  const int nkb = (int)(K / BC);
  const uint32_t rs = (uint32_t)(K / 2), srs = (uint32_t)(K / BC) * 4u;

  RdCtx c;
  c.wave = wave;
  c.nst = (int)((K + KST - 1) / KST);
  c.ra = rsrc4(o.a_codes + row0 * rs, (uint32_t)(rows_a * rs));
  c.rb = rsrc4(o.b_codes + col0 * rs, (uint32_t)(rows_b * rs));
  c.rsa = rsrc4(reinterpret_cast<const uint8_t*>(o.a_scales) + row0 * srs, (uint32_t)(rows_a * srs));
  c.rsb = rsrc4(reinterpret_cast<const uint8_t*>(o.b_scales) + col0 * srs, (uint32_t)(rows_b * srs));
  c.lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)lds;
  {
    // codes: lane i of wave load q -> row 64 w + 16 q + i / 4, the chunk whose
    // swizzled slot is i % 4
    const int lr = lane >> 2;
    const uint32_t chunk = (uint32_t)((lane & 3) ^ ((lr >> 1) & 3));
#pragma unroll
    for (int q = 0; q < 4; ++q) c.code_voff[q] = (uint32_t)(wave * 64 + q * 16 + lr) * rs + 16u * chunk;
    // scales: a wave load is 1 KiB = 1024 / SB rows; lane i -> row i / (SB/16), part i % (SB/16)
    constexpr int PER = L::SB / 16;
    constexpr int ROWS = 64 / PER;
#pragma unroll
    for (int q = 0; q < L::SCALE_LOADS / 4; ++q) {
      const int row = (wave * (L::SCALE_LOADS / 4) + q) * ROWS + lane / PER;
      c.scale_voff[q] = (uint32_t)row * srs + 16u * (uint32_t)(lane % PER);
    }
  }
  const ResidualMasks rm = make_masks();
  uint8_t* hlb = lds + NRAW * L::RAW;   // two decoded buffers

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx16{};

  const int nsteps = (int)(K / 16);
  if (nsteps > 0) {
    issue_stage<BC>(c, 0, 0);
    issue_stage<BC>(c, 1, 1);
    wait_vmcnt<L::VMEM>();
    __syncthreads();
    decode_row<GRID, BC>(lds, hlb, 0, tid, 0, 0 < nkb, rm);
    decode_row<GRID, BC>(lds, hlb, 1, tid, 0, 0 < nkb, rm);
    __syncthreads();
    // Step i (fragments F of step i in registers):
    //   24 MFMAs of step i, while this thread decodes its A and B rows of
    //   step i+1 into the other decoded buffer;
    //   barrier (step i+1 fully decoded; every wave has read step i's buffer);
    //   fragment reads of step i+1, in flight during the other 24 MFMAs of step i.
    // Raw stage s (8 steps) is issued at step 8 (s - 1) and waited for two
    // steps before its first decode.
    Frags f, fn;
    load_frags(hlb, lane, wm, wn, f);
    for (int i = 0; i < nsteps; ++i) {
      if (i > 0 && (i & 7) == 0) issue_stage<BC>(c, (i >> 3) + 1, ((i >> 3) + 1) & 1);
      const int n = i + 1;                                   // step being decoded
      const uint8_t* raw = lds + ((n >> 3) & 1) * L::RAW;
      const bool vn = n < nsteps && (n * 16) / BC < nkb;
      uint8_t* hn = hlb + (n & 1) * L::HL;
      const RawRow ra = read_row<BC>(raw, 0, tid, n & 7, vn);
      const RawRow rb = read_row<BC>(raw, 1, tid, n & 7, vn);
      // four 8-element decodes, each spread over five MFMAs
#pragma unroll
      for (int p = 0; p < 4; ++p) {
#pragma unroll
        for (int m = 5 * p; m < 5 * p + 5; ++m) mfma_step(acc, f, m);
        decode_half<GRID>(p < 2 ? ra : rb, hn, p >> 1, tid, p & 1, rm);
#pragma unroll
        for (int q = 0; q < 5; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);   // then up to 8 VALU
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int m = 20; m < 24; ++m) mfma_step(acc, f, m);
      if (((i + 2) & 7) == 0) wait_vmcnt<0>();   // raw stage of step i+2 has landed
      __syncthreads();
      load_frags(hn, lane, wm, wn, fn);
#pragma unroll
      for (int m = 24; m < 48; ++m) mfma_step(acc, f, m);
      f = fn;
    }
  }

  store_c<4, 4>(o.c + row0 * g.ldc + col0, g.ldc, (int)rows_a, (int)rows_b, wm * 128, wn * 128,
                lane, acc);
}

template <int GRID, int BC>
hipError_t launch_rd(const GemmLaunch& g, hipStream_t s) {
  constexpr int bytes = Layout<BC>::TOTAL;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)k_gemm_rd<GRID, BC>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((k_gemm_rd<GRID, BC>), dim3(g.total_tiles), dim3(kThreads), bytes, s, g);
  return hipGetLastError();
}

}  // namespace

bool gemm_rd_supported(const GemmLaunch& g) {
  return g.scale_mode == 0 && g.a_br == 1 && g.b_br == 1 && g.a_bc == g.b_bc &&
         (g.a_bc == 16 || g.a_bc == 32) && g.K % 16 == 0 &&
         (g.K / 2) * (int64_t)TM <= INT32_MAX;
}

hipError_t launch_gemm_rd(const GemmLaunch& g, hipStream_t s) {
  if (g.total_tiles == 0) return hipSuccess;
  const int key = g.grid * 2 + (g.a_bc == 32 ? 1 : 0);
  switch (key) {
    case 0: return launch_rd<0, 16>(g, s);
    case 1: return launch_rd<0, 32>(g, s);
    case 2: return launch_rd<1, 16>(g, s);
    case 3: return launch_rd<1, 32>(g, s);
    case 4: return launch_rd<2, 16>(g, s);
    default: return launch_rd<2, 32>(g, s);
  }
}

}  // namespace ufp4
