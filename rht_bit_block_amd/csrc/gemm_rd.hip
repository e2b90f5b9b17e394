// Block-scaled 4-bit GEMM with fp32 block scales (1 x 16 or 1 x 32 blocks):
// C[p][q] = sum_k dA[p][k] * dB[q][k], d = level * s, accumulated in fp32.
//
// [UFP4] = "Rethinking Shrinkage Bias in FP4 Pretraining of LLMs ... the UFP4
// Recipe" (hyper.ai summary: formats and blockwise quantization -- a block's
// elements are its scale times a codebook level; Method: both GEMM operands
// are quantized in the rotated basis and contracted directly).
//
// Arithmetic ("scale product").  Inside one 16-wide K step every element of
// a row shares one block scale, so
//   sum_k dA[p][k] dB[q][k] = (sA[p] sB[q]) * sum_k lA[p][k] lB[q][k].
// The level dot products P come from v_mfma_f32_32x32x16_fp8_fp8 on the
// levels as E4M3 bytes: every level of the three codebooks is an E4M3 number,
// so P is exact in fp32.  The scale products S come from a second MFMA on
// bf16 pieces of the scales: s = s0 + s1 + s2 exactly (s0 = bf16(s),
// s1 = bf16(s - s0), s2 = s - s0 - s1), and the eight K slots pair six of the
// nine cross products (all but s1 t2, s2 t1, s2 t2, each below 2^-25 of s t).
// That MFMA is v_mfma_f32_32x32x8_bf16: lane half h supplies slots 4h .. 4h + 3
// (two registers per operand).  C += P * S
// is one fp32 fma per element.  The result differs from the exact one by fp32
// rounding only (a few 2^-24 relative per step).
//
// Both MFMAs take fresh accumulators and are independent: a step costs two
// MFMAs and 16 fmas per 32 x 32 tile, and the two units work side by side
// within a wave (fmas of tile t while the products of tile t+1 execute) and
// across the two waves of a SIMD.
//
// Data flow: the packed codes and the fp32 scales are copied HBM -> LDS
// untouched by buffer_load ... lds (M0-based direct loads; four lanes per
// 64-byte code row, chunks XOR-swizzled), two raw stages of 128 K elements.
// Per 16-wide K step, each of the 512 threads turns one A or B row into a
// decoded double buffer: the row's 16 E4M3 levels, [op][K half][row] x 8 B,
// and its bf16 scale pieces, [op][row] x 16 B.  Lanes of the upper half read
// a zero slot for the scale operand.  Within a step the order of the K
// elements does not change the sum, so a K half holds its even elements then
// its odd ones, the same for A and B.
//
// Pipeline of step i (its fragments in registers): the decode of step i+2
// during the first two tiles (its raw inputs were read from LDS during step i-1)
// into one of four decoded buffers, a barrier on even steps, then the
// fragments of step i+1 are read as registers free up, so the LDS reads of a
// step are hidden under the tiles of the one before.
// Inside a step the 16-wide kernel walks its 8 tiles column by column; both
// products are double-buffered, and the products of tile t+1 are issued
// around the first half of tile t's fmas (level product, 8 fmas, scale
// product, 8 fmas, in that order), so no fma waits on an MFMA issued just
// before it; each operand fragment is reloaded right after its last product
// is issued.
//
// With 1 x 32 blocks one scale covers two 16-wide halves, so k_gemm_rd32
// takes 32-wide steps: two chained level MFMAs, one scale product and one set
// of fmas per tile and step.
//
// Tiling: 256 x 256 output tile per 512-thread workgroup, 2 x 4 waves of
// 128 x 64 (4 x 2 tiles of 32 x 32, accumulators in VGPRs).  Every launch
// gives each XCD a contiguous range of tiles in grouped order, so the tiles
// resident at once on an XCD share operand strips in its L2.  Rows past the
// operand read as zeros (buffer bound).
//
// Last round: one workgroup per CU fits (160 KiB of LDS), so a launch of T
// tiles runs in rounds of CU-count workgroups.  When the last round would be
// at most half full and the tiles are long (1024 K elements or more on
// average), each of its tiles is computed by two workgroups, one per half of
// K (split on a 128-element stage boundary), so the round keeps every CU
// busy for half as long.  Both halves add their fp32 partial sums into C,
// which a fill kernel has zeroed: with two addends on an exact zero the sum
// is the same in either order, so the result does not depend on timing (it
// is the rounding of P_first + P_second instead of one running sum).
#include "ufp4_internal.h"
#include "gemm_epilogue.h"

namespace ufp4 {

namespace {

constexpr int TM = 256, TN = 256, KST = 128;   // tile, K elements per LDS stage
constexpr int kThreads = 512, NRAW = 2;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int sgpr4 __attribute__((ext_vector_type(4)));

// --- codes -> E4M3 levels ------------------------------------------------------
// E4M3 bytes of the codebook magnitudes 0..7 (byte i = magnitude index i):
//   E1M2 levels k/4:                 0, .25, .5, .75, 1, 1.25, 1.5, 1.75
//   E2M1 levels:                     0, .5, 1, 1.5, 2, 3, 4, 6
// and for INT4 (two's complement) the values of nibbles 0..7 and 8..15:
//   0..7 and -8..-1.
template <int GRID> struct Lut;
template <> struct Lut<0> { static constexpr uint32_t lo = 0x34302800u, hi = 0x3E3C3A38u; };
template <> struct Lut<2> { static constexpr uint32_t lo = 0x3C383000u, hi = 0x4C484440u; };
template <> struct Lut<1> {
  static constexpr uint32_t lo = 0x44403800u, hi = 0x4E4C4A48u;     // 0..7
  static constexpr uint32_t nlo = 0xCACCCED0u, nhi = 0xB8C0C4C8u;   // -8..-1
};

// Nibbles in the low half of each byte of v (bit 3 the sign or the INT4
// high bit) -> E4M3 bytes.
template <int GRID>
__device__ __forceinline__ uint32_t nib_to_e4m3(uint32_t v) {
  const uint32_t m = v & 0x07070707u;
  const uint32_t pos = __builtin_amdgcn_perm(Lut<GRID>::hi, Lut<GRID>::lo, m);
  if constexpr (GRID == 1) {
    const uint32_t neg = __builtin_amdgcn_perm(Lut<1>::nhi, Lut<1>::nlo, m);
    // byte i from pos (selector i) or, where the nibble's bit 3 is set, from
    // neg (selector i + 4)
    const uint32_t sel = ((v >> 1) & 0x04040404u) | 0x03020100u;
    return __builtin_amdgcn_perm(neg, pos, sel);
  } else {
    return pos | ((v & 0x08080808u) << 4);
  }
}

// 8 code nibbles (element j at bits 4j) -> {E4M3 of elements 0, 2, 4, 6;
// E4M3 of elements 1, 3, 5, 7}.
template <int GRID>
__device__ __forceinline__ uint2 levels8(uint32_t w) {
  return make_uint2(nib_to_e4m3<GRID>(w & 0x0F0F0F0Fu), nib_to_e4m3<GRID>((w >> 4) & 0x0F0F0F0Fu));
}

__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};   // round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

// bf16 pieces of a block scale for the scale-product MFMA: s = s0 + s1 + s2
// (each rounding leaves an exact fp32 residual).  K slots 0..7, A side x B
// side:
//   A: s0 s0 s0 s1 s1 s2 0 0        B: t0 t1 t2 t0 t1 t0 0 0
// sum = s0 (t0 + t1 + t2) + s1 (t0 + t1) + s2 t0.  Both sides' slot pairs are
// byte permutes of [s0 s0] and [s1 s2]; `op` (uniform across the wave) picks
// the selectors, so a wave converts only its own side.
__device__ __forceinline__ uint4 scale_pieces(float s, int op) {
  const uint32_t u0 = pk_bf16(s, s);                        // [s0 s0]
  const float r1 = s - __uint_as_float(u0 << 16);
  const uint32_t u1 = pk_bf16(r1, r1);
  const float r2 = r1 - __uint_as_float(u1 << 16);
  const uint32_t g = pk_bf16(r1, r2);                       // [s1 s2]
  // bytes of {g, u0}: 0-3 = s0 s0, 4-5 = s1, 6-7 = s2
  const uint32_t sel0 = op ? 0x05040100u : 0x01000100u;    // t0 t1 | s0 s0
  const uint32_t sel1 = op ? 0x01000706u : 0x05040100u;    // t2 t0 | s0 s1
  const uint32_t sel2 = op ? 0x01000504u : 0x07060504u;    // t1 t0 | s1 s2
  return make_uint4(__builtin_amdgcn_perm(g, u0, sel0), __builtin_amdgcn_perm(g, u0, sel1),
                    __builtin_amdgcn_perm(g, u0, sel2), 0u);
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
  static constexpr int SB = (KST / BC) * 4;       // scale bytes per row per stage
  static constexpr int CODES = 2 * TM * 64;       // A then B
  static constexpr int SCALES = 2 * TM * SB;
  static constexpr int RAW = CODES + SCALES;      // one raw stage
  static constexpr int SLOADS = SCALES / 1024;    // 1 KiB wave loads of scales
  static constexpr int SPW = SLOADS / 8;          // per wave
  static constexpr int VMEM = 4 + SPW;            // loads per wave per raw stage
  // decoded buffer: levels [op][K half][row] x 8 E4M3, then scale pieces
  // [op][row] x 8 bf16 (lane half h of a fragment reads pieces 4h .. 4h + 3)
  static constexpr int LEV = 2 * 2 * TM * 8;
  static constexpr int PCS = 2 * TM * 16;
  static constexpr int DEC = LEV + PCS;
  static constexpr int TOTAL = NRAW * RAW + 4 * DEC;   // 160 KiB for 1 x 16 blocks
};

struct RdCtx {
  sgpr4 ra, rb, rsa, rsb;
  uint32_t lds0;
  uint32_t code_voff[2];     // wave code load q: row * (K/2) + 16 * chunk
  uint32_t scale_voff[2];    // wave scale load q
  uint32_t rs, srs;          // row strides of the codes and the scales (bytes)
  int wave, nst;
};

// Per-lane byte offsets of a wave's raw-stage loads.  Codes: lane i of wave
// load q -> row 32 w + 16 q + i / 4, the chunk whose swizzled slot is i % 4.
// Scales: wave load g covers 1024 / SB rows of operand g / (SLOADS/2); lane i
// -> row i / (SB/16), part i % (SB/16).
template <int BC>
__device__ __forceinline__ void load_offsets(int wave, uint32_t lane, uint32_t rs, uint32_t srs,
                                             uint32_t* code_voff, uint32_t* scale_voff) {
  using L = Layout<BC>;
  const uint32_t lr = lane >> 2;
  const uint32_t chunk = (lane & 3) ^ ((lr >> 1) & 3);
#pragma unroll
  for (int q = 0; q < 2; ++q) code_voff[q] = ((uint32_t)(wave * 32 + q * 16) + lr) * rs + 16u * chunk;
  constexpr uint32_t PER = L::SB / 16;
  constexpr uint32_t ROWS = 64 / PER;
#pragma unroll
  for (int q = 0; q < L::SPW; ++q) {
    const int gl = wave + 8 * q;
    const uint32_t row = (uint32_t)(gl % (L::SLOADS / 2)) * ROWS + lane / PER;
    scale_voff[q] = row * srs + 16u * (lane % PER);
  }
}

template <int BC>
__device__ __forceinline__ void issue_stage(const RdCtx& c, int stage, int slot) {
  using L = Layout<BC>;
  const int s = stage < c.nst ? stage : c.nst - 1;   // past the end: re-read, unused
  const uint32_t base = c.lds0 + (uint32_t)slot * L::RAW;
  const uint32_t koff = (uint32_t)s * 64u;
  uint32_t cv[2] = {c.code_voff[0], c.code_voff[1]};
  uint32_t sv[2] = {c.scale_voff[0], c.scale_voff[1]};
  if constexpr (BC == 32) {
    // The 32-wide kernel's loop has no register to spare (kept live, these
    // offsets were spilled, and the reload's wait then also waited for the
    // stage's own loads): recompute them from the lane id once per stage.
    uint32_t lane;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
    load_offsets<BC>(c.wave, lane, c.rs, c.srs, cv, sv);
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const uint32_t blk = (uint32_t)(c.wave * 2 + q) * 1024u;   // 16 rows x 64 B
    lds_load16(base + blk, c.ra, cv[q], koff);
    lds_load16(base + TM * 64 + blk, c.rb, cv[q], koff);
  }
  const uint32_t soff = (uint32_t)s * L::SB;
#pragma unroll
  for (int q = 0; q < L::SPW; ++q) {
    const int g = c.wave + 8 * q;                 // scale wave load, A loads first
    const bool is_b = g >= L::SLOADS / 2;
    lds_load16(base + L::CODES + (uint32_t)g * 1024u, is_b ? c.rsb : c.rsa, sv[q], soff);
  }
}

// Raw inputs of one row for one 16-wide K step: two code dwords and the scale.
struct DecIn {
  uint2 w;
  float s;
};

// Row `row` of operand `op` for 16-wide K step j (0..7) of the raw stage `raw`.
template <int BC>
__device__ __forceinline__ DecIn decode_load(const uint8_t* raw, int op, int row, int j) {
  using L = Layout<BC>;
  DecIn d;
  d.w = *reinterpret_cast<const uint2*>(raw + op * TM * 64 + code_off(row, j >> 1) + 8 * (j & 1));
  d.s = *reinterpret_cast<const float*>(raw + L::CODES + op * TM * L::SB + row * L::SB +
                                        4 * ((j * 16) / BC));
  return d;
}

// E4M3 levels and scale pieces of the row into the decoded buffer `dec`.
template <int GRID, int BC>
__device__ __forceinline__ void decode_store(const DecIn& d, uint8_t* dec, int op, int row) {
  using L = Layout<BC>;
  *reinterpret_cast<uint2*>(dec + ((op * 2 + 0) * TM + row) * 8) = levels8<GRID>(d.w.x);
  *reinterpret_cast<uint2*>(dec + ((op * 2 + 1) * TM + row) * 8) = levels8<GRID>(d.w.y);
  *reinterpret_cast<uint4*>(dec + L::LEV + (op * TM + row) * 16) =
      scale_pieces(d.s, op);
}

typedef short short4_t __attribute__((ext_vector_type(4)));

// Operand fragment of the 16-wide kernel: 8 E4M3 levels (level product) and
// the lane half's four scale pieces (scale product).
struct Frag {
  long code;
  short4_t pc;
};

__device__ __forceinline__ Frag frag_at(const uint8_t* dec, uint32_t code_off, uint32_t pc_off) {
  Frag f;
  f.code = *reinterpret_cast<const long*>(dec + code_off);
  f.pc = *reinterpret_cast<const short4_t*>(dec + pc_off);
  return f;
}

__device__ __forceinline__ floatx16 level_product(const Frag& a, const Frag& b) {
  return __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(a.code, b.code, floatx16{}, 0, 0, 0);
}

__device__ __forceinline__ floatx16 scale_product(const Frag& a, const Frag& b) {
  return __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(a.pc, b.pc, floatx16{}, 0, 0, 0);
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
// along K) and the tile's coordinates inside it, each problem in grouped
// order; slot_tile() picks the tile of slot b (XCD-contiguous ranges, or for
// unbalanced K-grouped launches runs of tiles dealt over the XCDs).
__device__ __forceinline__ Operands resolve(const GemmLaunch& g, int b, int& tm, int& tn) {
  int grp, local;
  slot_tile(g, b, grp, local);
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
  const int tiles_m = (int)((o.a_rows + TM - 1) / TM);
  grouped_order(local, tiles_m, tiles_n > 0 ? tiles_n : 1, tm, tn);
  return o;
}

// Per-tile state shared by the 16- and 32-wide kernels: the problem and the
// tile's place in it, and the direct-load context for its raw stages (wave w
// loads code rows 32 w .. 32 w + 31 of both operands and 1 KiB pieces of the
// scales).
struct TileCtx {
  Operands o;
  int64_t row0, col0, rows_a, rows_b;
  int64_t klen;   // K elements this workgroup sums (all of K unless split)
  int half;       // -1, or the K half of a split tile
  RdCtx c;
  int wave, wm, wn;
};

template <int BC>
__device__ __forceinline__ TileCtx tile_ctx(const GemmLaunch& g, const uint8_t* lds, int tid) {
  using L = Layout<BC>;
  TileCtx t;
  int tm, tn;
  // workgroups past split_first come in pairs: slot split_first + j / 2, K half j % 2
  int slot = blockIdx.x;
  t.half = -1;
  if (slot >= g.split_first) {
    const int j = slot - g.split_first;
    slot = g.split_first + (j >> 1);
    t.half = j & 1;
  }
  t.o = resolve(g, slot, tm, tn);
  const int lane = tid & 63;
  t.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  t.wm = t.wave >> 2;
  t.wn = t.wave & 3;
  const int64_t K = t.o.K;   // the operands' row length
  int64_t kbeg = 0;
  t.klen = K;                // this workgroup's part of it
  if (t.half >= 0) {
    const int64_t kh = (K / (2 * KST)) * KST;   // a stage boundary
    kbeg = t.half ? kh : 0;
    t.klen = t.half ? K - kh : kh;
  }
  t.row0 = (int64_t)tm * TM;
  t.col0 = (int64_t)tn * TN;
  t.rows_a = t.o.a_rows - t.row0 < TM ? t.o.a_rows - t.row0 : TM;
  t.rows_b = t.o.b_rows - t.col0 < TN ? t.o.b_rows - t.col0 : TN;
  const uint32_t rs = (uint32_t)(K / 2), srs = (uint32_t)(K / BC) * 4u;
  const uint32_t cb = (uint32_t)(kbeg / 2), sb = (uint32_t)(kbeg / BC) * 4u;   // K offsets
  RdCtx& c = t.c;
  c.wave = t.wave;
  c.nst = (int)((t.klen + KST - 1) / KST);
  c.ra = rsrc4(t.o.a_codes + t.row0 * rs + cb, (uint32_t)(t.rows_a * rs) - cb);
  c.rb = rsrc4(t.o.b_codes + t.col0 * rs + cb, (uint32_t)(t.rows_b * rs) - cb);
  c.rsa = rsrc4(reinterpret_cast<const uint8_t*>(t.o.a_scales) + t.row0 * srs + sb,
                (uint32_t)(t.rows_a * srs) - sb);
  c.rsb = rsrc4(reinterpret_cast<const uint8_t*>(t.o.b_scales) + t.col0 * srs + sb,
                (uint32_t)(t.rows_b * srs) - sb);
  c.lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)lds;
  c.rs = rs;
  c.srs = srs;
  c.scale_voff[1] = 0;
  load_offsets<BC>(t.wave, (uint32_t)lane, rs, srs, c.code_voff, c.scale_voff);
  return t;
}

template <int GRID, int BC>
__global__ __launch_bounds__(kThreads) void k_gemm_rd(GemmLaunch g) {
  using L = Layout<BC>;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

  const int tid = threadIdx.x, lane = tid & 63;
  const TileCtx ts = tile_ctx<BC>(g, lds, tid);
  const RdCtx& c = ts.c;
  const int wave = ts.wave, wm = ts.wm, wn = ts.wn;
  const int64_t K = ts.klen;
  uint8_t* decb = lds + NRAW * L::RAW;   // two decoded buffers

  floatx16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      acc[i][j] = floatx16{};
      asm volatile("" : "+v"(acc[i][j]));   // no peeled first step
    }

  const int nsteps = (int)(K / 16);
  const int h = lane >> 5, r32 = lane & 31;
  const int dop = wave >> 2, drow = tid & (TM - 1);   // the row this thread decodes
  // fragment offsets in a decoded buffer; tile t adds 256 t (levels), 512 t (pieces)
  const uint32_t code_a = (uint32_t)(((0 + h) * TM + wm * 128 + r32) * 8);
  const uint32_t code_b = (uint32_t)(((2 + h) * TM + wn * 64 + r32) * 8);
  const uint32_t pc_a = (uint32_t)(L::LEV + (wm * 128 + r32) * 16 + 8 * h);
  const uint32_t pc_b = (uint32_t)(L::LEV + (TM + wn * 64 + r32) * 16 + 8 * h);
  if (nsteps > 0) {
    issue_stage<BC>(c, 0, 0);
    issue_stage<BC>(c, 1, 1);
    wait_vmcnt<L::VMEM>();
    __syncthreads();
    decode_store<GRID, BC>(decode_load<BC>(lds, dop, drow, 0), decb, dop, drow);
    decode_store<GRID, BC>(decode_load<BC>(lds, dop, drow, 1), decb + L::DEC, dop, drow);
    DecIn dnx = decode_load<BC>(lds, dop, drow, 2);   // step 2 (stage 0 has landed)
    __syncthreads();
    Frag fa[4], fb[2];
#pragma unroll
    for (int t = 0; t < 4; ++t) fa[t] = frag_at(decb, code_a + 256 * t, pc_a + 512 * t);
#pragma unroll
    for (int t = 0; t < 2; ++t) fb[t] = frag_at(decb, code_b + 256 * t, pc_b + 512 * t);
    // Tiles of a step in column order: u = 0..7 is (A tile u & 3, B tile u >> 2).
    // The products of tile u+1 are issued during the fmas of tile u (two sets
    // in flight), the next step's tile 0 during tile 7.  An operand is
    // reloaded for the next step after its last product was issued: fb[0]
    // after u = 2, fa[k] after u = 3 + k, fb[1] after u = 6.
    // Four decoded buffers, step m in buffer m % 4: step i decodes step i+2
    // (levels at u = 0, scale pieces at u = 1, so the decode's VALU work is
    // split over two tiles) and reads the fragments of step i+1 (u >= 3); a
    // barrier on even steps only (u = 2).  Between the decode of step m (step
    // m-2) and its fragment reads (step m-1) lies the barrier of m-2 or m-1,
    // whichever is even; between the last reads of a buffer (step m-5) and its
    // next decode (step m-2) the barrier of m-4 or m-3.  A raw stage is waited
    // for on the even step before its first decode load (step 8 s - 4 for
    // stage s).
    floatx16 p[2], q[2];
    p[0] = level_product(fa[0], fb[0]);
    q[0] = scale_product(fa[0], fb[0]);
#pragma clang loop unroll(disable)
    for (int i = 0; i < nsteps; ++i) {
      if (i > 0 && (i & 7) == 0) issue_stage<BC>(c, (i >> 3) + 1, ((i >> 3) + 1) & 1);
      const int n = i + 2;   // decoded during this step (past the end: unused)
      const DecIn din = dnx;   // step n's raw inputs, loaded during the step before
      const uint8_t* dn = decb + ((i + 1) & 3) * L::DEC;   // fragments of step i+1
      const bool more = i + 1 < nsteps;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        // the next tile's level product, the first half of this tile's fmas,
        // the next tile's scale product, the second half (the scheduling
        // barriers keep this order: left to itself the compiler moves the
        // products to the end of the fmas, and the next tile's fmas then
        // wait for them)
        const Frag& na = u + 1 < 8 ? fa[(u + 1) & 3] : fa[0];
        const Frag& nb = u + 1 < 8 ? fb[(u + 1) >> 2] : fb[0];
        if (u + 1 < 8 || more) p[(u + 1) & 1] = level_product(na, nb);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < 8; ++r)
          acc[u & 3][u >> 2][r] = __builtin_fmaf(p[u & 1][r], q[u & 1][r], acc[u & 3][u >> 2][r]);
        __builtin_amdgcn_sched_barrier(0);
        if (u + 1 < 8 || more) q[(u + 1) & 1] = scale_product(na, nb);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 8; r < 16; ++r)
          acc[u & 3][u >> 2][r] = __builtin_fmaf(p[u & 1][r], q[u & 1][r], acc[u & 3][u >> 2][r]);
        asm volatile("" : "+v"(acc[u & 3][u >> 2]));   // the fmas stay here
        if (u == 0) {   // levels of step i+2 (scale pieces during the next tile)
          uint8_t* dec = decb + (n & 3) * L::DEC;
          *reinterpret_cast<uint2*>(dec + ((dop * 2 + 0) * TM + drow) * 8) = levels8<GRID>(din.w.x);
          *reinterpret_cast<uint2*>(dec + ((dop * 2 + 1) * TM + drow) * 8) = levels8<GRID>(din.w.y);
        }
        if (u == 1) {
          uint8_t* dec = decb + (n & 3) * L::DEC;
          *reinterpret_cast<uint4*>(dec + L::LEV + (dop * TM + drow) * 16) = scale_pieces(din.s, dop);
        }
        if (u == 2) {
          if ((i & 1) == 0) {   // uniform: every wave takes the same barriers
            if (((i + 4) & 7) == 0) wait_vmcnt<0>();   // raw stage of step i+4 has landed
            __syncthreads();
          }
          // raw inputs of step i+3 (its stage has landed for every wave)
          dnx = decode_load<BC>(lds + (((i + 3) >> 3) & 1) * L::RAW, dop, drow, (i + 3) & 7);
        }
        if (u == 3) fb[0] = frag_at(dn, code_b, pc_b);
        if (u >= 4) fa[u - 4] = frag_at(dn, code_a + 256 * (u - 4), pc_a + 512 * (u - 4));
        if (u == 7) fb[1] = frag_at(dn, code_b + 256, pc_b + 512);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  float* ct = ts.o.c + ts.row0 * g.ldc + ts.col0;
  if (ts.half < 0)
    store_c<4, 2>(ct, g.ldc, (int)ts.rows_a, (int)ts.rows_b, wm * 128, wn * 64, lane, acc);
  else
    add_c<4, 2>(ct, g.ldc, (int)ts.rows_a, (int)ts.rows_b, wm * 128, wn * 64, lane, acc);
}

template <int GRID, int BC>
hipError_t launch_rd(const GemmLaunch& g, int grid, hipStream_t s) {
  constexpr int bytes = Layout<BC>::TOTAL;
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t e = set_lds_limit((const void*)k_gemm_rd<GRID, BC>, bytes, lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_gemm_rd<GRID, BC>), dim3(grid), dim3(kThreads), bytes, s, g);
  return hipGetLastError();
}


// --- 1 x 32 blocks: 32-wide K steps -------------------------------------------
// One block scale covers 32 K elements, so a step takes two chained level
// MFMAs (K halves 0-15 and 16-31 of the block), one scale-product MFMA and one
// set of 16 fmas per tile: half the fmas and three quarters of the MFMAs of
// two 16-wide steps.  Decoded buffer: levels [op][16-wide half][K half][row] x
// 8 E4M3, scale pieces [op][row] x 8 bf16 (lane half h reads pieces 4h..4h+3).
struct Layout32 {
  static constexpr int LEV = 2 * 2 * 2 * TM * 8;
  static constexpr int PCS = 2 * TM * 16;
  static constexpr int DEC = LEV + PCS;
  static constexpr int TOTAL = NRAW * Layout<32>::RAW + 2 * DEC;
};

// Raw inputs of one row for one 32-wide K step: four code dwords (elements
// 8 i .. 8 i + 7 in dword i) and the block scale.
struct DecIn32 {
  uint4 w;
  float s;
};

// Row `row` of operand `op` for 32-wide K step j (0..3) of the raw stage `raw`.
__device__ __forceinline__ DecIn32 decode_load32(const uint8_t* raw, int op, int row, int j) {
  using L = Layout<32>;
  DecIn32 d;
  d.w = *reinterpret_cast<const uint4*>(raw + op * TM * 64 + code_off(row, j));
  d.s = *reinterpret_cast<const float*>(raw + L::CODES + op * TM * L::SB + row * L::SB + 4 * j);
  return d;
}

template <int GRID>
__device__ __forceinline__ void decode_store32(const DecIn32& d, uint8_t* dec, int op, int row) {
  using L = Layout32;
  *reinterpret_cast<uint2*>(dec + (((op * 2 + 0) * 2 + 0) * TM + row) * 8) = levels8<GRID>(d.w.x);
  *reinterpret_cast<uint2*>(dec + (((op * 2 + 0) * 2 + 1) * TM + row) * 8) = levels8<GRID>(d.w.y);
  *reinterpret_cast<uint2*>(dec + (((op * 2 + 1) * 2 + 0) * TM + row) * 8) = levels8<GRID>(d.w.z);
  *reinterpret_cast<uint2*>(dec + (((op * 2 + 1) * 2 + 1) * TM + row) * 8) = levels8<GRID>(d.w.w);
  *reinterpret_cast<uint4*>(dec + L::LEV + (op * TM + row) * 16) =
      scale_pieces(d.s, op);
}

struct Frag32 {
  long c0, c1;    // E4M3 levels of the two 16-wide halves
  short4_t pc;    // the lane half's four scale pieces (K = 8 scale product)
};

// code_off: the first half's levels; the second half's are 2 TM x 8 bytes on.
__device__ __forceinline__ Frag32 frag32_at(const uint8_t* dec, uint32_t code_off, uint32_t pc_off) {
  Frag32 f;
  f.c0 = *reinterpret_cast<const long*>(dec + code_off);
  f.c1 = *reinterpret_cast<const long*>(dec + code_off + 2 * TM * 8);
  f.pc = *reinterpret_cast<const short4_t*>(dec + pc_off);
  return f;
}

__device__ __forceinline__ floatx16 scale_product32(const Frag32& a, const Frag32& b) {
  return __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(a.pc, b.pc, floatx16{}, 0, 0, 0);
}

template <int GRID>
__global__ __launch_bounds__(kThreads) void k_gemm_rd32(GemmLaunch g) {
  using L = Layout<32>;
  using D = Layout32;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

  const int tid = threadIdx.x, lane = tid & 63;
  const TileCtx ts = tile_ctx<32>(g, lds, tid);
  const RdCtx& c = ts.c;
  const int wave = ts.wave, wm = ts.wm, wn = ts.wn;
  const int64_t K = ts.klen;
  uint8_t* decb = lds + NRAW * L::RAW;   // two decoded buffers

  floatx16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      acc[i][j] = floatx16{};
      asm volatile("" : "+v"(acc[i][j]));   // no peeled first step
    }

  const int nsteps = (int)(K / 32);
  const int h = lane >> 5, r32 = lane & 31;
  const int dop = wave >> 2, drow = tid & (TM - 1);   // the row this thread decodes
  // fragment offsets in a decoded buffer; tile t adds 256 t (levels), 512 t (pieces)
  const uint32_t code_a = (uint32_t)(((0 + h) * TM + wm * 128 + r32) * 8);
  const uint32_t code_b = (uint32_t)(((4 + h) * TM + wn * 64 + r32) * 8);
  const uint32_t pc_a = (uint32_t)(D::LEV + (wm * 128 + r32) * 16 + 8 * h);
  const uint32_t pc_b = (uint32_t)(D::LEV + (TM + wn * 64 + r32) * 16 + 8 * h);
  if (nsteps > 0) {
    issue_stage<32>(c, 0, 0);
    issue_stage<32>(c, 1, 1);
    wait_vmcnt<L::VMEM>();
    __syncthreads();
    decode_store32<GRID>(decode_load32(lds, dop, drow, 0), decb, dop, drow);
    DecIn32 dnx = decode_load32(lds, dop, drow, 1);   // step 1 (stage 0 has landed)
    __syncthreads();
    Frag32 fa[4], fb[2];
#pragma unroll
    for (int t = 0; t < 4; ++t) fa[t] = frag32_at(decb, code_a + 256 * t, pc_a + 512 * t);
#pragma unroll
    for (int t = 0; t < 2; ++t) fb[t] = frag32_at(decb, code_b + 256 * t, pc_b + 512 * t);
    // As in the 16-wide kernel: tiles in column order (u = 0..7 is A tile
    // u & 3, B tile u >> 2), the products of tile u+1 issued during the fmas
    // of tile u (level product of the first half, 8 fmas, scale product, 4
    // fmas, level product of the second half chained on the first, 4 fmas),
    // each fragment reloaded after its last product; decode of step i+1 at
    // u = 0 (inputs read one step ahead), one barrier per step at u = 1.  A
    // raw stage holds 4 steps: stage s is issued at step 4 (s - 1) and waited
    // for at step 4 s - 2.
    floatx16 p[2], q[2];
    p[0] = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(fa[0].c0, fb[0].c0, floatx16{}, 0, 0, 0);
    q[0] = scale_product32(fa[0], fb[0]);
    p[0] = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(fa[0].c1, fb[0].c1, p[0], 0, 0, 0);
#pragma clang loop unroll(disable)
    for (int i = 0; i < nsteps; ++i) {
      if (i > 0 && (i & 3) == 0) issue_stage<32>(c, (i >> 2) + 1, ((i >> 2) + 1) & 1);
      const int n = i + 1;   // decoded during this step (past the end: unused)
      const DecIn32 din = dnx;   // step n's raw inputs, loaded during the step before
      const uint8_t* dn = decb + (n & 1) * D::DEC;
      const bool more = i + 1 < nsteps;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const Frag32& na = u + 1 < 8 ? fa[(u + 1) & 3] : fa[0];
        const Frag32& nb = u + 1 < 8 ? fb[(u + 1) >> 2] : fb[0];
        const bool go = u + 1 < 8 || more;
        if (go) p[(u + 1) & 1] = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(na.c0, nb.c0, floatx16{}, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < 8; ++r)
          acc[u & 3][u >> 2][r] = __builtin_fmaf(p[u & 1][r], q[u & 1][r], acc[u & 3][u >> 2][r]);
        __builtin_amdgcn_sched_barrier(0);
        if (go) q[(u + 1) & 1] = scale_product32(na, nb);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 8; r < 12; ++r)
          acc[u & 3][u >> 2][r] = __builtin_fmaf(p[u & 1][r], q[u & 1][r], acc[u & 3][u >> 2][r]);
        __builtin_amdgcn_sched_barrier(0);
        if (go) p[(u + 1) & 1] = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(na.c1, nb.c1, p[(u + 1) & 1], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 12; r < 16; ++r)
          acc[u & 3][u >> 2][r] = __builtin_fmaf(p[u & 1][r], q[u & 1][r], acc[u & 3][u >> 2][r]);
        asm volatile("" : "+v"(acc[u & 3][u >> 2]));   // the fmas stay here
        if (u == 0) decode_store32<GRID>(din, decb + (n & 1) * D::DEC, dop, drow);
        if (u == 1) {
          if (((i + 2) & 3) == 0) wait_vmcnt<0>();   // raw stage of step i+2 has landed
          __syncthreads();
          // raw inputs of step i+2 (its stage has landed for every wave)
          dnx = decode_load32(lds + (((i + 2) >> 2) & 1) * L::RAW, dop, drow, (i + 2) & 3);
        }
        if (u == 3) fb[0] = frag32_at(dn, code_b, pc_b);
        if (u >= 4) fa[u - 4] = frag32_at(dn, code_a + 256 * (u - 4), pc_a + 512 * (u - 4));
        if (u == 7) fb[1] = frag32_at(dn, code_b + 256, pc_b + 512);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  float* ct = ts.o.c + ts.row0 * g.ldc + ts.col0;
  if (ts.half < 0)
    store_c<4, 2>(ct, g.ldc, (int)ts.rows_a, (int)ts.rows_b, wm * 128, wn * 64, lane, acc);
  else
    add_c<4, 2>(ct, g.ldc, (int)ts.rows_a, (int)ts.rows_b, wm * 128, wn * 64, lane, acc);
}

template <int GRID>
hipError_t launch_rd32(const GemmLaunch& g, int grid, hipStream_t s) {
  constexpr int bytes = Layout32::TOTAL;
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t e = set_lds_limit((const void*)k_gemm_rd32<GRID>, bytes, lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_gemm_rd32<GRID>), dim3(grid), dim3(kThreads), bytes, s, g);
  return hipGetLastError();
}

// Zeros the C regions of the split tiles (slots split_first .. total_tiles-1).
__global__ __launch_bounds__(256) void k_zero_split(GemmLaunch g) {
  int tm, tn;
  const Operands o = resolve(g, g.split_first + (int)blockIdx.x, tm, tn);
  const int64_t row0 = (int64_t)tm * TM, col0 = (int64_t)tn * TN;
  const int rows = (int)(o.a_rows - row0 < TM ? o.a_rows - row0 : TM);
  const int cols = (int)(o.b_rows - col0 < TN ? o.b_rows - col0 : TN);
  float* c = o.c + row0 * g.ldc + col0;
  for (int r = (int)threadIdx.x >> 6; r < rows; r += 4)
    for (int k = (int)threadIdx.x & 63; k < cols; k += 64) c[(int64_t)r * g.ldc + k] = 0.0f;
}

// Compute units of the current device (cached per device id).
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace

bool gemm_rd_supported(const GemmLaunch& g) {
  return g.scale_mode == 0 && g.a_br == 1 && g.b_br == 1 && g.a_bc == g.b_bc &&
         (g.a_bc == 16 || g.a_bc == 32) && g.K % 16 == 0 &&
         (g.K / 2) * (int64_t)TM <= INT32_MAX;
}

hipError_t launch_gemm_rd(const GemmLaunch& g0, hipStream_t s) {
  if (g0.total_tiles == 0) return hipSuccess;
  // split the tiles of a last round that is at most half full (long tiles only:
  // 1024 K elements or more on average, so the zero fill is a small cost)
  GemmLaunch g = g0;
  const int T = g.total_tiles, cus = cu_count();
  const int rem = cus > 0 ? T % cus : 0;
  const int64_t kavg = g.mode == 2 ? (g.off[g.ngroups] - g.off[0]) / g.ngroups : g.K;
  g.split_first = rem > 0 && rem <= cus / 2 && kavg >= 1024 ? T - rem : T;
  const int nsplit = T - g.split_first;
  if (nsplit > 0) {
    hipLaunchKernelGGL(k_zero_split, dim3(nsplit), dim3(256), 0, s, g);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int grid = T + nsplit;
  const int key = g.grid * 2 + (g.a_bc == 32 ? 1 : 0);
  switch (key) {
    case 0: return launch_rd<0, 16>(g, grid, s);
    case 1: return launch_rd32<0>(g, grid, s);
    case 2: return launch_rd<1, 16>(g, grid, s);
    case 3: return launch_rd32<1>(g, grid, s);
    case 4: return launch_rd<2, 16>(g, grid, s);
    default: return launch_rd32<2>(g, grid, s);
  }
}

}  // namespace ufp4
