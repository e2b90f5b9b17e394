// Block-scaled 4-bit GEMM with power-of-two (E8M0) block scales on the
// gfx950 scaled matrix cores: C[p][q] = sum_k A[p][k] * B[q][k].
//
// [2DFP4] = "Stable FP4 Training via Transposition-Invariant Block
// Quantization" (agifrontier tutorial: 2D square-block quantization and its
// power-of-two scale equation).  [UFP4] = "Rethinking Shrinkage Bias in FP4
// Pretraining of LLMs ... the UFP4 Recipe" (hyper.ai summary, Method: both
// GEMM operands are quantized, the GEMM contracts the 4-bit values).
//
// With power-of-two scales every dequantized element is level * 2^e, so the
// matrix core can apply the scales itself: v_mfma_scale_f32_32x32x64_f8f6f4
// multiplies each lane's operand slice by 2^(byte - 127) for its 32-element
// K block and accumulates in fp32.  Operand formats:
//   E2M1: the stored sign-magnitude nibbles ARE OCP FP4 codes -- the codes go
//         from HBM through LDS into the instruction untouched (FP4 rate).
//   E1M2 (k/4) and INT4 (k): every level is exactly an FP8 E4M3 value, so each
//         nibble becomes one E4M3 byte through an 8-entry byte table
//         (v_perm) plus the sign bit when the tile is staged into LDS (FP8
//         rate).  The scale bytes are used unchanged in both cases.
// Both operands must have 32-element K blocks (2D 32 x 32 blocks, or 1 x 32
// rows) and K % 128 == 0; the dispatcher sends anything else to the
// general split-bf16 kernel.
//
// Operand layout inside the instruction (verified against a host model):
//   FP4: lane l holds row l % 32 and K elements 32 (l / 32) .. +31 of the
//        64-wide step, 16 bytes, element j in nibble j; its scale byte is the
//        one of that row and that 32-element block.
//   FP8: lane l holds row l % 32; bytes 0..15 belong to the first 32-element
//        block and bytes 16..31 to the second (16 elements of each), scaled by
//        the scale byte of lane (l % 32) and of lane 32 + (l % 32).  Any
//        element order inside a 16-byte group is fine as long as A and B use
//        the same one; the LDS staging below uses (even, odd) halves.
//   C:   as v_mfma_f32_32x32x16_bf16 (column l % 32, rows 8(r/4)+4(l/32)+r%4).
//
// Tiling (all kernels): 256 x 256 output tile per 256-thread workgroup,
// 2 x 2 waves of 128 x 128 (4 x 4 MFMA tiles, accumulators in AGPRs).  Tiles
// are ordered so that the tiles resident at one time on an XCD (workgroups are
// dealt round-robin over the 8 XCDs) are neighbours and share operand strips
// in that XCD's L2.  LDS rows are XOR-swizzled in 16-byte chunks so staging
// writes and fragment reads are free of bank conflicts.
//   k_gemm_mx4w (E2M1, K % 256 == 0): K step 256, codes copied HBM -> LDS by
//     buffer_load ... lds (no registers), each wave load = 8 rows x one full
//     128-byte line; two 68 KiB stages.
//   k_gemm_mx4 (E2M1, K % 128 == 0): K step 128, the same copy with 4 stages.
//   k_gemm_mx<GRID> (E1M2, INT4): K step 128; codes are loaded into registers
//     two steps ahead, converted to E4M3 and written to LDS (two stages).
//   k_gemm_mxrow<FMT> (one byte per element per row, copied HBM -> LDS
//     untouched, K step 128): FMT 0 = MXFP8 E4M3 codes; FMT 2 = E1M2 / INT4
//     levels as FP6 E2M3 operands, written beforehand by k_fp6_expand into a
//     caller workspace (a 32-byte slot per 32-element block: 24 bytes of
//     6-bit fields, element j at bits 6j..6j+5, then 8 unused bytes), so the
//     matrix cores run at the FP6 rate with no decode in the main loop.
//     (Packing two blocks into 48 bytes saves a quarter of the operand bytes
//     but made the main loop slower on the GPU: the fragment of a block then
//     spans two LDS chunks at different swizzle positions.)
//
// FP6 E2M3 embedding (sign, 2 exponent bits with bias 1, 3 mantissa bits; the
// subnormal step is 1/8): E1M2 level k/4 is the E2M3 code 2k, and every INT4
// level n in -7..7 is an E2M3 value (4..7 = 4 x 1, 1.25, 1.5, 1.75).  FP6 operand in the instruction (checked on the GPU against a
// host model): lane l holds row l % 32 and the 32 elements of one 32-element
// block (lane half h = block 2s + h of the 64-wide substep s) as 6-bit
// fields in its first 6 registers.
#include "ufp4_internal.h"
#include "gemm_epilogue.h"

namespace ufp4 {

namespace {

constexpr int TM = 256, TN = 256, KS = 128;   // tile rows, tile cols, K per step
constexpr int kThreads = 256;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// E4M3 bytes of the level magnitudes k = 0..7 (table for v_perm: entries 0..3
// in the low word, 4..7 in the high word).
//   E1M2 k/4: 0, 0.25, 0.5, 0.75, 1, 1.25, 1.5, 1.75
//   INT4 k:   0, 1, ..., 7
template <int GRID> struct E4m3Lut;
template <> struct E4m3Lut<0> { static constexpr uint32_t lo = 0x34302800u, hi = 0x3E3C3A38u; };
template <> struct E4m3Lut<1> { static constexpr uint32_t lo = 0x44403800u, hi = 0x4E4C4A48u; };

// Two's-complement nibbles -> sign-magnitude (8 | |k| for k < 0).
__device__ __forceinline__ uint32_t tc_to_sm(uint32_t w) {
  const uint32_t n = (w >> 3) & 0x11111111u;
  const uint32_t m = (n << 4) - n;
  return (((w ^ m) + n) & 0x77777777u) | (n << 3);
}

// Eight sign-magnitude nibbles (element j at bits 4j) -> E4M3 bytes of the
// even elements (0, 2, 4, 6) and of the odd ones (1, 3, 5, 7).
template <int GRID>
__device__ __forceinline__ void to_e4m3(uint32_t w, uint32_t lut_lo, uint32_t lut_hi,
                                        uint32_t& ev, uint32_t& od) {
  if constexpr (GRID == 1) w = tc_to_sm(w);
  const uint32_t me = w & 0x07070707u;
  const uint32_t mo = (w >> 4) & 0x07070707u;
  const uint32_t le = __builtin_amdgcn_perm(lut_hi, lut_lo, me);
  const uint32_t lo = __builtin_amdgcn_perm(lut_hi, lut_lo, mo);
  ev = ((w & 0x08080808u) << 4) | le;   // sign of element 2i: bit 3 -> bit 7
  od = (w & 0x80808080u) | lo;          // sign of element 2i+1 is already bit 7
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ v4i buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// LDS byte offset of 16-byte chunk c of tile row `row`, XOR-swizzled so that
// the rows read together by one pass of a fragment read and the threads
// writing the chunks of one row (a staging write) hit distinct banks.  With
// 128-byte rows two rows share the 64 banks, so the swizzle takes row bits
// 1..3: 16 consecutive rows reading the same chunk fill all 64 banks (row
// bits 0..2 gave 2-way conflicts; 1-3 % faster on the MX GEMMs).
__device__ __forceinline__ uint32_t off64(int row, int c) {    // 64-byte rows
  return (uint32_t)(row * 64 + 16 * (c ^ ((row >> 1) & 3)));
}
__device__ __forceinline__ uint32_t off128(int row, int c) {   // 128-byte rows
  return (uint32_t)(row * 128 + 16 * (c ^ ((row >> 1) & 7)));
}

// The operands of one output tile.  mode 0: the dense operands; mode 1
// (grouped along A's rows): rows off[g] .. off[g+1] of A against rows
// g*R .. g*R + R of B; mode 2 (grouped along K): segment g of both operands,
// stored [P][L_g] at element offset P*off[g] with 1 x 32 scales at P*off[g]/32.
// CPE4 = code bytes per four elements (2: packed nibbles, 4: byte rows).
struct MxTile {
  const uint8_t* a_codes;
  const uint8_t* b_codes;
  const uint8_t* a_scales;
  const uint8_t* b_scales;
  int64_t a_rows, b_rows, K;
  float* c;
  int tm, tn;
};

// The dense case alone (no group search, fewer live scalar values).
__device__ __forceinline__ MxTile mx_dense(const GemmLaunch& g, int b) {
  MxTile t;
  t.a_codes = g.a_codes; t.b_codes = g.b_codes;
  t.a_scales = reinterpret_cast<const uint8_t*>(g.a_scales);
  t.b_scales = reinterpret_cast<const uint8_t*>(g.b_scales);
  t.a_rows = g.PA; t.b_rows = g.PB; t.K = g.K; t.c = g.c;
  tile_order(b, g.total_tiles, (int)((g.PA + TM - 1) / TM), (int)((g.PB + TN - 1) / TN), t.tm,
             t.tn);
  return t;
}

template <int CPE4>
__device__ __forceinline__ MxTile mx_resolve(const GemmLaunch& g, int b) {
  int grp, local;
  slot_tile(g, b, grp, local);
  const uint8_t* sa = reinterpret_cast<const uint8_t*>(g.a_scales);
  const uint8_t* sb = reinterpret_cast<const uint8_t*>(g.b_scales);
  MxTile t;
  if (g.mode == 0) {
    t.a_codes = g.a_codes; t.b_codes = g.b_codes; t.a_scales = sa; t.b_scales = sb;
    t.a_rows = g.PA; t.b_rows = g.PB; t.K = g.K; t.c = g.c;
  } else if (g.mode == 1) {
    const int64_t r0 = g.off[grp], rb0 = (int64_t)grp * g.b_rows_per_group;
    t.a_codes = g.a_codes + r0 * g.K * CPE4 / 4;
    t.b_codes = g.b_codes + rb0 * g.K * CPE4 / 4;
    t.a_scales = sa + (r0 / g.a_br) * (g.K / 32);
    t.b_scales = sb + (rb0 / g.b_br) * (g.K / 32);
    t.a_rows = g.off[grp + 1] - r0; t.b_rows = g.b_rows_per_group; t.K = g.K;
    t.c = g.c + r0 * g.ldc;
  } else {
    const int64_t e = g.off[grp];
    t.a_codes = g.a_codes + g.PA * e * CPE4 / 4;
    t.b_codes = g.b_codes + g.PB * e * CPE4 / 4;
    t.a_scales = sa + g.PA * (e / 32);
    t.b_scales = sb + g.PB * (e / 32);
    t.a_rows = g.PA; t.b_rows = g.PB; t.K = g.off[grp + 1] - e;
    t.c = g.c + (int64_t)grp * g.PA * g.ldc;
  }
  const int tiles_m = (int)((t.a_rows + TM - 1) / TM);
  const int tiles_n = (int)((t.b_rows + TN - 1) / TN);
  grouped_order(local, tiles_m, tiles_n > 0 ? tiles_n : 1, t.tm, t.tn);
  return t;
}

// Raw loads of one K step for this thread: 4 code chunks of A and of B (rows
// t/4 + 64q, block t%4) and the scale words of the wave's rows.
struct StepLoads {
  v4i a[4], b[4];
  uint32_t sa[4], sb[4];   // scale bytes of blocks 4s..4s+3 (one word per MFMA row tile)
};

struct Ctx {
  __amdgpu_buffer_rsrc_t ra, rb;        // codes of this tile's rows
  uint32_t row_stride;                  // K / 2 bytes
  uint32_t ld_off;                      // this thread's byte offset within a step
  const uint8_t* sa_row[4];             // scale row of each A / B MFMA row tile (this lane)
  const uint8_t* sb_row[4];
  int nsteps;
};

__device__ __forceinline__ void fetch(const Ctx& c, int step, StepLoads& L) {
  const int st = step < c.nsteps ? step : c.nsteps - 1;   // past the end: re-read, unused
  const uint32_t base = (uint32_t)st * (KS / 2) + c.ld_off;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    L.a[q] = buf_load16(c.ra, base + (uint32_t)q * 64u * c.row_stride);
    L.b[q] = buf_load16(c.rb, base + (uint32_t)q * 64u * c.row_stride);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    L.sa[i] = *reinterpret_cast<const uint32_t*>(c.sa_row[i] + 4 * st);
    L.sb[i] = *reinterpret_cast<const uint32_t*>(c.sb_row[i] + 4 * st);
  }
}

// Stage one step's code chunks into LDS (converted to E4M3 for FP8).
template <int GRID>
__device__ __forceinline__ void stage(uint8_t* buf, const StepLoads& L, int tid) {
  constexpr int OPB = TM * 128;   // bytes per operand per stage
  const int r0 = tid >> 2, blk = tid & 3;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = r0 + 64 * q;
#pragma unroll
    for (int op = 0; op < 2; ++op) {
      const v4i v = op ? L.b[q] : L.a[q];
      uint8_t* dst = buf + op * OPB;
      const uint32_t lo = E4m3Lut<GRID>::lo, hi = E4m3Lut<GRID>::hi;
      uint32_t e[4], o[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) to_e4m3<GRID>((uint32_t)v[w], lo, hi, e[w], o[w]);
      const v4i h0 = {(int)e[0], (int)o[0], (int)e[1], (int)o[1]};   // elements 0..15
      const v4i h1 = {(int)e[2], (int)o[2], (int)e[3], (int)o[3]};   // elements 16..31
      *reinterpret_cast<v4i*>(dst + off128(row, 2 * blk)) = h0;
      *reinterpret_cast<v4i*>(dst + off128(row, 2 * blk + 1)) = h1;
    }
  }
}

// Fragments of one 64-wide k-substep for the wave's 4 A and 4 B row tiles.
struct Frags {
  v8i a[4], b[4];
};

// FP8 fragment of A row tile i (which = 0) or B row tile i (which = 1):
// block 2s -> chunk 4s + h, block 2s + 1 -> chunk 4s + 2 + h.
__device__ __forceinline__ v8i load_frag(const uint8_t* buf, int which, int s, int lane, int w,
                                         int i) {
  const int h = lane >> 5;
  const int r = w * 128 + i * 32 + (lane & 31);
  const uint8_t* base = buf + which * TM * 128;
  const v4i x0 = *reinterpret_cast<const v4i*>(base + off128(r, 4 * s + h));
  const v4i x1 = *reinterpret_cast<const v4i*>(base + off128(r, 4 * s + 2 + h));
  return v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
}

// The 16 MFMAs of one 64-wide k-substep.  Each fragment is reloaded with the
// next substep's (from LDS buffer `nbuf`, substep `ns`) as soon as its last
// use has issued, so one set of fragment registers suffices.
template <int GRID>
__device__ __forceinline__ void mfma_substep(floatx16 (&acc)[4][4], Frags& f,
                                             const uint32_t (&sa)[4], const uint32_t (&sb)[4],
                                             int s, int h, const uint8_t* nbuf, int ns, int lane,
                                             int wm, int wn) {
  const uint32_t sh = 8u * (uint32_t)(2 * s + h);
  int xa[4], xb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    xa[i] = (int)__builtin_amdgcn_ubfe(sa[i], sh, 8);
    xb[i] = (int)__builtin_amdgcn_ubfe(sb[i], sh, 8);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[i], f.b[j], acc[i][j], 0, 0, 0,
                                                                  xa[i], 0, xb[j]);
    }
  }
  if (nbuf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f.a[i] = load_frag(nbuf, 0, ns, lane, wm, i);
      f.b[i] = load_frag(nbuf, 1, ns, lane, wn, i);
    }
  }
}

template <int GRID, bool GROUPED, bool SCALED>
__global__ __launch_bounds__(kThreads) void k_gemm_mx(GemmLaunch g) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr int STAGE = 2 * TM * 128;

  const MxTile t = GROUPED ? mx_resolve<2>(g, blockIdx.x) : mx_dense(g, blockIdx.x);
  const int tm = t.tm, tn = t.tn;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, h = lane >> 5;
  const int64_t K = t.K;
  const int64_t row0 = (int64_t)tm * TM, col0 = (int64_t)tn * TN;
  const int64_t rows_a = t.a_rows - row0 < TM ? t.a_rows - row0 : TM;
  const int64_t rows_b = t.b_rows - col0 < TN ? t.b_rows - col0 : TN;

  Ctx c;
  c.row_stride = (uint32_t)(K / 2);
  c.ra = make_rsrc(t.a_codes + row0 * (K / 2), (uint32_t)(rows_a * (K / 2)));
  c.rb = make_rsrc(t.b_codes + col0 * (K / 2), (uint32_t)(rows_b * (K / 2)));
  c.ld_off = (uint32_t)(tid >> 2) * c.row_stride + 16u * (uint32_t)(tid & 3);
  c.nsteps = (int)(K / KS);
  const int64_t nkb = K / 32;
  const uint8_t* sa = t.a_scales;
  const uint8_t* sb = t.b_scales;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int64_t ra = row0 + wm * 128 + i * 32 + (lane & 31);
    int64_t rb = col0 + wn * 128 + i * 32 + (lane & 31);
    if (ra >= t.a_rows) ra = t.a_rows - 1;   // codes of such rows are zero; any scale works
    if (rb >= t.b_rows) rb = t.b_rows - 1;
    c.sa_row[i] = sa + (ra / g.a_br) * nkb;
    c.sb_row[i] = sb + (rb / g.b_br) * nkb;
  }

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx16{};

  StepLoads x{}, y{};
  uint32_t cs_a[4], cs_b[4];     // scale words of the step being multiplied
  // an empty K segment (grouped along K) reads nothing and leaves C = 0: the
  // step loop below does not run, and what the prologue stages is never used
  if (c.nsteps > 0) {
    fetch(c, 0, x);
    fetch(c, 1, y);
  }
  stage<GRID>(lds, x, tid);
#pragma unroll
  for (int i = 0; i < 4; ++i) { cs_a[i] = x.sa[i]; cs_b[i] = x.sb[i]; }
  __syncthreads();
  Frags f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f.a[i] = load_frag(lds, 0, 0, lane, wm, i);
    f.b[i] = load_frag(lds, 1, 0, lane, wn, i);
  }

  // Step i: LDS stage i&1 holds step i; `nx` holds the loads of step i+1;
  // `fr` receives the loads of step i+2.
  auto body = [&](int step, StepLoads& nx, StepLoads& fr) {
    const uint8_t* cur = lds + (step & 1) * STAGE;
    uint8_t* nxt = lds + ((step + 1) & 1) * STAGE;
    fetch(c, step + 2, fr);
    mfma_substep<GRID>(acc, f, cs_a, cs_b, 0, h, cur, 1, lane, wm, wn);
    stage<GRID>(nxt, nx, tid);
    mfma_substep<GRID>(acc, f, cs_a, cs_b, 1, h, nullptr, 0, lane, wm, wn);
#pragma unroll
    for (int i = 0; i < 4; ++i) { cs_a[i] = nx.sa[i]; cs_b[i] = nx.sb[i]; }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f.a[i] = load_frag(nxt, 0, 0, lane, wm, i);
      f.b[i] = load_frag(nxt, 1, 0, lane, wn, i);
    }
  };
  int step = 0;
  for (; step + 1 < c.nsteps; step += 2) {
    body(step, y, x);
    body(step + 1, x, y);
  }
  if (step < c.nsteps) body(step, y, x);
  store_c<4, 4>(t.c + row0 * g.ldc + col0, g.ldc, (int)rows_a, (int)rows_b, wm * 128, wn * 128,
                lane, acc, SCALED ? g.c_mul : 1.0f);
}

// ---------------------------------------------------------------------------
// E2M1 (FP4) kernel: the codes need no conversion, so they are copied from
// HBM straight into LDS (buffer_load ... lds: lane i's 16 bytes land at
// M0 + 16 i), four stages deep, with no register staging at all.  Each step
// moves, per operand, 256 rows x 64 code bytes (16 wave loads of 16 rows) and
// the 256 rows' scale words (4 bytes = the step's four 32-element blocks).
// The loads are issued from inline assembly and waited for with explicit
// vmcnt counts, so the compiler's own wait insertion (which does not see
// them) never stalls on the prefetch.
// ---------------------------------------------------------------------------
constexpr int NST = 4;                          // LDS stages
constexpr int F4_CODES = 2 * TM * 64;           // code bytes per stage (A then B)
constexpr int F4_SCALES = 2 * TM * 4;           // scale words per stage (A then B)
constexpr int F4_STAGE = F4_CODES + F4_SCALES;  // 34 KiB
constexpr int F4_VMEM_PER_STEP = 10;            // loads per wave per step (8 code, 2 scale)

typedef int sgpr4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ sgpr4 rsrc4(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  sgpr4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xFFFF);   // stride 0
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}

__device__ __forceinline__ void lds_load16(uint32_t lds_addr, const sgpr4& r, uint32_t voff,
                                           uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(r),
                 "s"(__builtin_amdgcn_readfirstlane(soff))
               : "memory");
}

__device__ __forceinline__ void lds_load4(uint32_t lds_addr, const sgpr4& r, uint32_t voff,
                                          uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(r),
                 "s"(__builtin_amdgcn_readfirstlane(soff))
               : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

struct F4Ctx {
  sgpr4 ra, rb, rsa, rsb;   // codes of the tile's A / B rows; scale arrays
  uint32_t lds0;            // LDS byte address of stage 0
  uint32_t code_voff[4];    // per wave load q: row * (K/2) + 16 * block
  uint32_t sa_voff, sb_voff;  // this lane's scale row byte offsets
  int wave, nsteps;
};

// Issue all loads of K step `step` (clamped to the last one) into stage `st`.
__device__ __forceinline__ void f4_issue(const F4Ctx& c, int step, int st) {
  const int s = step < c.nsteps ? step : c.nsteps - 1;
  const uint32_t base = c.lds0 + (uint32_t)st * F4_STAGE;
  const uint32_t koff = (uint32_t)s * 64u;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t blk = (uint32_t)(c.wave * 4 + q) * 1024u;   // 16 rows x 64 B
    lds_load16(base + blk, c.ra, c.code_voff[q], koff);
    lds_load16(base + TM * 64 + blk, c.rb, c.code_voff[q], koff);
  }
  const uint32_t swave = (uint32_t)c.wave * 256u;   // 64 rows x 4 B
  lds_load4(base + F4_CODES + swave, c.rsa, c.sa_voff, (uint32_t)s * 4u);
  lds_load4(base + F4_CODES + TM * 4 + swave, c.rsb, c.sb_voff, (uint32_t)s * 4u);
}

struct F4Frags {
  v8i a[4], b[4];
};

__device__ __forceinline__ void f4_frags(const uint8_t* stage, int s, int lane, int wm, int wn,
                                         F4Frags& f) {
  const int h = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ra = wm * 128 + i * 32 + (lane & 31);
    const int rb = wn * 128 + i * 32 + (lane & 31);
    const v4i x = *reinterpret_cast<const v4i*>(stage + off64(ra, 2 * s + h));
    const v4i y = *reinterpret_cast<const v4i*>(stage + TM * 64 + off64(rb, 2 * s + h));
    f.a[i] = v8i{x[0], x[1], x[2], x[3], 0, 0, 0, 0};
    f.b[i] = v8i{y[0], y[1], y[2], y[3], 0, 0, 0, 0};
  }
}

__device__ __forceinline__ void f4_scales(const uint8_t* stage, int lane, int wm, int wn,
                                          uint32_t (&sa)[4], uint32_t (&sb)[4]) {
  const uint32_t* sw = reinterpret_cast<const uint32_t*>(stage + F4_CODES);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sa[i] = sw[wm * 128 + i * 32 + (lane & 31)];
    sb[i] = sw[TM + wn * 128 + i * 32 + (lane & 31)];
  }
}

__device__ __forceinline__ void f4_mfma(floatx16 (&acc)[4][4], const F4Frags& f,
                                        const uint32_t (&sa)[4], const uint32_t (&sb)[4],
                                        int s, int h) {
  const uint32_t sh = 8u * (uint32_t)(2 * s + h);
  int xa[4], xb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    xa[i] = (int)__builtin_amdgcn_ubfe(sa[i], sh, 8);
    xb[i] = (int)__builtin_amdgcn_ubfe(sb[i], sh, 8);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[i], f.b[j], acc[i][j], 4, 4,
                                                                  0, xa[i], 0, xb[j]);
}

template <bool SCALED>
__global__ __launch_bounds__(kThreads) void k_gemm_mx4(GemmLaunch g) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

  const MxTile t = mx_resolve<2>(g, blockIdx.x);
  const int tm = t.tm, tn = t.tn;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, h = lane >> 5;
  const int64_t K = t.K;
  const int64_t row0 = (int64_t)tm * TM, col0 = (int64_t)tn * TN;
  const int64_t rows_a = t.a_rows - row0 < TM ? t.a_rows - row0 : TM;
  const int64_t rows_b = t.b_rows - col0 < TN ? t.b_rows - col0 : TN;
  const uint32_t rs = (uint32_t)(K / 2);
  const int64_t nkb = K / 32;
  const int sha = g.a_br == 32 ? 5 : 0, shb = g.b_br == 32 ? 5 : 0;

  F4Ctx c;
  c.wave = wave;
  c.nsteps = (int)(K / KS);
  c.ra = rsrc4(t.a_codes + row0 * rs, (uint32_t)(rows_a * rs));
  c.rb = rsrc4(t.b_codes + col0 * rs, (uint32_t)(rows_b * rs));
  // scale arrays: rows of nkb bytes, one row per block row
  c.rsa = rsrc4(t.a_scales, (uint32_t)(((t.a_rows - 1) >> sha) + 1) * (uint32_t)nkb);
  c.rsb = rsrc4(t.b_scales, (uint32_t)(((t.b_rows - 1) >> shb) + 1) * (uint32_t)nkb);
  c.lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)lds;
  // code loads: lane i of wave load q covers tile row 64 w + 16 q + i / 4 and
  // the block whose swizzled LDS chunk is i % 4 (rows past the operand fall
  // outside the buffer bound and read as zeros)
  const int lrow = lane >> 2;
  const uint32_t blk = (uint32_t)((lane & 3) ^ ((lrow >> 1) & 3));
#pragma unroll
  for (int q = 0; q < 4; ++q)
    c.code_voff[q] = (uint32_t)(wave * 64 + q * 16 + lrow) * rs + 16u * blk;
  // scale loads: lane i covers tile row 64 w + i (clamped into the operand)
  {
    int64_t ra = row0 + wave * 64 + lane, rb = col0 + wave * 64 + lane;
    if (ra >= t.a_rows) ra = t.a_rows - 1;
    if (rb >= t.b_rows) rb = t.b_rows - 1;
    c.sa_voff = (uint32_t)((ra >> sha) * nkb);
    c.sb_voff = (uint32_t)((rb >> shb) * nkb);
  }

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx16{};

  if (c.nsteps > 0) {   // an empty K segment leaves C = 0
    f4_issue(c, 0, 0);
    f4_issue(c, 1, 1);
    f4_issue(c, 2, 2);
    wait_vmcnt<2 * F4_VMEM_PER_STEP>();
    __syncthreads();
    F4Frags f0, f1;
    uint32_t sa[4], sb[4];
    f4_frags(lds, 0, lane, wm, wn, f0);
    f4_scales(lds, lane, wm, wn, sa, sb);

    // Step i computes from stage i % 4 while steps i+1, i+2 are in flight and
    // step i+3 is issued into the stage step i-1 used.
    auto body = [&](int step, int st) {
      const uint8_t* cur = lds + st * F4_STAGE;
      f4_issue(c, step + 3, (st + 3) & 3);
      f4_frags(cur, 1, lane, wm, wn, f1);
      f4_mfma(acc, f0, sa, sb, 0, h);
      f4_mfma(acc, f1, sa, sb, 1, h);
      wait_vmcnt<2 * F4_VMEM_PER_STEP>();   // step i+1 has landed (this wave's part)
      __syncthreads();                      // ... and every other wave's
      const uint8_t* nxt = lds + ((st + 1) & 3) * F4_STAGE;
      f4_frags(nxt, 0, lane, wm, wn, f0);
      f4_scales(nxt, lane, wm, wn, sa, sb);
    };
    int step = 0;
    for (; step + 3 < c.nsteps; step += 4) {
      body(step, 0);
      body(step + 1, 1);
      body(step + 2, 2);
      body(step + 3, 3);
    }
    for (; step < c.nsteps; ++step) body(step, step & 3);
    wait_vmcnt<0>();   // drain the clamped prefetches before the workgroup ends
  }

  store_c<4, 4>(t.c + row0 * g.ldc + col0, g.ldc, (int)rows_a, (int)rows_b, wm * 128, wn * 128,
                lane, acc, SCALED ? g.c_mul : 1.0f);
}

template <bool SCALED>
hipError_t launch_mx4_s(const GemmLaunch& g, hipStream_t s) {
  constexpr int bytes = NST * F4_STAGE;
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t e = set_lds_limit((const void*)k_gemm_mx4<SCALED>, bytes, lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_gemm_mx4<SCALED>), dim3(g.total_tiles), dim3(kThreads), bytes, s, g);
  return hipGetLastError();
}

hipError_t launch_mx4(const GemmLaunch& g, hipStream_t s) {
  return g.c_mul == 1.0f ? launch_mx4_s<false>(g, s) : launch_mx4_s<true>(g, s);
}

// ---------------------------------------------------------------------------
// Wide-step E2M1 kernel: K step 256, so every row contributes one whole
// 128-byte line per step and each wave load covers 8 full lines (8 rows x
// 128 B).  Two LDS stages of 68 KiB (codes 2 x 32 KiB, scale words 2 x 2 KiB).
// ---------------------------------------------------------------------------
constexpr int KW = 256;
constexpr int W4_CODES = 2 * TM * 128;
constexpr int W4_SCALES = 2 * 2 * TM * 4;       // [op][half][row] words
constexpr int W4_STAGE = W4_CODES + W4_SCALES;  // 68 KiB

struct W4Ctx {
  sgpr4 ra, rb, rsa, rsb;
  uint32_t lds0;
  uint32_t code_voff[8];      // wave load q: row * (K/2) + 16 * chunk
  uint32_t sa_voff, sb_voff;  // this lane's scale row byte offsets
  int wave, nsteps;
};

__device__ __forceinline__ void w4_issue(const W4Ctx& c, int step, int st) {
  const int s = step < c.nsteps ? step : c.nsteps - 1;
  const uint32_t base = c.lds0 + (uint32_t)st * W4_STAGE;
  const uint32_t koff = (uint32_t)s * 128u;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const uint32_t blk = (uint32_t)(c.wave * 8 + q) * 1024u;   // 8 rows x 128 B
    lds_load16(base + blk, c.ra, c.code_voff[q], koff);
    lds_load16(base + TM * 128 + blk, c.rb, c.code_voff[q], koff);
  }
  const uint32_t swave = (uint32_t)c.wave * 256u;
  const uint32_t sbase = base + W4_CODES;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    lds_load4(sbase + hf * TM * 4 + swave, c.rsa, c.sa_voff, (uint32_t)s * 8u + 4u * hf);
    lds_load4(sbase + 2 * TM * 4 + hf * TM * 4 + swave, c.rsb, c.sb_voff,
              (uint32_t)s * 8u + 4u * hf);
  }
}

__device__ __forceinline__ void w4_frags(const uint8_t* stage, int s, int lane, int wm, int wn,
                                         F4Frags& f) {
  const int h = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ra = wm * 128 + i * 32 + (lane & 31);
    const int rb = wn * 128 + i * 32 + (lane & 31);
    const v4i x = *reinterpret_cast<const v4i*>(stage + off128(ra, 2 * s + h));
    const v4i y = *reinterpret_cast<const v4i*>(stage + TM * 128 + off128(rb, 2 * s + h));
    f.a[i] = v8i{x[0], x[1], x[2], x[3], 0, 0, 0, 0};
    f.b[i] = v8i{y[0], y[1], y[2], y[3], 0, 0, 0, 0};
  }
}

__device__ __forceinline__ void w4_scales(const uint8_t* stage, int lane, int wm, int wn,
                                          uint32_t (&sa)[2][4], uint32_t (&sb)[2][4]) {
  const uint32_t* sw = reinterpret_cast<const uint32_t*>(stage + W4_CODES);
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sa[hf][i] = sw[hf * TM + wm * 128 + i * 32 + (lane & 31)];
      sb[hf][i] = sw[2 * TM + hf * TM + wn * 128 + i * 32 + (lane & 31)];
    }
}

template <bool SCALED>
__global__ __launch_bounds__(kThreads) void k_gemm_mx4w(GemmLaunch g) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

  const MxTile t = mx_resolve<2>(g, blockIdx.x);
  const int tm = t.tm, tn = t.tn;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, h = lane >> 5;
  const int64_t K = t.K;
  const int64_t row0 = (int64_t)tm * TM, col0 = (int64_t)tn * TN;
  const int64_t rows_a = t.a_rows - row0 < TM ? t.a_rows - row0 : TM;
  const int64_t rows_b = t.b_rows - col0 < TN ? t.b_rows - col0 : TN;
  const uint32_t rs = (uint32_t)(K / 2);
  const int64_t nkb = K / 32;
  const int sha = g.a_br == 32 ? 5 : 0, shb = g.b_br == 32 ? 5 : 0;

  W4Ctx c;
  c.wave = wave;
  c.nsteps = (int)(K / KW);
  c.ra = rsrc4(t.a_codes + row0 * rs, (uint32_t)(rows_a * rs));
  c.rb = rsrc4(t.b_codes + col0 * rs, (uint32_t)(rows_b * rs));
  c.rsa = rsrc4(t.a_scales, (uint32_t)(((t.a_rows - 1) >> sha) + 1) * (uint32_t)nkb);
  c.rsb = rsrc4(t.b_scales, (uint32_t)(((t.b_rows - 1) >> shb) + 1) * (uint32_t)nkb);
  c.lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)lds;
  // lane i of wave load q: tile row 64 w + 8 q + i / 8, the chunk whose
  // swizzled slot (off128) is i % 8
  const int lrow = lane >> 3;
#pragma unroll
  for (int q = 0; q < 8; ++q)
    c.code_voff[q] = (uint32_t)(wave * 64 + q * 8 + lrow) * rs +
                     16u * (uint32_t)((lane & 7) ^ ((4 * q + (lrow >> 1)) & 7));
  {
    int64_t ra = row0 + wave * 64 + lane, rb = col0 + wave * 64 + lane;
    if (ra >= t.a_rows) ra = t.a_rows - 1;
    if (rb >= t.b_rows) rb = t.b_rows - 1;
    c.sa_voff = (uint32_t)((ra >> sha) * nkb);
    c.sb_voff = (uint32_t)((rb >> shb) * nkb);
  }

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx16{};

  if (c.nsteps > 0) {   // an empty K segment leaves C = 0
    w4_issue(c, 0, 0);
    wait_vmcnt<0>();
    __syncthreads();
    F4Frags f0, f1;
    uint32_t sa[2][4], sb[2][4];
    w4_frags(lds, 0, lane, wm, wn, f0);
    w4_scales(lds, lane, wm, wn, sa, sb);

    for (int step = 0; step < c.nsteps; ++step) {
      const uint8_t* cur = lds + (step & 1) * W4_STAGE;
      w4_issue(c, step + 1, (step + 1) & 1);
      w4_frags(cur, 1, lane, wm, wn, f1);
      f4_mfma(acc, f0, sa[0], sb[0], 0, h);
      w4_frags(cur, 2, lane, wm, wn, f0);
      f4_mfma(acc, f1, sa[0], sb[0], 1, h);
      w4_frags(cur, 3, lane, wm, wn, f1);
      f4_mfma(acc, f0, sa[1], sb[1], 0, h);
      f4_mfma(acc, f1, sa[1], sb[1], 1, h);
      wait_vmcnt<0>();
      __syncthreads();
      const uint8_t* nxt = lds + ((step + 1) & 1) * W4_STAGE;
      w4_frags(nxt, 0, lane, wm, wn, f0);
      w4_scales(nxt, lane, wm, wn, sa, sb);
    }
  }

  store_c<4, 4>(t.c + row0 * g.ldc + col0, g.ldc, (int)rows_a, (int)rows_b, wm * 128, wn * 128,
                lane, acc, SCALED ? g.c_mul : 1.0f);
}

// ---------------------------------------------------------------------------
// Byte-row kernels: one byte per element per row (MXFP8 E4M3 codes, or FP6
// E2M3 fields in 32-byte slots), copied HBM -> LDS untouched as in
// k_gemm_mx4w.  K step 128 = one 128-byte line per row; two 66 KiB stages
// (codes 2 x 32 KiB, one scale word per row and operand).  FP8 fragments and
// the scale operand as in the FP8 path of k_gemm_mx: lane l takes 16 bytes of
// blocks 2s and 2s+1 (chunks 4s + h and 4s + 2 + h) and supplies the scale of
// row l % 32, block 2s + h.  FP6 fragments: lane l takes the 24 bytes of
// block 2s + h (chunk 4s + 2h and the first half of chunk 4s + 2h + 1), same
// scale.
// ---------------------------------------------------------------------------
constexpr int K8 = 128;
constexpr int W8_CODES = 2 * TM * 128;
constexpr int W8_STAGE = W8_CODES + 2 * TM * 4;   // 66 KiB

typedef int v2i __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void w8_issue(const W4Ctx& c, int step, int st) {
  const int s = step < c.nsteps ? step : c.nsteps - 1;   // past the end: re-read, unused
  const uint32_t base = c.lds0 + (uint32_t)st * W8_STAGE;
  const uint32_t koff = (uint32_t)s * 128u;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const uint32_t blk = (uint32_t)(c.wave * 8 + q) * 1024u;   // 8 rows x 128 B
    lds_load16(base + blk, c.ra, c.code_voff[q], koff);
    lds_load16(base + TM * 128 + blk, c.rb, c.code_voff[q], koff);
  }
  const uint32_t swave = (uint32_t)c.wave * 256u;
  lds_load4(base + W8_CODES + swave, c.rsa, c.sa_voff, (uint32_t)s * 4u);
  lds_load4(base + W8_CODES + TM * 4 + swave, c.rsb, c.sb_voff, (uint32_t)s * 4u);
}

template <int FMT>
__device__ __forceinline__ void w8_frags(const uint8_t* stage, int s, int lane, int wm, int wn,
                                         F4Frags& f) {
  const int h = lane >> 5;
  const uint8_t* b = stage + TM * 128;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ra = wm * 128 + i * 32 + (lane & 31);
    const int rb = wn * 128 + i * 32 + (lane & 31);
    if constexpr (FMT == 0) {
      const v4i x0 = *reinterpret_cast<const v4i*>(stage + off128(ra, 4 * s + h));
      const v4i x1 = *reinterpret_cast<const v4i*>(stage + off128(ra, 4 * s + 2 + h));
      const v4i y0 = *reinterpret_cast<const v4i*>(b + off128(rb, 4 * s + h));
      const v4i y1 = *reinterpret_cast<const v4i*>(b + off128(rb, 4 * s + 2 + h));
      f.a[i] = v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      f.b[i] = v8i{y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
    } else {
      const v4i x0 = *reinterpret_cast<const v4i*>(stage + off128(ra, 4 * s + 2 * h));
      const v2i x1 = *reinterpret_cast<const v2i*>(stage + off128(ra, 4 * s + 2 * h + 1));
      const v4i y0 = *reinterpret_cast<const v4i*>(b + off128(rb, 4 * s + 2 * h));
      const v2i y1 = *reinterpret_cast<const v2i*>(b + off128(rb, 4 * s + 2 * h + 1));
      f.a[i] = v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], 0, 0};
      f.b[i] = v8i{y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], 0, 0};
    }
  }
}

__device__ __forceinline__ void w8_scales(const uint8_t* stage, int lane, int wm, int wn,
                                          uint32_t (&sa)[4], uint32_t (&sb)[4]) {
  const uint32_t* sw = reinterpret_cast<const uint32_t*>(stage + W8_CODES);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sa[i] = sw[wm * 128 + i * 32 + (lane & 31)];
    sb[i] = sw[TM + wn * 128 + i * 32 + (lane & 31)];
  }
}

// FMT is the operand format code of the instruction (0 = FP8 E4M3, 2 = FP6 E2M3).
template <int FMT>
__device__ __forceinline__ void f8_mfma(floatx16 (&acc)[4][4], const F4Frags& f,
                                        const uint32_t (&sa)[4], const uint32_t (&sb)[4],
                                        int s, int h) {
  const uint32_t sh = 8u * (uint32_t)(2 * s + h);
  int xa[4], xb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    xa[i] = (int)__builtin_amdgcn_ubfe(sa[i], sh, 8);
    xb[i] = (int)__builtin_amdgcn_ubfe(sb[i], sh, 8);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[i], f.b[j], acc[i][j], FMT,
                                                                  FMT, 0, xa[i], 0, xb[j]);
}

template <int FMT, bool GROUPED, bool SCALED>
__global__ __launch_bounds__(kThreads) void k_gemm_mxrow(GemmLaunch g) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

  const MxTile t = GROUPED ? mx_resolve<4>(g, blockIdx.x) : mx_dense(g, blockIdx.x);
  const int tm = t.tm, tn = t.tn;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, h = lane >> 5;
  const int64_t K = t.K;
  const int64_t row0 = (int64_t)tm * TM, col0 = (int64_t)tn * TN;
  const int64_t rows_a = t.a_rows - row0 < TM ? t.a_rows - row0 : TM;
  const int64_t rows_b = t.b_rows - col0 < TN ? t.b_rows - col0 : TN;
  const uint32_t rs = (uint32_t)K;            // one byte per element
  const int64_t nkb = K / 32;
  const int sha = g.a_br == 32 ? 5 : 0, shb = g.b_br == 32 ? 5 : 0;

  W4Ctx c;
  c.wave = wave;
  c.nsteps = (int)(K / K8);
  c.ra = rsrc4(t.a_codes + row0 * rs, (uint32_t)(rows_a * rs));
  c.rb = rsrc4(t.b_codes + col0 * rs, (uint32_t)(rows_b * rs));
  c.rsa = rsrc4(t.a_scales, (uint32_t)(((t.a_rows - 1) >> sha) + 1) * (uint32_t)nkb);
  c.rsb = rsrc4(t.b_scales, (uint32_t)(((t.b_rows - 1) >> shb) + 1) * (uint32_t)nkb);
  c.lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)lds;
  // lane i of wave load q: tile row 64 w + 8 q + i / 8, the chunk whose
  // swizzled slot (off128) is i % 8
  const int lrow = lane >> 3;
#pragma unroll
  for (int q = 0; q < 8; ++q)
    c.code_voff[q] = (uint32_t)(wave * 64 + q * 8 + lrow) * rs +
                     16u * (uint32_t)((lane & 7) ^ ((4 * q + (lrow >> 1)) & 7));
  {
    int64_t ra = row0 + wave * 64 + lane, rb = col0 + wave * 64 + lane;
    if (ra >= t.a_rows) ra = t.a_rows - 1;   // codes of such rows read as zero; any scale works
    if (rb >= t.b_rows) rb = t.b_rows - 1;
    c.sa_voff = (uint32_t)((ra >> sha) * nkb);
    c.sb_voff = (uint32_t)((rb >> shb) * nkb);
  }

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx16{};

  // an empty K segment (grouped along K) reads nothing and leaves C = 0: the
  // step loop below does not run, and what the prologue stages is never used
  if (c.nsteps > 0) w8_issue(c, 0, 0);
  wait_vmcnt<0>();
  __syncthreads();
  F4Frags f0, f1;
  uint32_t sa[4], sb[4];
  w8_frags<FMT>(lds, 0, lane, wm, wn, f0);
  w8_scales(lds, lane, wm, wn, sa, sb);

  for (int step = 0; step < c.nsteps; ++step) {
    const uint8_t* cur = lds + (step & 1) * W8_STAGE;
    w8_issue(c, step + 1, (step + 1) & 1);
    w8_frags<FMT>(cur, 1, lane, wm, wn, f1);
    f8_mfma<FMT>(acc, f0, sa, sb, 0, h);
    f8_mfma<FMT>(acc, f1, sa, sb, 1, h);
    wait_vmcnt<0>();
    __syncthreads();
    const uint8_t* nxt = lds + ((step + 1) & 1) * W8_STAGE;
    w8_frags<FMT>(nxt, 0, lane, wm, wn, f0);
    w8_scales(nxt, lane, wm, wn, sa, sb);
  }

  store_c<4, 4>(t.c + row0 * g.ldc + col0, g.ldc, (int)rows_a, (int)rows_b, wm * 128, wn * 128,
                lane, acc, SCALED ? g.c_mul : 1.0f);
}

// E2M3 fields of four 4-bit codes, one per byte (bits 0..3 of each byte in,
// bits 0..5 out; see the header): E1M2 sign-magnitude s|k -> s<<5 | 2k, which
// is 2 (c + (c & 8)); INT4 two's complement n -> sign<<5 | E2M3(|n|) through two
// 8-entry byte tables (nibbles 0..7 and 8..15) and a per-byte select:
// 1 -> 8, 2 -> 16, 3 -> 20, 4..7 -> 24, 26, 28, 30.  The nibble 8 (-8, no code
// of the symmetric grid) has no E2M3 value and reads as -7.5 (63).
template <int GRID>
__device__ __forceinline__ uint32_t fp6_fields4(uint32_t c) {
  if constexpr (GRID == 0) {
    return (c + (c & 0x08080808u)) << 1;
  } else {
    const uint32_t m = c & 0x07070707u;
    const uint32_t pos = __builtin_amdgcn_perm(0x1E1C1A18u, 0x14100800u, m);   // nibbles 0..7
    const uint32_t neg = __builtin_amdgcn_perm(0x28303438u, 0x3A3C3E3Fu, m);   // nibbles 8..15
    const uint32_t b = (c >> 3) & 0x01010101u;
    const uint32_t sel = (b << 8) - b;   // 0xFF in the bytes of negative nibbles
    return (neg & sel) | (pos & ~sel);
  }
}

// The eight fields of one code word (element j at bits 4j) as 48 bits,
// element j at bits 6j: lo = bits 0..31, hi = bits 32..47.  Fields of the
// even and odd elements come one per byte; [f0 f1 f4 f5] and [f2 f3 f6 f7]
// are gathered by byte permutes, each byte pair closes up to 12 bits, and the
// four 12-bit groups are laid end to end.
template <int GRID>
__device__ __forceinline__ void fp6_word(uint32_t w, uint32_t& lo, uint32_t& hi) {
  const uint32_t fe = fp6_fields4<GRID>(w & 0x0F0F0F0Fu);          // f0 f2 f4 f6
  const uint32_t fo = fp6_fields4<GRID>((w >> 4) & 0x0F0F0F0Fu);   // f1 f3 f5 f7
  const uint32_t a = __builtin_amdgcn_perm(fo, fe, 0x06020400u);     // f0 f1 f4 f5
  const uint32_t b = __builtin_amdgcn_perm(fo, fe, 0x07030501u);     // f2 f3 f6 f7
  const uint32_t ga = (a & 0x003F003Fu) | ((a >> 2) & 0x0FC00FC0u);  // g01 | g45 << 16
  const uint32_t gb = (b & 0x003F003Fu) | ((b >> 2) & 0x0FC00FC0u);  // g23 | g67 << 16
  lo = (ga & 0xFFFu) | ((gb & 0xFFFu) << 12) | ((ga & 0x00FF0000u) << 8);
  hi = (ga >> 24) | (gb >> 12);
}

// Six 32-bit words of 6-bit E2M3 fields (element j at bits 6j) from the
// 32 code nibbles of one block (four 48-bit runs).
template <int GRID>
__device__ __forceinline__ void fp6_block(const v4i& w, uint32_t (&o)[6]) {
  uint32_t lo[4], hi[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) fp6_word<GRID>((uint32_t)w[i], lo[i], hi[i]);
  o[0] = lo[0];
  o[1] = hi[0] | (lo[1] << 16);
  o[2] = (lo[1] >> 16) | (hi[1] << 16);
  o[3] = lo[2];
  o[4] = hi[2] | (lo[3] << 16);
  o[5] = (lo[3] >> 16) | (hi[3] << 16);
}

// One thread per 32-element block: 16 code bytes in, the 24 field bytes of
// its 32-byte slot out (the last 8 bytes of a slot are copied into LDS with
// the rest but no fragment reads them, so they are left unwritten).  Blocks
// 0 .. na-1 come from `a` (into `oa`), the rest from `b` (into `ob`): both
// operands in one launch.
template <int GRID>
__global__ __launch_bounds__(256) void k_fp6_expand(const uint8_t* __restrict__ a,
                                                    uint8_t* __restrict__ oa, int64_t na,
                                                    const uint8_t* __restrict__ b,
                                                    uint8_t* __restrict__ ob, int64_t nb) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t bk = (int64_t)blockIdx.x * 256 + threadIdx.x; bk < na + nb; bk += stride) {
    const bool in_a = bk < na;
    const int64_t k = in_a ? bk : bk - na;
    uint32_t f[6];
    fp6_block<GRID>(*reinterpret_cast<const v4i*>((in_a ? a : b) + k * 16), f);
    uint8_t* dst = (in_a ? oa : ob) + k * 32;
    *reinterpret_cast<v4i*>(dst) = v4i{(int)f[0], (int)f[1], (int)f[2], (int)f[3]};
    *reinterpret_cast<v2i*>(dst + 16) = v2i{(int)f[4], (int)f[5]};
  }
}

template <int FMT, bool GROUPED, bool SCALED>
hipError_t launch_mxrow_s(const GemmLaunch& g, hipStream_t s) {
  constexpr int bytes = 2 * W8_STAGE;
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t e =
      set_lds_limit((const void*)k_gemm_mxrow<FMT, GROUPED, SCALED>, bytes, lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_gemm_mxrow<FMT, GROUPED, SCALED>), dim3(g.total_tiles), dim3(kThreads),
                     bytes, s, g);
  return hipGetLastError();
}

// MXFP8 (FMT 0) is dense only; the FP6 operands may be grouped.
template <int FMT>
hipError_t launch_mxrow(const GemmLaunch& g, hipStream_t s) {
  const bool scaled = g.c_mul != 1.0f;
  if constexpr (FMT == 2) {
    if (g.mode != 0)
      return scaled ? launch_mxrow_s<FMT, true, true>(g, s)
                    : launch_mxrow_s<FMT, true, false>(g, s);
  }
  return scaled ? launch_mxrow_s<FMT, false, true>(g, s) : launch_mxrow_s<FMT, false, false>(g, s);
}

// Both operands' codes (PA x K and PB x K) into FP6 slots at oa and ob.
template <int GRID>
hipError_t launch_fp6_expand(const GemmLaunch& g, uint8_t* oa, uint8_t* ob, hipStream_t s) {
  const int64_t na = g.PA * (g.K / 32), nb = g.PB * (g.K / 32);
  if (na + nb == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((na + nb + 255) / 256, 8192);
  hipLaunchKernelGGL((k_fp6_expand<GRID>), dim3((unsigned)blocks), dim3(256), 0, s, g.a_codes,
                     oa, na, g.b_codes, ob, nb);
  return hipGetLastError();
}

template <bool SCALED>
hipError_t launch_mx4w_s(const GemmLaunch& g, hipStream_t s) {
  constexpr int bytes = 2 * W4_STAGE;
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t e = set_lds_limit((const void*)k_gemm_mx4w<SCALED>, bytes, lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_gemm_mx4w<SCALED>), dim3(g.total_tiles), dim3(kThreads), bytes, s, g);
  return hipGetLastError();
}

hipError_t launch_mx4w(const GemmLaunch& g, hipStream_t s) {
  return g.c_mul == 1.0f ? launch_mx4w_s<false>(g, s) : launch_mx4w_s<true>(g, s);
}

template <int GRID, bool GROUPED, bool SCALED>
hipError_t launch_mx_g(const GemmLaunch& g, hipStream_t s) {
  constexpr int bytes = 2 * 2 * TM * 128;   // 2 stages x 2 operands
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t e =
      set_lds_limit((const void*)k_gemm_mx<GRID, GROUPED, SCALED>, bytes, lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_gemm_mx<GRID, GROUPED, SCALED>), dim3(g.total_tiles), dim3(kThreads),
                     bytes, s, g);
  return hipGetLastError();
}

template <int GRID>
hipError_t launch_mx(const GemmLaunch& g, hipStream_t s) {
  if (g.c_mul != 1.0f)
    return g.mode == 0 ? launch_mx_g<GRID, false, true>(g, s) : launch_mx_g<GRID, true, true>(g, s);
  return g.mode == 0 ? launch_mx_g<GRID, false, false>(g, s) : launch_mx_g<GRID, true, false>(g, s);
}

}  // namespace

namespace {

// Every shared-dimension length of the launch (K, or each segment's length
// when grouped along K) is a multiple of `step`.
bool k_multiple(const GemmLaunch& g, int64_t step) {
  if (g.mode != 2) return g.K % step == 0;
  for (int i = 0; i < g.ngroups; ++i)
    if ((g.off[i + 1] - g.off[i]) % step) return false;
  return true;
}

// Block shapes, grouping and 32-bit buffer sizes the scaled-MFMA kernels
// take (`bpe4`: code bytes per four elements of the kernel's operand rows).
bool mx_layout_ok(const GemmLaunch& g, int64_t step, int64_t bpe4) {
  if (g.scale_mode != 1 || g.a_bc != 32 || g.b_bc != 32) return false;
  const bool rows_ok = (g.a_br == 1 || g.a_br == 32) && (g.b_br == 1 || g.b_br == 32);
  if (g.mode == 0 && !rows_ok) return false;
  if (g.mode == 1 && !(rows_ok && g.b_rows_per_group % g.b_br == 0)) return false;
  if (g.mode == 2 && !(g.a_br == 1 && g.b_br == 1)) return false;
  return k_multiple(g, step) && g.K * bpe4 / 4 * (int64_t)TM <= INT32_MAX &&
         ((g.PA - 1) / g.a_br + 1) * (g.K / 32) <= INT32_MAX &&
         ((g.PB - 1) / g.b_br + 1) * (g.K / 32) <= INT32_MAX;
}

}  // namespace

bool gemm_mx_supported(const GemmLaunch& g) {
  if (g.grid == 3)   // MXFP8: dense, 1 x 32 blocks, byte codes
    return g.mode == 0 && g.a_br == 1 && g.b_br == 1 && mx_layout_ok(g, K8, 4);
  return mx_layout_ok(g, KS, 2);
}

bool gemm_mx6_supported(const GemmLaunch& g) {
  return (g.grid == 0 || g.grid == 1) && mx_layout_ok(g, K8, 4);
}

// FP6 operands: one 32-byte slot per 32-element block (one byte per element),
// A then B at a 256-byte boundary.
int64_t gemm_mx6_workspace(const GemmLaunch& g) {
  return ((g.PA * g.K + 255) / 256) * 256 + g.PB * g.K;
}

hipError_t launch_gemm_mx6(const GemmLaunch& g, uint8_t* ws, hipStream_t s) {
  if (g.total_tiles == 0) return hipSuccess;
  GemmLaunch x = g;
  x.a_codes = ws;
  x.b_codes = ws + ((g.PA * g.K + 255) / 256) * 256;
  uint8_t* wb = const_cast<uint8_t*>(x.b_codes);
  const hipError_t e = g.grid == 0 ? launch_fp6_expand<0>(g, ws, wb, s)
                                   : launch_fp6_expand<1>(g, ws, wb, s);
  if (e != hipSuccess) return e;
  return launch_mxrow<2>(x, s);
}

hipError_t launch_gemm_mx(const GemmLaunch& g, hipStream_t s) {
  if (g.total_tiles == 0) return hipSuccess;
  switch (g.grid) {
    case 0: return launch_mx<0>(g, s);
    case 1: return launch_mx<1>(g, s);
    case 3: return launch_mxrow<0>(g, s);
    default: return k_multiple(g, KW) ? launch_mx4w(g, s) : launch_mx4(g, s);
  }
}

}  // namespace ufp4
