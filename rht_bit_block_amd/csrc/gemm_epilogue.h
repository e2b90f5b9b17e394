// Tile order and the store of a wave's fp32 C block, shared by the
// 256 x 256-tile GEMM kernels.
//
// The accumulators of a 32 x 32 MFMA tile hold, in lane l and register r,
// column l % 32 and row 8 (r / 4) + 4 (l / 32) + r % 4.  The stores go
// through a buffer resource whose base is the tile's first element and whose
// size ends at the last valid row, so rows past the operand are dropped by
// the hardware bound check; lanes whose column is past the operand get an
// offset beyond the bound.  Each store is then one 32-bit add and one
// buffer_store_dword, instead of 64-bit address arithmetic and a branch per
// element.
#pragma once

#include "ufp4_internal.h"

namespace ufp4 {

typedef float c_floatx16 __attribute__((ext_vector_type(16)));

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup b runs on
// XCD b % 8) and each XCD has its own L2.  xcd_linear gives every XCD a
// contiguous range of the launch's T tiles: XCD x takes T / 8 tiles, one more
// when x < T % 8, and workgroup b is the (b / 8)-th of its XCD -- a bijection
// of 0 .. T-1 for any T.
__device__ __forceinline__ int xcd_linear(int b, int T) {
  const int q = T / 8, r = T % 8, x = b % 8;
  return x * q + (x < r ? x : r) + b / 8;
}

// Tile (tm, tn) at position w of the grouped order of a tiles_m x tiles_n
// problem: kGroupRows tile rows at a time, walking down a group's rows before
// moving one tile column right.  The 32 tiles one XCD runs at once then cover
// about 8 rows x 4 columns of C and share 12 operand strips, where a
// row-major range shares one A strip and reads up to 32 B strips.
constexpr int kGroupRows = 8;
__device__ __forceinline__ void grouped_order(int w, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int group = w / (kGroupRows * tiles_n);
  const int first = group * kGroupRows;
  const int gm = tiles_m - first < kGroupRows ? tiles_m - first : kGroupRows;
  const int u = w - first * tiles_n;
  tm = first + u % gm;
  tn = u / gm;
}

// Group and tile index inside it of launch slot b.  Default: position
// xcd_linear(b) of the launch's tiles in group order, so each XCD works
// through a contiguous range (whole experts).  K-grouped launches whose
// contiguous ranges would be unbalanced (deal > 0: a tile costs in proportion
// to its group's segment, and the host found one XCD's range well above the
// mean): the groups in gorder, longest first, and runs of `deal` consecutive
// tiles (a share of one group, in grouped order) dealt to the XCDs in turn,
// so every XCD gets an equal part of every group and the short tiles fill the
// end; a last partial round of runs takes contiguous ranges.
__device__ __forceinline__ void slot_tile(const GemmLaunch& g, int b, int& grp, int& local) {
  const int T = g.total_tiles;
  if (g.mode == 2 && g.deal > 0) {
    const int per = g.tile_start[1], c = g.deal;
    const int j = b / 8, x = b % 8, R = T / (8 * c);
    const int s = j < R * c ? ((j / c) * 8 + x) * c + j % c
                            : 8 * c * R + xcd_linear(b - 8 * c * R, T - 8 * c * R);
    grp = g.gorder[s / per];
    local = s % per;
    return;
  }
  const int tile = xcd_linear(b, T);
  grp = 0;
  while (grp + 1 < g.ngroups && g.tile_start[grp + 1] <= tile) ++grp;
  local = tile - g.tile_start[grp];
}

// Tile (tm, tn) that workgroup b of a dense T-tile launch computes.
__device__ __forceinline__ void tile_order(int b, int T, int tiles_m, int tiles_n, int& tm,
                                           int& tn) {
  grouped_order(xcd_linear(b, T), tiles_m, tiles_n, tm, tn);
}

// True when a tile's C region fits a 32-bit buffer offset (else the caller
// uses plain stores).
__device__ __forceinline__ bool c_fits_buffer(int64_t ldc, int rows) {
  return (int64_t)rows * ldc * 4 < ((int64_t)1 << 31);
}

// Store the NI x NJ MFMA tiles of one wave.  c_tile: C + row0 * ldc + col0;
// rows_valid / cols_valid: extent of C inside the tile; r0 / c0: the wave's
// first row / column inside the tile.
template <int NI, int NJ>
__device__ __forceinline__ void store_c_tile(float* c_tile, int64_t ldc, int rows_valid,
                                             int cols_valid, int r0, int c0, int lane,
                                             const c_floatx16 (&acc)[NI][NJ], float m) {
  const uint32_t ld4 = (uint32_t)ldc * 4u;
  const uint32_t bound = (uint32_t)rows_valid * ld4;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(c_tile, (short)0, (int)bound, 0x00020000);
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int col = c0 + j * 32 + (lane & 31);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint32_t row = (uint32_t)(r0 + i * 32 + 4 * (lane >> 5));
      const uint32_t base = col < cols_valid ? row * ld4 + 4u * (uint32_t)col : bound;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t off = base + (uint32_t)(8 * (r >> 2) + (r & 3)) * ld4;
        // __float_as_uint, not __builtin_bit_cast: the bit cast of an
        // accumulator element reaching this intrinsic was lowered to the same
        // register for every element.  Cache policy 2 = non-temporal: C is
        // written once and not read back by the kernel, so it streams out
        // without displacing the operand strips other tiles still read
        // (the dense layer's step measured 0.8 % faster, 6 of 6 same-box pairs).
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][r] * m), rs, (int)off, 0,
                                              2);
      }
    }
  }
}

// Plain stores with explicit bounds (large leading dimensions).
template <int NI, int NJ>
__device__ __forceinline__ void store_c_plain(float* c_tile, int64_t ldc, int rows_valid,
                                              int cols_valid, int r0, int c0, int lane,
                                              const c_floatx16 (&acc)[NI][NJ], float m) {
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int col = c0 + j * 32 + (lane & 31);
    if (col >= cols_valid) continue;
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = r0 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < rows_valid) c_tile[(int64_t)row * ldc + col] = acc[i][j][r] * m;
      }
  }
}

// Add a wave's partial sums into C (one of the two K halves of a split tile;
// C was zeroed before the launch).  Hardware fp32 atomic adds: with exactly
// two addends on an exact zero the result is the same in either order.
template <int NI, int NJ>
__device__ __forceinline__ void add_c(float* c_tile, int64_t ldc, int rows_valid, int cols_valid,
                                      int r0, int c0, int lane, const c_floatx16 (&acc)[NI][NJ]) {
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int col = c0 + j * 32 + (lane & 31);
    if (col >= cols_valid) continue;
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = r0 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < rows_valid) unsafeAtomicAdd(c_tile + (int64_t)row * ldc + col, acc[i][j][r]);
      }
  }
}

// m: a factor on every element of C (two-level scaling: the operands'
// tensor factors; 1 otherwise, an exact multiply).
template <int NI, int NJ>
__device__ __forceinline__ void store_c(float* c_tile, int64_t ldc, int rows_valid,
                                        int cols_valid, int r0, int c0, int lane,
                                        const c_floatx16 (&acc)[NI][NJ], float m = 1.0f) {
  if (c_fits_buffer(ldc, 256))
    store_c_tile<NI, NJ>(c_tile, ldc, rows_valid, cols_valid, r0, c0, lane, acc, m);
  else
    store_c_plain<NI, NJ>(c_tile, ldc, rows_valid, cols_valid, r0, c0, lane, acc, m);
}

}  // namespace ufp4
