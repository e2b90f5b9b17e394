// Internal interface between the C-ABI layer (api.cpp: validation, planning)
// and the HIP kernels (quant.hip, gemm.hip, misc.hip).  Host-visible structs
// only; every pointer is a device pointer unless named host_*.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ufp4.h"

#include <atomic>

namespace ufp4 {

constexpr int kMaxSegments = 128;  // segments per segmented quantization launch
constexpr int kMaxGroups = 64;     // groups per grouped GEMM launch

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
// as 1, 2, 3", SC'11): ten rounds of the 4x32 Philox S-box with the Weyl key
// schedule.  Usable on host (sign draw) and device (stochastic rounding).
__host__ __device__ inline void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
    const uint32_t n1 = (uint32_t)p1;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
    const uint32_t n3 = (uint32_t)p0;
    c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
  }
}

// The same generator in device code: each round's two three-input XORs
// are one gfx950 three-input bitwise op each (truth table 0x96 = a ^ b ^ c;
// the compiler emits two two-input XORs for them otherwise).
__device__ __forceinline__ uint32_t xor3_key(uint32_t a, uint32_t b, uint32_t key) {
  return __builtin_amdgcn_bitop3_b32(a, b, key, 0x96);
}

__device__ __forceinline__ void philox4x32_10_dev(uint32_t c[4], uint32_t k0,
                                                          uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
    const uint32_t n0 = xor3_key((uint32_t)(p1 >> 32), c[1], k0);
    const uint32_t n2 = xor3_key((uint32_t)(p0 >> 32), c[3], k1);
    c[1] = (uint32_t)p1;
    c[3] = (uint32_t)p0;
    c[0] = n0;
    c[2] = n2;
  }
}

// RN(1/d) for d in [2^-60, 2^60]: gfx950's reciprocal (within one ulp) with
// one Newton correction through its exact fma residual.  On gfx950 this
// equals the IEEE quotient 1/d for every mantissa, checked exhaustively in
// binades from 2^-60 to 2^59 (the raw reciprocal misses RN on about one
// mantissa in nine, the same ones in every binade; one correction removes all
// of them).  A GPU test repeats the check.
__device__ __forceinline__ float rcp_rn(float d) {
  const float y = __builtin_amdgcn_rcpf(d);
  return __builtin_fmaf(__builtin_fmaf(-d, y, 1.0f), y, y);
}

// Unsigned 32-bit division by a launch constant d >= 1, as a multiply-high
// (Granlund & Montgomery, "Division by invariant integers using
// multiplication", PLDI'94): q = (umulhi(m, n) + n) >> l with l = ceil(log2 d),
// m = floor(2^32 (2^l - d) / d) + 1, exact for every 32-bit n.
struct FastDiv {
  uint32_t d, m, l;
};
inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  const uint64_t m = ((1ull << 32) * ((1ull << l) - d)) / d + 1;
  return FastDiv{d, (uint32_t)m, l};
}

struct QuantLaunch {
  const uint16_t* x;
  int64_t ld;        // row pitch of x in elements
  int64_t rows;      // rows of x (segmented / column-wise: K extent)
  int64_t cols;      // columns of x
  int64_t P, K;      // logical operand (dense calls)
  uint8_t* codes;
  void* scales;
  float* rotated;
  uint32_t sign_pat[4];  // sign bits of chunk positions 32i..32i+31
  float cn;              // RN(1/sqrt(n))
  int32_t n;
  int32_t grid, rounding, scale_mode, br, bc;
  uint64_t sr_seed;
  uint32_t sr_stream;
  float tmul;            // two-level scaling: RN(1 / s_T); 1 for single-level
  // segmented column-wise
  int32_t nseg;
  int64_t seg_off[kMaxSegments + 1];
  int32_t tile_start[kMaxSegments + 1];
};

// Column extent of a dual-axis quantization tile (its row extent is 128):
// the row-wise Hadamard chunks must fit inside a tile.
constexpr int dual_tile_cols(int n) { return n > 64 ? 128 : 64; }

// Row-wise side of a two-axis quantization: its own outputs, signs and draws
// (the geometry and the column-wise side live in the QuantLaunch).
struct RowSide {
  uint8_t* codes;
  void* scales;
  float* rotated;   // always null (no debug output for the fused call)
  uint32_t sign_pat[4];
  float cn;
  uint64_t sr_seed;
  uint32_t sr_stream;
  float tmul;       // two-level scaling: RN(1 / s_T); 1 for single-level
};

hipError_t launch_quant_rows(const QuantLaunch& q, hipStream_t s);
hipError_t launch_quant_dual(const QuantLaunch& q, const RowSide& r, hipStream_t s);
// Level statistics: `partials` is a device buffer of kDiagWorkspaceBytes,
// 8-byte aligned, cleared and used by the call (partial sums of the
// workgroups); calls that overlap must not share it.
constexpr int kDiagSlots = 64;
constexpr size_t kDiagWorkspaceBytes = (size_t)kDiagSlots * 16 * sizeof(unsigned long long);
hipError_t launch_quant_diag(const QuantLaunch& q, unsigned long long* stats,
                             unsigned long long* partials, hipStream_t s);
// Argument checks and launch description of a level-statistics call (the
// arguments of ufp4_quant_diag without its workspace); UFP4_OK or a status.
int diag_prepare(const void* x, int64_t rows, int64_t cols, int64_t ld, const ufp4_quant_cfg* cfg,
                 const uint64_t* stats, QuantLaunch& q);

hipError_t launch_quant_cols(const QuantLaunch& q, hipStream_t s);
hipError_t launch_quant_rows_2d(const QuantLaunch& q, hipStream_t s);

struct GemmLaunch {
  const uint8_t* a_codes;
  const void* a_scales;
  const uint8_t* b_codes;
  const void* b_scales;
  float* c;
  int64_t ldc;
  int32_t a_br, a_bc, b_br, b_bc;
  int32_t grid, scale_mode;
  int32_t mode;     // 0 dense, 1 grouped along A rows, 2 grouped along K
  int32_t ngroups;
  int64_t PA, PB, K;
  int64_t b_rows_per_group;
  int64_t off[kMaxGroups + 1];
  int32_t tile_start[kMaxGroups + 1];
  int32_t total_tiles;
  // mode 2 (every group has the same tile count), set when contiguous XCD
  // ranges would be unbalanced: deal > 0 tiles at a time go to each XCD in
  // turn, walking the groups in gorder (longest segment first); 0: contiguous
  int32_t deal;
  int32_t gorder[kMaxGroups];
  float c_mul;      // factor on C: the operands' tensor factors (two-level scaling), 1 if none
  // fp32-scale kernels only, set by their launcher: tile slots from
  // split_first on are each computed by two workgroups, one per half of K,
  // whose partial sums are added into a zeroed C (total_tiles: no split)
  int32_t split_first;
};

// Raises a kernel's dynamic LDS limit to `bytes` once per kernel and device
// (the attribute belongs to the device that is current); `done` holds one bit
// per device id.  Two threads racing on the first call both set it, which is
// harmless.
inline hipError_t set_lds_limit(const void* kernel, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t)1 << dev : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
  return e;
}

hipError_t launch_gemm(const GemmLaunch& g, hipStream_t s);
// Power-of-two (E8M0) scales on the scaled matrix cores; only for launches
// gemm_mx_supported() accepts.
bool gemm_mx_supported(const GemmLaunch& g);
// fp32 scales, 1 x 16 / 1 x 32 blocks: per 16-wide K step, exact level dot
// products on the fp8 matrix cores times scale products from the bf16 ones;
// only for launches gemm_rd_supported() accepts.
bool gemm_rd_supported(const GemmLaunch& g);
hipError_t launch_gemm_rd(const GemmLaunch& g, hipStream_t s);
hipError_t launch_gemm_mx(const GemmLaunch& g, hipStream_t s);
// E1M2 / INT4 with 32-element E8M0 blocks as FP6 E2M3 operands: both
// operands are first expanded into `ws` (gemm_mx6_workspace bytes, 256-byte
// aligned), then multiplied on the scaled matrix cores at the FP6 rate.
bool gemm_mx6_supported(const GemmLaunch& g);
int64_t gemm_mx6_workspace(const GemmLaunch& g);
hipError_t launch_gemm_mx6(const GemmLaunch& g, uint8_t* ws, hipStream_t s);

// `ts`: the two-level tensor factor s_T (1 for single-level scaling).
hipError_t launch_dequant(const uint8_t* codes, const void* scales, int64_t P, int64_t K,
                          int32_t grid, int32_t scale_mode, int32_t br, int32_t bc, float ts,
                          float* out, int64_t ldo, hipStream_t s);
hipError_t launch_transpose(const uint8_t* codes, const void* scales, int64_t P, int64_t K,
                            int32_t b, int32_t scale_mode, uint8_t* dcodes, void* dscales,
                            hipStream_t s);
// Writes zeros into C [rows][ld] (columns 0 .. cols-1): a GEMM whose shared
// dimension is empty.
hipError_t launch_zero_c(float* c, int64_t rows, int64_t cols, int64_t ld, hipStream_t s);
hipError_t launch_stream_copy(const void* src, void* dst, int64_t nbytes, hipStream_t s);
hipError_t launch_philox_fill(uint64_t seed, uint32_t stream_id, uint64_t first, int64_t n,
                              uint16_t* out, hipStream_t s);

}  // namespace ufp4
