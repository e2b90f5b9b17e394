// Dequantization, quantized-operand transpose and the draw generator check
// kernel for gfx950.
//
// [UFP4] = "Rethinking Shrinkage Bias in FP4 Pretraining of LLMs ... the UFP4
// Recipe" (hyper.ai summary, formats section: Q_G(T) stands for the
// dequantized tensor, level times block scale).
// [2DFP4] = "Stable FP4 Training via Transposition-Invariant Block
// Quantization" (2D section: S(B) = S(B^T), so a square-block operand is
// reused transposed without requantizing).
#include "ufp4_internal.h"

namespace ufp4 {

namespace {

__device__ __forceinline__ float level_of(uint32_t c, int grid) {
  if (grid == 3) {                                                 // E4M3 byte (MXFP8)
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    const float mag = e == 0u ? ldexpf((float)m, -9) : ldexpf((float)(8u + m), (int)e - 10);
    return (c & 0x80u) ? -mag : mag;
  }
  if (grid == 1) return (float)(((int)(c << 28)) >> 28);          // INT4 two's complement
  const uint32_t k = c & 7u;
  float m;
  if (grid == 0) {
    m = (float)k * 0.25f;                                          // E1M2: k/4
  } else {                                                         // E2M1
    // {0, .5, 1, 1.5} below index 4, then (2 + mantissa) * 2^(exponent - 2)
    m = (k < 4u) ? 0.5f * (float)k : (float)((2u + (k & 1u)) << ((k >> 1) - 2u));
  }
  return (c & 8u) ? -m : m;
}

// out[p][k] = RN(level(code) * s) -- one thread per 8 elements.
__global__ void k_dequant(const uint8_t* codes, const void* scales, int64_t P, int64_t K,
                          int grid, int smode, int br, int bc, float ts, float* out, int64_t ldo) {
  const int64_t n8 = P * (K / 8);
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n8;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t p = i / (K / 8), k0 = (i - p * (K / 8)) * 8;
    uint2 cw;
    if (grid == 3) cw = *reinterpret_cast<const uint2*>(codes + p * K + k0);
    else cw.x = *reinterpret_cast<const uint32_t*>(codes + p * (K / 2) + k0 / 2);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t c = grid == 3 ? (((j < 4 ? cw.x : cw.y) >> (8 * (j & 3))) & 0xFFu)
                                   : ((cw.x >> (4 * j)) & 15u);
      const int64_t k = k0 + j;
      float s;
      if (smode == 0) {
        s = reinterpret_cast<const float*>(scales)[p * (K / bc) + k / bc];
      } else {
        const uint8_t e = reinterpret_cast<const uint8_t*>(scales)[(p / br) * (K / bc) + k / bc];
        s = ldexpf(1.0f, (int)e - 127);
      }
      // level * 2^e is exact, so with two-level scaling one rounding of
      // level * 2^e * s_T (ts = 1 otherwise: exact)
      out[p * ldo + k] = __fmul_rn(__fmul_rn(level_of(c, grid), s), ts);
    }
  }
}

// dst[k][p] nibble = src[p][k] nibble; one thread per destination byte pair
// of rows (two source columns).
__global__ void k_transpose_codes(const uint8_t* src, int64_t P, int64_t K, uint8_t* dst) {
  const int64_t nbytes = K * (P / 2);
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < nbytes;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t k = i / (P / 2), j = i - k * (P / 2);
    const int64_t p0 = 2 * j;
    const uint8_t b0 = src[p0 * (K / 2) + k / 2];
    const uint8_t b1 = src[(p0 + 1) * (K / 2) + k / 2];
    const uint32_t sh = (k & 1) ? 4u : 0u;
    dst[i] = (uint8_t)(((b0 >> sh) & 15u) | (((b1 >> sh) & 15u) << 4));
  }
}

// 8 x 8 nibble transpose in registers: r[i] holds row i (column c at bits
// 4c); afterwards r[c] holds column c (row i at bits 4i).  Three rounds swap
// the off-diagonal 4 x 4, then 2 x 2, then 1 x 1 blocks.
__device__ __forceinline__ void transpose_nibbles8(uint32_t (&r)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t t = ((r[i] >> 16) ^ r[i + 4]) & 0x0000FFFFu;
    r[i] ^= t << 16;
    r[i + 4] ^= t;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = (q & 1) + 4 * (q >> 1);   // 0, 1, 4, 5
    const uint32_t t = ((r[i] >> 8) ^ r[i + 2]) & 0x00FF00FFu;
    r[i] ^= t << 8;
    r[i + 2] ^= t;
  }
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    const uint32_t t = ((r[i] >> 4) ^ r[i + 1]) & 0x0F0F0F0Fu;
    r[i] ^= t << 4;
    r[i + 1] ^= t;
  }
}

constexpr int kTE = 256;   // transpose tile edge, in nibbles

// Word w of staged tile row `row`, XOR-swizzled so that the 16-byte staging
// writes (8 lanes per row) and the block reads (32 lanes, one row each 8
// apart) both fall on distinct banks.
__device__ __forceinline__ int staged_word(int row, int w) {
  return row * 32 + (w ^ (((row >> 3) ^ (row & 7)) & 31));
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Tiled codes transpose (P, K multiples of 8; P * K / 2 < 2^31): one
// workgroup per 256 x 256-nibble tile.  The source tile (256 rows x 128 B)
// is staged in LDS with full 16-byte row loads; each thread then transposes
// four 8 x 8 nibble blocks in registers and 32 consecutive lanes store one
// 128-byte run of a destination row.  Rows past P read as zero (buffer bound)
// and nothing past P or K is stored.
__global__ __launch_bounds__(256) void k_transpose_codes_tiled(const uint8_t* src, int64_t P,
                                                               int64_t K, uint8_t* dst,
                                                               int tiles_k) {
  __shared__ uint32_t t[kTE * 32];
  const int tid = threadIdx.x;
  const int64_t p0 = (int64_t)(blockIdx.x / tiles_k) * kTE;
  const int64_t k0 = (int64_t)(blockIdx.x % tiles_k) * kTE;
  const uint32_t row_bytes = (uint32_t)(K / 2);
  const uint32_t bound = (uint32_t)(P * (K / 2));
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(src), (short)0, (int)bound, 0x00020000);
  const int c = tid & 7;
#pragma unroll
  for (int ps = 0; ps < 8; ++ps) {
    const int r = ps * 32 + (tid >> 3);
    const int64_t p = p0 + r;
    const uint32_t off = p < P ? (uint32_t)p * row_bytes + (uint32_t)(k0 / 2) + 16u * c : bound;
    const u32x4_t v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0));
#pragma unroll
    for (int e = 0; e < 4; ++e) t[staged_word(r, 4 * c + e)] = v[e];
  }
  __syncthreads();
  const int lane = tid & 63, wave = tid >> 6, pb = lane & 31;
  const bool p_ok = p0 + 8 * pb < P;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int kb = (lane >> 5) + 2 * wave + 8 * j;
    uint32_t r[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = t[staged_word(8 * pb + i, kb)];
    transpose_nibbles8(r);
    if (!p_ok) continue;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t k = k0 + 8 * kb + e;
      if (k < K) *reinterpret_cast<uint32_t*>(dst + k * (P / 2) + p0 / 2 + 4 * pb) = r[e];
    }
  }
}

__global__ void k_transpose_scales(const uint8_t* src, int64_t rb, int64_t cb, int esize,
                                   uint8_t* dst) {
  const int64_t n = rb * cb;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / cb, c = i - r * cb;
    for (int b = 0; b < esize; ++b) dst[(c * rb + r) * esize + b] = src[i * esize + b];
  }
}

__global__ void k_philox_fill(uint64_t seed, uint32_t stream, uint64_t first, int64_t n,
                              uint16_t* out) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const uint64_t e = first + (uint64_t)i;
    const uint64_t g = e >> 3;
    uint32_t c[4] = {(uint32_t)g, (uint32_t)(g >> 32), stream, 0u};
    philox4x32_10_dev(c, (uint32_t)seed, (uint32_t)(seed >> 32));
    const uint32_t w = c[(e & 7) >> 1];
    out[i] = (uint16_t)((e & 1) ? (w >> 16) : (w & 0xFFFFu));
  }
}

// C[r][c] = 0 for r < rows, c < cols of a row-major fp32 matrix with pitch
// ld: the product over an empty shared dimension.
__global__ void k_zero_c(float* c, int64_t rows, int64_t cols, int64_t ld) {
  const int64_t n = rows * cols;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / cols;
    c[r * ld + (i - r * cols)] = 0.0f;
  }
}

// Streaming copy of n16 16-byte vectors: one vector per thread and a grid
// that covers the buffer (a grid-stride loop only past 2^24 workgroups), with
// non-temporal loads and stores (nothing is reused); the bytes past the last
// whole vector are copied one by one.  Measured on gfx950 (1 GiB): this form
// reaches 6.5 TB/s, grid-stride loops over 2048 - 65536 workgroups with one to
// eight vectors in flight per thread 4.3 - 5.6 TB/s.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void k_stream_copy(const u32x4* __restrict__ src,
                                                     u32x4* __restrict__ dst, int64_t n16,
                                                     const uint8_t* __restrict__ tsrc,
                                                     uint8_t* __restrict__ tdst, int tail) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
  if (blockIdx.x == 0 && threadIdx.x < tail) tdst[threadIdx.x] = tsrc[threadIdx.x];
}

int grid_for(int64_t work, int threads) {
  int64_t b = (work + threads - 1) / threads;
  if (b > 65536) b = 65536;
  return (int)(b < 1 ? 1 : b);
}

}  // namespace

hipError_t launch_dequant(const uint8_t* codes, const void* scales, int64_t P, int64_t K,
                          int32_t grid, int32_t smode, int32_t br, int32_t bc, float ts,
                          float* out, int64_t ldo, hipStream_t s) {
  const int64_t n8 = P * (K / 8);
  if (n8 == 0) return hipSuccess;
  hipLaunchKernelGGL(k_dequant, dim3(grid_for(n8, 256)), dim3(256), 0, s, codes, scales, P, K,
                     (int)grid, (int)smode, (int)br, (int)bc, ts, out, ldo);
  return hipGetLastError();
}

hipError_t launch_transpose(const uint8_t* codes, const void* scales, int64_t P, int64_t K,
                            int32_t b, int32_t smode, uint8_t* dcodes, void* dscales,
                            hipStream_t s) {
  const int64_t nbytes = K * (P / 2);
  if (nbytes == 0) return hipSuccess;
  const bool tiled = P % 8 == 0 && K % 8 == 0 && P * (K / 2) < ((int64_t)1 << 31) &&
                     reinterpret_cast<uintptr_t>(codes) % 4 == 0 &&
                     reinterpret_cast<uintptr_t>(dcodes) % 4 == 0;
  if (tiled) {
    const int64_t tiles_k = (K + kTE - 1) / kTE, tiles = ((P + kTE - 1) / kTE) * tiles_k;
    hipLaunchKernelGGL(k_transpose_codes_tiled, dim3((unsigned)tiles), dim3(256), 0, s, codes, P,
                       K, dcodes, (int)tiles_k);
  } else {
    hipLaunchKernelGGL(k_transpose_codes, dim3(grid_for(nbytes, 256)), dim3(256), 0, s, codes, P,
                       K, dcodes);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rb = P / b, cb = K / b;
  hipLaunchKernelGGL(k_transpose_scales, dim3(grid_for(rb * cb, 256)), dim3(256), 0, s,
                     reinterpret_cast<const uint8_t*>(scales), rb, cb, smode == 0 ? 4 : 1,
                     reinterpret_cast<uint8_t*>(dscales));
  return hipGetLastError();
}

hipError_t launch_zero_c(float* c, int64_t rows, int64_t cols, int64_t ld, hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  hipLaunchKernelGGL(k_zero_c, dim3(grid_for(rows * cols, 256)), dim3(256), 0, s, c, rows, cols,
                     ld);
  return hipGetLastError();
}

hipError_t launch_stream_copy(const void* src, void* dst, int64_t nbytes, hipStream_t s) {
  if (nbytes == 0) return hipSuccess;
  const int64_t n16 = nbytes / 16;
  const int tail = (int)(nbytes - n16 * 16);
  int64_t blocks = (n16 + 255) / 256;
  if (blocks > ((int64_t)1 << 24)) blocks = (int64_t)1 << 24;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_stream_copy, dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16,
                     static_cast<const uint8_t*>(src) + n16 * 16,
                     static_cast<uint8_t*>(dst) + n16 * 16, tail);
  return hipGetLastError();
}

hipError_t launch_philox_fill(uint64_t seed, uint32_t stream_id, uint64_t first, int64_t n,
                              uint16_t* out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_philox_fill, dim3(grid_for(n, 256)), dim3(256), 0, s, seed, stream_id,
                     first, n, out);
  return hipGetLastError();
}

}  // namespace ufp4
