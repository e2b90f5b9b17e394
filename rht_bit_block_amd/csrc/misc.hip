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
                          int grid, int smode, int br, int bc, float* out, int64_t ldo) {
  const int64_t n8 = P * (K / 8);
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n8;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t p = i / (K / 8), k0 = (i - p * (K / 8)) * 8;
    const uint32_t w = *reinterpret_cast<const uint32_t*>(codes + p * (K / 2) + k0 / 2);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t k = k0 + j;
      float s;
      if (smode == 0) {
        s = reinterpret_cast<const float*>(scales)[p * (K / bc) + k / bc];
      } else {
        const uint8_t e = reinterpret_cast<const uint8_t*>(scales)[(p / br) * (K / bc) + k / bc];
        s = ldexpf(1.0f, (int)e - 127);
      }
      out[p * ldo + k] = __fmul_rn(level_of((w >> (4 * j)) & 15u, grid), s);
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
    philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
    const uint32_t w = c[(e & 7) >> 1];
    out[i] = (uint16_t)((e & 1) ? (w >> 16) : (w & 0xFFFFu));
  }
}

int grid_for(int64_t work, int threads) {
  int64_t b = (work + threads - 1) / threads;
  if (b > 65536) b = 65536;
  return (int)(b < 1 ? 1 : b);
}

}  // namespace

hipError_t launch_dequant(const uint8_t* codes, const void* scales, int64_t P, int64_t K,
                          int32_t grid, int32_t smode, int32_t br, int32_t bc, float* out,
                          int64_t ldo, hipStream_t s) {
  const int64_t n8 = P * (K / 8);
  if (n8 == 0) return hipSuccess;
  hipLaunchKernelGGL(k_dequant, dim3(grid_for(n8, 256)), dim3(256), 0, s, codes, scales, P, K,
                     (int)grid, (int)smode, (int)br, (int)bc, out, ldo);
  return hipGetLastError();
}

hipError_t launch_transpose(const uint8_t* codes, const void* scales, int64_t P, int64_t K,
                            int32_t b, int32_t smode, uint8_t* dcodes, void* dscales,
                            hipStream_t s) {
  const int64_t nbytes = K * (P / 2);
  if (nbytes == 0) return hipSuccess;
  hipLaunchKernelGGL(k_transpose_codes, dim3(grid_for(nbytes, 256)), dim3(256), 0, s, codes, P, K,
                     dcodes);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rb = P / b, cb = K / b;
  hipLaunchKernelGGL(k_transpose_scales, dim3(grid_for(rb * cb, 256)), dim3(256), 0, s,
                     reinterpret_cast<const uint8_t*>(scales), rb, cb, smode == 0 ? 4 : 1,
                     reinterpret_cast<uint8_t*>(dscales));
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
