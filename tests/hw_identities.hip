// Test library (not part of the product): checks on the GPU that the
// quantizer's reciprocal helper rcp_rn(d) equals the IEEE quotient 1/d for
// every float d whose mantissa lies in [1, 2) in the binade 2^e.
#include "ufp4_internal.h"

namespace {

__global__ __launch_bounds__(256) void k_rcp_check(int e, unsigned int* bad) {
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;
  if (i >= (1u << 23)) return;
  const float d = __builtin_ldexpf(__uint_as_float(0x3F800000u | i), e);
  if (__float_as_uint(ufp4::rcp_rn(d)) != __float_as_uint(__fdiv_rn(1.0f, d))) atomicAdd(bad, 1u);
}

}  // namespace

// Mismatch count for binade 2^e (-126 < e < 127) into *host_out; 0 on success.
extern "C" int ufp4_test_rcp_mismatches(int e, unsigned int* host_out) {
  if (!host_out || e <= -126 || e >= 127) return -1;
  unsigned int* d = nullptr;
  if (hipMalloc(&d, sizeof(unsigned int)) != hipSuccess) return -2;
  hipError_t err = hipMemset(d, 0, sizeof(unsigned int));
  if (err == hipSuccess) {
    hipLaunchKernelGGL(k_rcp_check, dim3((1u << 23) / 256), dim3(256), 0, 0, e, d);
    err = hipGetLastError();
  }
  if (err == hipSuccess) err = hipMemcpy(host_out, d, sizeof(unsigned int), hipMemcpyDeviceToHost);
  (void)hipFree(d);
  return err == hipSuccess ? 0 : -3;
}
