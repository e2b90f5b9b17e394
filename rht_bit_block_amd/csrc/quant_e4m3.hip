// Quantizer kernels for the MXFP8 codebook (OCP E4M3 elements, one byte per
// code, 1 x 32 power-of-two scales, RTNE; see quant_core.h).  [2DFP4] =
// "Stable FP4 Training via Transposition-Invariant Block Quantization"
// (mixed-precision section: the Query/Key projections stay in MXFP8).
#include "quant_core.h"

namespace ufp4 {
namespace qk {

template <bool COLS>
hipError_t run_e4m3(const QuantLaunch& q, hipStream_t s) {
  if (q.bc != 32 || q.scale_mode != 1 || q.rounding != 0) return hipErrorInvalidValue;
#define UFP4_RUN(N_) \
  if (q.n == N_) return COLS ? run_cols<32, 32, N_, 3, 2>(q, s) : run_rows<32, 32, N_, 3, 2>(q, s);
  UFP4_RUN(1) UFP4_RUN(2) UFP4_RUN(4) UFP4_RUN(8) UFP4_RUN(16) UFP4_RUN(32) UFP4_RUN(64)
  UFP4_RUN(128)
#undef UFP4_RUN
  return hipErrorInvalidValue;
}

}  // namespace qk

template <>
hipError_t quant_rows_grid<3>(const QuantLaunch& q, hipStream_t s) {
  return qk::run_e4m3<false>(q, s);
}
template <>
hipError_t quant_cols_grid<3>(const QuantLaunch& q, hipStream_t s) {
  return qk::run_e4m3<true>(q, s);
}

}  // namespace ufp4
