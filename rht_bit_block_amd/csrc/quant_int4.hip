// Quantizer kernels for the INT4 codebook (see quant_core.h).
#include "quant_core.h"

namespace ufp4 {

template <>
hipError_t quant_rows_grid<1>(const QuantLaunch& q, hipStream_t s) {
  return qk::run_1d<1, false>(q, s);
}
template <>
hipError_t quant_cols_grid<1>(const QuantLaunch& q, hipStream_t s) {
  return qk::run_1d<1, true>(q, s);
}
template <>
hipError_t quant_rows_2d_grid<1>(const QuantLaunch& q, hipStream_t s) {
  return qk::run_2d<1>(q, s);
}

template <>
hipError_t quant_dual_grid<1>(const QuantLaunch& q, const RowSide& r, hipStream_t s) {
  return qk::run_dual_1d<1>(q, r, s);
}

template <>
hipError_t quant_diag_grid<1>(const QuantLaunch& q, unsigned long long* stats,
                             unsigned long long* partials, hipStream_t s) {
  return qk::run_diag_1d<1>(q, stats, partials, s);
}

}  // namespace ufp4
