// Quantizer kernels for the E1M2 codebook (see quant_core.h).
#include "quant_core.h"

namespace ufp4 {

template <>
hipError_t quant_rows_grid<0>(const QuantLaunch& q, hipStream_t s) {
  return qk::run_1d<0, false>(q, s);
}
template <>
hipError_t quant_cols_grid<0>(const QuantLaunch& q, hipStream_t s) {
  return qk::run_1d<0, true>(q, s);
}
template <>
hipError_t quant_rows_2d_grid<0>(const QuantLaunch& q, hipStream_t s) {
  return qk::run_2d<0>(q, s);
}

template <>
hipError_t quant_dual_grid<0>(const QuantLaunch& q, const RowSide& r, hipStream_t s) {
  return qk::run_dual_1d<0>(q, r, s);
}

template <>
hipError_t quant_diag_grid<0>(const QuantLaunch& q, unsigned long long* stats,
                             unsigned long long* partials, hipStream_t s) {
  return qk::run_diag_1d<0>(q, stats, partials, s);
}

}  // namespace ufp4
