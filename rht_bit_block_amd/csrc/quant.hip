// Quantizer dispatch by codebook; the kernels live in quant_core.h and are
// compiled per codebook in quant_e1m2.hip, quant_int4.hip, quant_e2m1.hip and
// quant_e4m3.hip (MXFP8: row- and column-wise 1 x 32 only).
#include "quant_core.h"

namespace ufp4 {

hipError_t launch_quant_rows(const QuantLaunch& q, hipStream_t s) {
  switch (q.grid) {
    case 0: return quant_rows_grid<0>(q, s);
    case 1: return quant_rows_grid<1>(q, s);
    case 3: return quant_rows_grid<3>(q, s);
    default: return quant_rows_grid<2>(q, s);
  }
}

hipError_t launch_quant_cols(const QuantLaunch& q, hipStream_t s) {
  switch (q.grid) {
    case 0: return quant_cols_grid<0>(q, s);
    case 1: return quant_cols_grid<1>(q, s);
    case 3: return quant_cols_grid<3>(q, s);
    default: return quant_cols_grid<2>(q, s);
  }
}

hipError_t launch_quant_rows_2d(const QuantLaunch& q, hipStream_t s) {
  switch (q.grid) {
    case 0: return quant_rows_2d_grid<0>(q, s);
    case 1: return quant_rows_2d_grid<1>(q, s);
    default: return quant_rows_2d_grid<2>(q, s);
  }
}

hipError_t launch_quant_dual(const QuantLaunch& q, const RowSide& r, hipStream_t s) {
  switch (q.grid) {
    case 0: return quant_dual_grid<0>(q, r, s);
    case 1: return quant_dual_grid<1>(q, r, s);
    default: return quant_dual_grid<2>(q, r, s);
  }
}

hipError_t launch_quant_diag(const QuantLaunch& q, unsigned long long* stats,
                             unsigned long long* partials, hipStream_t s) {
  switch (q.grid) {
    case 0: return quant_diag_grid<0>(q, stats, partials, s);
    case 1: return quant_diag_grid<1>(q, stats, partials, s);
    default: return quant_diag_grid<2>(q, stats, partials, s);
  }
}

}  // namespace ufp4
