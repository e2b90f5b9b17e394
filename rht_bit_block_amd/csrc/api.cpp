// C ABI of the UFP4 hot path: argument validation, launch planning and the
// sign draw.  Validation runs before any HIP call, so every rejected call is
// free of side effects and testable without a GPU.
//
// [UFP4] = "Rethinking Shrinkage Bias in FP4 Pretraining of LLMs ... the UFP4
// Recipe" (hyper.ai summary: formats section, Method).
// [2DFP4] = "Stable FP4 Training via Transposition-Invariant Block
// Quantization" (agifrontier tutorial: 2D square-block quantization).
#include <cmath>
#include <algorithm>
#include <cstring>

#include "../../include/ufp4.h"
#include "ufp4_internal.h"

using namespace ufp4;

namespace {

constexpr uint32_t kSignStream = 0xFFFFFFFFu;

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int check_cfg(const ufp4_quant_cfg* c) {
  if (!c) return UFP4_ERR_INVALID_ARG;
  if (c->grid < 0 || c->grid > 3 || c->rounding < 0 || c->rounding > 1 || c->scale_mode < 0 ||
      c->scale_mode > 1)
    return UFP4_ERR_INVALID_ARG;
  // two-level scaling: a positive, finite, normal per-tensor factor
  if (c->tensor_scale != 0.0f && !(std::isnormal(c->tensor_scale) && c->tensor_scale > 0.0f))
    return UFP4_ERR_INVALID_ARG;
  if (c->tensor_scale != 0.0f && c->scale_mode != UFP4_SCALE_POW2) return UFP4_ERR_UNSUPPORTED;
  if (!is_pow2(c->rht_n) || c->rht_n > 128) return UFP4_ERR_SHAPE;
  if (c->sr_stream == kSignStream) return UFP4_ERR_UNSUPPORTED;
  const bool one_d = c->block_rows == 1 && (c->block_cols == 16 || c->block_cols == 32);
  const bool two_d = c->block_rows == c->block_cols && (c->block_rows == 16 || c->block_rows == 32);
  if (!one_d && !two_d) return UFP4_ERR_UNSUPPORTED;
  // 1D power-of-two scales only for the MX block shape 1 x 32
  if (one_d && c->scale_mode != UFP4_SCALE_F32 && c->block_cols != 32) return UFP4_ERR_UNSUPPORTED;
  // square blocks: power-of-two scales, Hadamard chunks inside a block row
  if (two_d && (c->scale_mode != UFP4_SCALE_POW2 || c->rht_n > c->block_cols))
    return UFP4_ERR_UNSUPPORTED;
  // MXFP8 (E4M3 elements): 1 x 32 power-of-two blocks, round to nearest even
  if (c->grid == UFP4_E4M3 && (!one_d || c->block_cols != 32 || c->scale_mode != UFP4_SCALE_POW2 ||
                               c->rounding != UFP4_RTNE))
    return UFP4_ERR_UNSUPPORTED;
  return UFP4_OK;
}

int lane_width(int n, int bc) { return (bc == 32 || n >= 32) ? 32 : 16; }

// Random signs S_n ([UFP4] Method: H' = S_n H_n): bit i of one Philox block
// keyed by sign_seed at counter (0, 0, 0xFFFFFFFF, 0); bit 1 means -1.  The
// pattern handed to a lane of width W is word q of that block when a chunk
// spans several lanes, else the n-periodic pattern of the first n bits.
void sign_patterns(const ufp4_quant_cfg* c, int W, uint32_t out[4]) {
  uint32_t w[4] = {0u, 0u, kSignStream, 0u};
  philox4x32_10(w, (uint32_t)c->sign_seed, (uint32_t)(c->sign_seed >> 32));
  const int n = c->rht_n;
  if (n == 1) {
    out[0] = out[1] = out[2] = out[3] = 0u;
  } else if (n > W) {
    for (int i = 0; i < 4; ++i) out[i] = w[i];
  } else {
    uint32_t pat = 0;
    for (int j = 0; j < 32; ++j) {
      const int i = j % n;
      pat |= ((w[i >> 5] >> (i & 31)) & 1u) << j;
    }
    out[0] = out[1] = out[2] = out[3] = pat;
  }
}

// Two-level scaling: the multiplier m_T = RN_fp32(1 / s_T) of the rotated
// values (IEEE fp32 division), 1 for single-level scaling.
float tensor_mul(const ufp4_quant_cfg* c) {
  return c->tensor_scale != 0.0f ? 1.0f / c->tensor_scale : 1.0f;
}

// Factor on a GEMM's output: the product of the operands' tensor factors.
float tensor_factor(const ufp4_quant_cfg& c) { return c.tensor_scale != 0.0f ? c.tensor_scale : 1.0f; }

void fill_common(QuantLaunch& q, const void* x, int64_t rows, int64_t cols, int64_t ld,
                 const ufp4_quant_cfg* c, uint8_t* codes, void* scales, float* rotated) {
  std::memset(&q, 0, sizeof(q));
  q.x = reinterpret_cast<const uint16_t*>(x);
  q.ld = ld;
  q.rows = rows;
  q.cols = cols;
  q.codes = codes;
  q.scales = scales;
  q.rotated = rotated;
  q.n = c->rht_n;
  // c_n = RN_fp32(n^-1/2): exact for n = 4^j; for n = 2 * 4^j the double
  // value is far from any fp32 rounding boundary.
  q.cn = (float)(1.0 / std::sqrt((double)c->rht_n));
  q.grid = c->grid;
  q.rounding = c->rounding;
  q.scale_mode = c->scale_mode;
  q.br = c->block_rows;
  q.bc = c->block_cols;
  q.sr_seed = c->sr_seed;
  q.sr_stream = c->sr_stream;
  q.tmul = tensor_mul(c);
  sign_patterns(c, c->block_rows > 1 ? c->block_rows : lane_width(c->rht_n, c->block_cols),
                q.sign_pat);
}

int hip_status(hipError_t e) { return e == hipSuccess ? UFP4_OK : UFP4_ERR_HIP; }

int check_qtensor(const ufp4_qtensor* t) {
  if (!t || t->P < 0 || t->K < 0) return UFP4_ERR_INVALID_ARG;
  // an empty operand may carry null storage
  if ((t->P > 0 && t->K > 0) && (!t->codes || !t->scales)) return UFP4_ERR_INVALID_ARG;
  int st = check_cfg(&t->cfg);
  if (st) return st;
  if (t->K % t->cfg.block_cols || t->K % t->cfg.rht_n || t->P % t->cfg.block_rows)
    return UFP4_ERR_SHAPE;
  if (t->K % 16) return UFP4_ERR_SHAPE;
  if (!aligned(t->codes, 8) || !aligned(t->scales, t->cfg.scale_mode == UFP4_SCALE_F32 ? 4 : 1))
    return UFP4_ERR_INVALID_ARG;
  return UFP4_OK;
}

int check_pair(const ufp4_qtensor* a, const ufp4_qtensor* b) {
  int st = check_qtensor(a);
  if (st) return st;
  st = check_qtensor(b);
  if (st) return st;
  if (a->K != b->K || a->cfg.grid != b->cfg.grid || a->cfg.scale_mode != b->cfg.scale_mode ||
      a->cfg.rht_n != b->cfg.rht_n ||
      (a->cfg.rht_n > 1 && a->cfg.sign_seed != b->cfg.sign_seed))
    return UFP4_ERR_MISMATCH;
  return UFP4_OK;
}

void fill_gemm(GemmLaunch& g, const ufp4_qtensor* a, const ufp4_qtensor* b, float* c, int64_t ldc) {
  std::memset(&g, 0, sizeof(g));
  g.a_codes = a->codes;
  g.a_scales = a->scales;
  g.b_codes = b->codes;
  g.b_scales = b->scales;
  g.c = c;
  g.ldc = ldc;
  g.a_br = a->cfg.block_rows;
  g.a_bc = a->cfg.block_cols;
  g.b_br = b->cfg.block_rows;
  g.b_bc = b->cfg.block_cols;
  g.grid = a->cfg.grid;
  g.scale_mode = a->cfg.scale_mode;
  g.PA = a->P;
  g.PB = b->P;
  g.K = a->K;
  g.c_mul = tensor_factor(a->cfg) * tensor_factor(b->cfg);   // two-level: s_TA * s_TB
}

constexpr int64_t kTile = 256;
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// FP6 workspace bytes a GEMM of A and B described by `g` can use (0: none).
int64_t fp6_bytes(const ufp4_qtensor* A, const ufp4_qtensor* B, const GemmLaunch& g) {
  if (!aligned(A->codes, 16) || !aligned(B->codes, 16) || !aligned(A->scales, 4) ||
      !aligned(B->scales, 4))
    return 0;
  return gemm_mx6_supported(g) ? gemm_mx6_workspace(g) : 0;
}

int64_t dense_fp6_bytes(const ufp4_qtensor* A, const ufp4_qtensor* B) {
  if (check_pair(A, B) || A->P == 0 || B->P == 0 || A->K == 0) return 0;
  GemmLaunch g;
  fill_gemm(g, A, B, nullptr, B->P);
  g.mode = 0;
  return fp6_bytes(A, B, g);
}

// The scaled-MFMA kernels take this launch (shape, blocks and alignment).
bool mx_route(const GemmLaunch& g) {
  return gemm_mx_supported(g) && aligned(g.a_scales, 4) && aligned(g.b_scales, 4) &&
         aligned(g.a_codes, 16) && aligned(g.b_codes, 16);
}

// Launch of a filled GemmLaunch: FP6 operands through the workspace when one
// is given and the operands qualify, else the scaled matrix cores for
// E8M0 blocks they take, else the general kernels.
int launch_any(const ufp4_qtensor* A, const ufp4_qtensor* B, const GemmLaunch& g, void* ws,
               size_t ws_bytes, void* stream) {
  if (ws) {
    const int64_t need = fp6_bytes(A, B, g);
    if (need > 0) {
      if ((uint64_t)need > (uint64_t)ws_bytes || !aligned(ws, 256)) return UFP4_ERR_INVALID_ARG;
      return hip_status(launch_gemm_mx6(g, static_cast<uint8_t*>(ws), (hipStream_t)stream));
    }
  }
  if (mx_route(g)) return hip_status(launch_gemm_mx(g, (hipStream_t)stream));
  if (g.grid == UFP4_E4M3) return UFP4_ERR_UNSUPPORTED;   // MXFP8 runs on the scaled MFMA only
  return hip_status(launch_gemm(g, (hipStream_t)stream));
}

// Dense C = A B^T.  With a workspace (ws != null) E1M2 / INT4 operands with
// 32-element E8M0 blocks run as FP6 operands; every other case ignores it.
int gemm_dense(const ufp4_qtensor* A, const ufp4_qtensor* B, float* C, int64_t ldc, void* stream,
               void* ws = nullptr, size_t ws_bytes = 0) {
  int st = check_pair(A, B);
  if (st) return st;
  if (ldc < B->P) return UFP4_ERR_INVALID_ARG;
  if (A->P == 0 || B->P == 0) return UFP4_OK;
  if (!C) return UFP4_ERR_INVALID_ARG;
  // empty shared dimension: C = 0, no operand storage is read (it may be null)
  if (A->K == 0) return hip_status(launch_zero_c(C, A->P, B->P, ldc, (hipStream_t)stream));
  GemmLaunch g;
  fill_gemm(g, A, B, C, ldc);
  g.mode = 0;
  g.ngroups = 1;
  const int64_t tiles = cdiv(A->P, kTile) * cdiv(B->P, kTile);
  if (tiles > INT32_MAX) return UFP4_ERR_UNSUPPORTED;
  g.tile_start[0] = 0;
  g.tile_start[1] = (int32_t)tiles;
  g.total_tiles = (int32_t)tiles;
  return launch_any(A, B, g, ws, ws_bytes, stream);
}

int check_offsets(const int64_t* off, int32_t G, int64_t total, int64_t align) {
  if (!off || G < 1 || G > kMaxGroups) return UFP4_ERR_INVALID_ARG;
  if (off[0] != 0 || off[G] != total) return UFP4_ERR_INVALID_ARG;
  for (int i = 0; i < G; ++i) {
    if (off[i + 1] < off[i]) return UFP4_ERR_INVALID_ARG;
    if (off[i] % align) return UFP4_ERR_SHAPE;
  }
  return UFP4_OK;
}

// Grouped along A's rows: fprop (B = W stacked) and dgrad (B = W^T stacked).
int gemm_grouped_rows(const ufp4_qtensor* A, const ufp4_qtensor* B, int32_t G,
                      const int64_t* off, float* C, int64_t ldc, void* stream,
                      void* ws = nullptr, size_t ws_bytes = 0) {
  int st = check_pair(A, B);
  if (st) return st;
  if (A->cfg.grid == UFP4_E4M3) return UFP4_ERR_UNSUPPORTED;
  if (G < 1 || G > kMaxGroups || B->P % G) return G < 1 || G > kMaxGroups ? UFP4_ERR_INVALID_ARG
                                                                          : UFP4_ERR_SHAPE;
  st = check_offsets(off, G, A->P, A->cfg.block_rows);
  if (st) return st;
  const int64_t R = B->P / G;
  if (!C || ldc < R) return UFP4_ERR_INVALID_ARG;
  if (A->K == 0) return hip_status(launch_zero_c(C, A->P, R, ldc, (hipStream_t)stream));
  GemmLaunch g;
  fill_gemm(g, A, B, C, ldc);
  g.mode = 1;
  g.ngroups = G;
  g.b_rows_per_group = R;
  int64_t t = 0;
  for (int i = 0; i < G; ++i) {
    g.off[i] = off[i];
    g.tile_start[i] = (int32_t)t;
    t += cdiv(off[i + 1] - off[i], kTile) * cdiv(R, kTile);
    if (t > INT32_MAX) return UFP4_ERR_UNSUPPORTED;
  }
  g.off[G] = off[G];
  g.tile_start[G] = (int32_t)t;
  g.total_tiles = (int32_t)t;
  return launch_any(A, B, g, ws, ws_bytes, stream);
}

// K-grouped launch (every group `per` tiles, a tile's cost proportional to its
// segment): keep contiguous XCD ranges of whole groups unless the busiest of
// the 8 ranges has over 5 % more work than the mean; then deal runs of tiles
// (an eighth of a group, or one column of its grouped order, tiles_m tiles at
// most 8) to the XCDs in turn, groups longest first.
void plan_deal(GemmLaunch& g, int64_t per, int64_t tiles_m) {
  const int G = g.ngroups;
  const int64_t T = g.total_tiles;
  double work[8] = {}, total = 0;
  for (int x = 0; x < 8; ++x) {
    const int64_t lo = x * (T / 8) + std::min<int64_t>(x, T % 8);
    const int64_t hi = lo + T / 8 + (x < T % 8 ? 1 : 0);
    for (int grp = 0; grp < G; ++grp) {
      const int64_t a = std::max<int64_t>(lo, grp * per), b = std::min<int64_t>(hi, (grp + 1) * per);
      if (b > a) work[x] += (double)(b - a) * (double)(g.off[grp + 1] - g.off[grp]);
    }
    total += work[x];
  }
  double worst = 0;
  for (int x = 0; x < 8; ++x) worst = std::max(worst, work[x]);
  g.deal = 0;
  if (total <= 0 || worst <= 1.05 * total / 8) return;
  g.deal = (int32_t)(per % 8 == 0 ? per / 8 : std::min<int64_t>(8, tiles_m));
  for (int i = 0; i < G; ++i) g.gorder[i] = i;
  std::stable_sort(g.gorder, g.gorder + G, [&](int32_t x, int32_t y) {
    return g.off[x + 1] - g.off[x] > g.off[y + 1] - g.off[y];
  });
}

// Grouped along K: wgrad (segmented column-wise operands).  fp32 scales run
// on the general kernels; 1 x 32 E8M0 blocks on the scaled matrix cores when
// every segment length is a multiple of 128, else UFP4_ERR_UNSUPPORTED.
int gemm_grouped_k(const ufp4_qtensor* dYt, const ufp4_qtensor* Xt, int32_t G,
                   const int64_t* offsets, float* dW, int64_t ldw, void* stream,
                   void* ws = nullptr, size_t ws_bytes = 0) {
  int st = check_pair(dYt, Xt);
  if (st) return st;
  if (dYt->cfg.grid == UFP4_E4M3) return UFP4_ERR_UNSUPPORTED;
  if (dYt->cfg.block_rows != 1 || Xt->cfg.block_rows != 1) return UFP4_ERR_UNSUPPORTED;
  const int64_t align = 16;
  st = check_offsets(offsets, G, dYt->K, align);
  if (st) return st;
  for (int i = 0; i < G; ++i) {
    const int64_t L = offsets[i + 1] - offsets[i];
    if (L % dYt->cfg.block_cols || L % Xt->cfg.block_cols || L % dYt->cfg.rht_n || L % 16)
      return UFP4_ERR_SHAPE;
  }
  if (!dW || ldw < Xt->P) return UFP4_ERR_INVALID_ARG;
  if (dYt->P == 0 || Xt->P == 0) return UFP4_OK;
  GemmLaunch g;
  fill_gemm(g, dYt, Xt, dW, ldw);
  g.mode = 2;
  g.ngroups = G;
  const int64_t per = cdiv(dYt->P, kTile) * cdiv(Xt->P, kTile);
  if (per * G > INT32_MAX) return UFP4_ERR_UNSUPPORTED;
  for (int i = 0; i <= G; ++i) {
    g.off[i] = offsets[i];
    g.tile_start[i] = (int32_t)(per * i);
  }
  g.total_tiles = (int32_t)(per * G);
  plan_deal(g, per, cdiv(dYt->P, kTile));
  // the general kernels take fp32 scales only when grouped along K
  if (g.scale_mode == UFP4_SCALE_POW2 && !(mx_route(g) || (ws && fp6_bytes(dYt, Xt, g) > 0)))
    return UFP4_ERR_UNSUPPORTED;
  return launch_any(dYt, Xt, g, ws, ws_bytes, stream);
}

}  // namespace

namespace ufp4 {

static_assert(kDiagWorkspaceBytes == UFP4_DIAG_WORKSPACE_BYTES, "diagnostics workspace size");

// Validation and launch description of a level-statistics call (shared by
// ufp4_quant_diag and its variant on the library's own scratch array).
int diag_prepare(const void* x, int64_t rows, int64_t cols, int64_t ld, const ufp4_quant_cfg* cfg,
                 const uint64_t* stats, QuantLaunch& q) {
  if (rows < 0 || cols < 0 || (rows > 0 && ld < cols)) return UFP4_ERR_INVALID_ARG;
  int st = check_cfg(cfg);
  if (st) return st;
  if (!stats || !aligned(stats, 8)) return UFP4_ERR_INVALID_ARG;
  if (cfg->block_rows != 1 || cfg->grid == UFP4_E4M3) return UFP4_ERR_UNSUPPORTED;
  const int64_t P = rows, K = cols;
  if (P > 0 && K > 0) {
    if (!x) return UFP4_ERR_INVALID_ARG;
    if (K % cfg->rht_n || K % cfg->block_cols) return UFP4_ERR_SHAPE;
    if (!aligned(x, 16) || ld % 8) return UFP4_ERR_INVALID_ARG;
    const int W = lane_width(cfg->rht_n, cfg->block_cols);
    if (P * (K / W) > (int64_t)UINT32_MAX || K > (int64_t)UINT32_MAX) return UFP4_ERR_UNSUPPORTED;
  }
  fill_common(q, x, rows, cols, ld, cfg, nullptr, nullptr, nullptr);
  q.P = P;
  q.K = K;
  return UFP4_OK;
}

}  // namespace ufp4

extern "C" {

const char* ufp4_status_string(int status) {
  switch (status) {
    case UFP4_OK: return "ok";
    case UFP4_ERR_INVALID_ARG: return "invalid argument";
    case UFP4_ERR_SHAPE: return "shape not divisible by rht_n / block size";
    case UFP4_ERR_MISMATCH: return "GEMM operands disagree (K, grid, scale mode or rotation)";
    case UFP4_ERR_UNSUPPORTED: return "unsupported combination";
    case UFP4_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

size_t ufp4_codes_bytes(int64_t P, int64_t K) {
  if (P < 0 || K < 0) return 0;
  return (size_t)P * (size_t)((K + 1) / 2);
}

size_t ufp4_scales_bytes(int64_t P, int64_t K, const ufp4_quant_cfg* cfg) {
  if (!cfg || P < 0 || K < 0 || cfg->block_rows < 1 || cfg->block_cols < 1) return 0;
  const size_t nb = (size_t)cdiv(P, cfg->block_rows) * (size_t)cdiv(K, cfg->block_cols);
  return nb * (cfg->scale_mode == UFP4_SCALE_F32 ? 4 : 1);
}

int ufp4_rht_quant(const void* x, int64_t rows, int64_t cols, int64_t ld, int32_t along,
                   const ufp4_quant_cfg* cfg, uint8_t* codes, void* scales, float* rotated,
                   void* stream) {
  if (rows < 0 || cols < 0 || (rows > 0 && ld < cols) || (along != 0 && along != 1))
    return UFP4_ERR_INVALID_ARG;
  int st = check_cfg(cfg);
  if (st) return st;
  const int64_t P = along ? cols : rows, K = along ? rows : cols;
  if (P == 0 || K == 0) return UFP4_OK;  // empty: nothing to read or write
  if (!x || !codes || !scales) return UFP4_ERR_INVALID_ARG;
  if (K % cfg->rht_n || K % cfg->block_cols || P % cfg->block_rows) return UFP4_ERR_SHAPE;
  if (!aligned(x, 16) || ld % 8 || !aligned(codes, 16) || !aligned(scales, 4) ||
      (rotated && !aligned(rotated, 16)))
    return UFP4_ERR_INVALID_ARG;
  const int64_t bs = cfg->block_rows;       // square block size; 1 for 1D blocks
  const bool two_d = bs > 1;
  if (two_d && along == 1) return UFP4_ERR_UNSUPPORTED;  // quantize once, then transpose
  QuantLaunch q;
  fill_common(q, x, rows, cols, ld, cfg, codes, scales, rotated);
  q.P = P;
  q.K = K;
  if (two_d) {
    if ((P / bs) * cdiv(K / bs, 64 / bs) > (int64_t)UINT32_MAX) return UFP4_ERR_UNSUPPORTED;
    return hip_status(launch_quant_rows_2d(q, (hipStream_t)stream));
  }
  if (along == 0) {
    const int W = lane_width(cfg->rht_n, cfg->block_cols);
    if (P * (K / W) > (int64_t)UINT32_MAX || K > (int64_t)UINT32_MAX) return UFP4_ERR_UNSUPPORTED;
    return hip_status(launch_quant_rows(q, (hipStream_t)stream));
  }
  // column-wise: one segment covering all rows
  q.nseg = 1;
  q.seg_off[0] = 0;
  q.seg_off[1] = rows;
  const int64_t tiles = cdiv(rows, 128) * cdiv(cols, 64);
  if (tiles > INT32_MAX) return UFP4_ERR_UNSUPPORTED;
  q.tile_start[0] = 0;
  q.tile_start[1] = (int32_t)tiles;
  return hip_status(launch_quant_cols(q, (hipStream_t)stream));
}

int ufp4_quant_diag(const void* x, int64_t rows, int64_t cols, int64_t ld,
                    const ufp4_quant_cfg* cfg, uint64_t* stats, void* workspace,
                    void* stream) {
  QuantLaunch q;
  const int st = ufp4::diag_prepare(x, rows, cols, ld, cfg, stats, q);
  if (st) return st;
  if (!workspace || !aligned(workspace, 8)) return UFP4_ERR_INVALID_ARG;
  // an empty operand still zeroes stats (the zeroing kernel runs first)
  return hip_status(launch_quant_diag(q, reinterpret_cast<unsigned long long*>(stats),
                                      reinterpret_cast<unsigned long long*>(workspace),
                                      (hipStream_t)stream));
}

int ufp4_rht_quant_dual(const void* x, int64_t rows, int64_t cols, int64_t ld,
                        const int64_t* row_offsets, int32_t num_segments,
                        const ufp4_quant_cfg* cfg_row, const ufp4_quant_cfg* cfg_col,
                        uint8_t* codes_row, void* scales_row, uint8_t* codes_col,
                        void* scales_col, void* stream) {
  if (rows < 0 || cols < 0 || (rows > 0 && ld < cols)) return UFP4_ERR_INVALID_ARG;
  if (row_offsets && (num_segments < 1 || num_segments > kMaxSegments))
    return UFP4_ERR_INVALID_ARG;
  int st = check_cfg(cfg_row);
  if (st) return st;
  st = check_cfg(cfg_col);
  if (st) return st;
  // one kernel instance serves both sides: they may differ only in signs and draws
  if (cfg_row->block_rows != 1 || cfg_col->block_rows != 1 || cfg_row->grid != cfg_col->grid ||
      cfg_row->rounding != cfg_col->rounding || cfg_row->scale_mode != cfg_col->scale_mode ||
      cfg_row->block_cols != cfg_col->block_cols || cfg_row->rht_n != cfg_col->rht_n ||
      cfg_row->grid == UFP4_E4M3)
    return UFP4_ERR_UNSUPPORTED;
  const int64_t n = cfg_row->rht_n, b = cfg_row->block_cols;
  const int64_t align = n > b ? n : b;
  const int nseg = row_offsets ? num_segments : 1;
  if (row_offsets) {
    if (row_offsets[0] != 0 || row_offsets[nseg] != rows) return UFP4_ERR_INVALID_ARG;
    for (int g = 0; g < nseg; ++g) {
      if (row_offsets[g + 1] < row_offsets[g]) return UFP4_ERR_INVALID_ARG;
      if ((row_offsets[g + 1] - row_offsets[g]) % align) return UFP4_ERR_SHAPE;
    }
  } else if (rows % align) {
    return UFP4_ERR_SHAPE;
  }
  if (cols % align) return UFP4_ERR_SHAPE;
  if (rows == 0 || cols == 0) return UFP4_OK;
  if (!x || !codes_row || !scales_row || !codes_col || !scales_col) return UFP4_ERR_INVALID_ARG;
  if (!aligned(x, 16) || ld % 8 || !aligned(codes_row, 16) || !aligned(scales_row, 4) ||
      !aligned(codes_col, 16) || !aligned(scales_col, 4))
    return UFP4_ERR_INVALID_ARG;
  QuantLaunch q;
  fill_common(q, x, rows, cols, ld, cfg_col, codes_col, scales_col, nullptr);
  q.P = cols;
  q.K = rows;
  q.nseg = nseg;
  int64_t t = 0;
  const int64_t tp = cdiv(cols, dual_tile_cols(cfg_row->rht_n));
  for (int g = 0; g < nseg; ++g) {
    const int64_t a = row_offsets ? row_offsets[g] : 0, e = row_offsets ? row_offsets[g + 1] : rows;
    q.seg_off[g] = a;
    q.tile_start[g] = (int32_t)t;
    t += cdiv(e - a, 128) * tp;
    if (t > INT32_MAX) return UFP4_ERR_UNSUPPORTED;
  }
  q.seg_off[nseg] = rows;
  q.tile_start[nseg] = (int32_t)t;
  RowSide r;
  std::memset(&r, 0, sizeof(r));
  r.codes = codes_row;
  r.scales = scales_row;
  r.rotated = nullptr;
  r.cn = q.cn;
  r.sr_seed = cfg_row->sr_seed;
  r.sr_stream = cfg_row->sr_stream;
  r.tmul = tensor_mul(cfg_row);
  sign_patterns(cfg_row, lane_width(cfg_row->rht_n, cfg_row->block_cols), r.sign_pat);
  return hip_status(launch_quant_dual(q, r, (hipStream_t)stream));
}

int ufp4_rht_quant_segmented(const void* x, int64_t rows, int64_t cols, int64_t ld,
                             const int64_t* row_offsets, int32_t num_segments,
                             const ufp4_quant_cfg* cfg, uint8_t* codes, void* scales,
                             void* stream) {
  if (!row_offsets) return UFP4_ERR_INVALID_ARG;
  if (rows < 0 || cols < 0 || (rows > 0 && ld < cols)) return UFP4_ERR_INVALID_ARG;
  if (num_segments < 1 || num_segments > kMaxSegments) return UFP4_ERR_INVALID_ARG;
  int st = check_cfg(cfg);
  if (st) return st;
  if (cfg->block_rows != 1 || cfg->grid == UFP4_E4M3) return UFP4_ERR_UNSUPPORTED;
  if (row_offsets[0] != 0 || row_offsets[num_segments] != rows) return UFP4_ERR_INVALID_ARG;
  const int64_t align = cfg->rht_n > cfg->block_cols ? cfg->rht_n : cfg->block_cols;
  for (int g = 0; g < num_segments; ++g) {
    if (row_offsets[g + 1] < row_offsets[g]) return UFP4_ERR_INVALID_ARG;
    if ((row_offsets[g + 1] - row_offsets[g]) % align) return UFP4_ERR_SHAPE;
  }
  if (rows == 0 || cols == 0) return UFP4_OK;
  if (!x || !codes || !scales) return UFP4_ERR_INVALID_ARG;
  if (!aligned(x, 16) || ld % 8 || !aligned(codes, 16) || !aligned(scales, 4))
    return UFP4_ERR_INVALID_ARG;
  QuantLaunch q;
  fill_common(q, x, rows, cols, ld, cfg, codes, scales, nullptr);
  q.P = cols;
  q.K = rows;
  q.nseg = num_segments;
  int64_t t = 0;
  const int64_t tp = cdiv(cols, 64);
  for (int g = 0; g < num_segments; ++g) {
    q.seg_off[g] = row_offsets[g];
    q.tile_start[g] = (int32_t)t;
    t += cdiv(row_offsets[g + 1] - row_offsets[g], 128) * tp;
    if (t > INT32_MAX) return UFP4_ERR_UNSUPPORTED;
  }
  q.seg_off[num_segments] = row_offsets[num_segments];
  q.tile_start[num_segments] = (int32_t)t;
  return hip_status(launch_quant_cols(q, (hipStream_t)stream));
}

int ufp4_dequant(const ufp4_qtensor* q, float* out, int64_t ldo, void* stream) {
  int st = check_qtensor(q);
  if (st) return st;
  if (ldo < q->K) return UFP4_ERR_INVALID_ARG;
  if (q->P == 0 || q->K == 0) return UFP4_OK;
  if (!out) return UFP4_ERR_INVALID_ARG;
  if (!aligned(q->codes, q->cfg.grid == UFP4_E4M3 ? 8 : 4)) return UFP4_ERR_INVALID_ARG;
  return hip_status(launch_dequant(q->codes, q->scales, q->P, q->K, q->cfg.grid,
                                   q->cfg.scale_mode, q->cfg.block_rows, q->cfg.block_cols,
                                   tensor_factor(q->cfg), out, ldo, (hipStream_t)stream));
}

int ufp4_gemm_fprop(const ufp4_qtensor* X, const ufp4_qtensor* W, float* Y, int64_t ldy,
                    void* stream) {
  return gemm_dense(X, W, Y, ldy, stream);
}

int ufp4_gemm_dgrad(const ufp4_qtensor* dY, const ufp4_qtensor* Wt, float* dX, int64_t ldx,
                    void* stream) {
  return gemm_dense(dY, Wt, dX, ldx, stream);
}

int ufp4_gemm_wgrad(const ufp4_qtensor* dYt, const ufp4_qtensor* Xt, float* dW, int64_t ldw,
                    void* stream) {
  return gemm_dense(dYt, Xt, dW, ldw, stream);
}

int ufp4_gemm_fprop_grouped(const ufp4_qtensor* Xp, const ufp4_qtensor* W, int32_t G,
                            const int64_t* offsets, float* Y, int64_t ldy, void* stream) {
  return gemm_grouped_rows(Xp, W, G, offsets, Y, ldy, stream);
}

int ufp4_gemm_dgrad_grouped(const ufp4_qtensor* dYp, const ufp4_qtensor* Wt, int32_t G,
                            const int64_t* offsets, float* dX, int64_t ldx, void* stream) {
  return gemm_grouped_rows(dYp, Wt, G, offsets, dX, ldx, stream);
}

int ufp4_gemm_wgrad_grouped(const ufp4_qtensor* dYt, const ufp4_qtensor* Xt, int32_t G,
                            const int64_t* offsets, float* dW, int64_t ldw, void* stream) {
  return gemm_grouped_k(dYt, Xt, G, offsets, dW, ldw, stream);
}

size_t ufp4_gemm_workspace_bytes(int32_t op, const ufp4_qtensor* A, const ufp4_qtensor* B,
                                 int32_t G) {
  if (op < UFP4_GEMM_FPROP || op > UFP4_GEMM_WGRAD || G < 0 || G > kMaxGroups) return 0;
  if (G == 0) return (size_t)dense_fp6_bytes(A, B);
  if (check_pair(A, B) || A->P == 0 || B->P == 0 || A->K == 0) return 0;
  GemmLaunch g;
  fill_gemm(g, A, B, nullptr, B->P);
  g.ngroups = 1;
  if (op == UFP4_GEMM_WGRAD) {   // segment lengths are the call's to check
    g.mode = 2;
    g.off[0] = 0;
    g.off[1] = A->K;
  } else {
    if (B->P % G) return 0;
    g.mode = 1;
    g.ngroups = G;
    g.b_rows_per_group = B->P / G;
  }
  return (size_t)fp6_bytes(A, B, g);
}

int ufp4_gemm_ws(int32_t op, const ufp4_qtensor* A, const ufp4_qtensor* B, int32_t G,
                 const int64_t* offsets, float* C, int64_t ldc, void* workspace,
                 size_t workspace_bytes, void* stream) {
  if (op < UFP4_GEMM_FPROP || op > UFP4_GEMM_WGRAD || G < 0) return UFP4_ERR_INVALID_ARG;
  if (!workspace && workspace_bytes) return UFP4_ERR_INVALID_ARG;
  if (G == 0) return gemm_dense(A, B, C, ldc, stream, workspace, workspace_bytes);
  if (op == UFP4_GEMM_WGRAD)
    return gemm_grouped_k(A, B, G, offsets, C, ldc, stream, workspace, workspace_bytes);
  return gemm_grouped_rows(A, B, G, offsets, C, ldc, stream, workspace, workspace_bytes);
}

int ufp4_transpose_qtensor(const ufp4_qtensor* src, uint8_t* dst_codes, void* dst_scales,
                           void* stream) {
  int st = check_qtensor(src);
  if (st) return st;
  if (!dst_codes || !dst_scales) return UFP4_ERR_INVALID_ARG;
  const int b = src->cfg.block_rows;
  if (b != src->cfg.block_cols || src->cfg.rht_n != 1) return UFP4_ERR_UNSUPPORTED;
  if (src->P % 2 || src->K % 2) return UFP4_ERR_SHAPE;
  return hip_status(launch_transpose(src->codes, src->scales, src->P, src->K, b,
                                     src->cfg.scale_mode, dst_codes, dst_scales,
                                     (hipStream_t)stream));
}

int ufp4_stream_copy(const void* src, void* dst, int64_t nbytes, void* stream) {
  if (nbytes < 0) return UFP4_ERR_INVALID_ARG;
  if (nbytes == 0) return UFP4_OK;
  if (!src || !dst) return UFP4_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16)
    return UFP4_ERR_INVALID_ARG;
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  if (a < b + (uintptr_t)nbytes && b < a + (uintptr_t)nbytes) return UFP4_ERR_INVALID_ARG;
  return hip_status(launch_stream_copy(src, dst, nbytes, (hipStream_t)stream));
}

int ufp4_philox_fill(uint64_t seed, uint32_t stream_id, uint64_t first, int64_t n,
                     uint16_t* out, void* stream) {
  if (!out || n < 0) return UFP4_ERR_INVALID_ARG;
  if (stream_id == kSignStream) return UFP4_ERR_UNSUPPORTED;
  return hip_status(launch_philox_fill(seed, stream_id, first, n, out, (hipStream_t)stream));
}

}  // extern "C"
