/*
 * ufp4.h -- C ABI of the MI355X (gfx950) UFP4 hot path: fused random
 * Hadamard transform + blockwise 4-bit quantizer, dequantizer, and the
 * block-scaled 4-bit GEMMs FPROP / DGRAD / WGRAD (dense and grouped for MoE).
 *
 * Pages (cited by title, section and equation):
 *   [UFP4]  "Rethinking Shrinkage Bias in FP4 Pretraining of LLMs: Geometric
 *           Origin, Systemic Impact and the UFP4 Recipe" -- hyper.ai summary
 *           (formats and blockwise quantization; Method) and abstract.
 *   [2DFP4] "Stable FP4 Training via Transposition-Invariant Block
 *           Quantization" -- agifrontier tutorial (root cause; 2D square-block
 *           quantization).
 *
 * Conventions shared by every entry point
 *   - Pointers named x, codes, scales, rotated, out, workspace, Y, dX, dW
 *     are DEVICE pointers owned by the caller; arrays named *_offsets are
 *     HOST arrays.  The library allocates no memory and keeps no data
 *     between calls (only per-device kernel attributes and compute-unit
 *     counts, each set or read once), so every
 *     entry point is safe to call from several host threads and on several
 *     streams at once, as long as the calls do not write the same buffers
 *     (workspaces included).  The one exception is ufp4_quant_diag_noalloc,
 *     whose partial sums live in a per-GPU array of the library: its calls
 *     on one GPU must not overlap.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *     default stream).  Nothing synchronizes inside the library.
 *   - Every function returns UFP4_OK (0) or a negative status; arguments are
 *     validated before any HIP call, so a rejected call has no side effect.
 *     ufp4_status_string() names a status.  Nothing is thrown across the ABI.
 *   - A "logical operand" A is P x K with K the dimension a GEMM contracts.
 *     Quantized operands are stored K-contiguous:
 *       codes  : uint8 [P][K/2]; byte j of a row holds the 4-bit codes of
 *                elements 2j (low nibble) and 2j+1 (high nibble);
 *       scales : UFP4_SCALE_F32  -> float [P/block_rows][K/block_cols]
 *                UFP4_SCALE_POW2 -> uint8 E8M0 [P/block_rows][K/block_cols],
 *                                   value 2^(byte - 127).
 *   - Code nibbles: E1M2 and E2M1 are sign-magnitude (sign*8 + level index;
 *     E2M1 is the OCP FP4 bit pattern), INT4 is two's complement of -7..7;
 *     zero is always code 0.
 */
#ifndef UFP4_H
#define UFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Codebooks G ([UFP4] formats section; uniform grids in Method):
 * E1M2 levels {0, +-0.25, ..., +-1.75}, INT4 {-7..7},
 * E2M1 {0, +-0.5, +-1, +-1.5, +-2, +-3, +-4, +-6}.
 * E4M3 is the MXFP8 element format ([2DFP4] mixed-precision section keeps
 * the Query/Key projections in MXFP8): every finite OCP FP8 E4M3 value
 * (|v| <= 448), one byte per code (the OCP bit pattern, zero as 0x00), only
 * with 1 x 32 power-of-two scales and RTNE (ties to the even pattern); its
 * codes take P*K bytes (ufp4_codes_bytes covers the 4-bit codebooks).  Its
 * quantizations are row- or column-wise (ufp4_rht_quant) and its GEMMs dense
 * with K % 128 == 0; other entry points return UFP4_ERR_UNSUPPORTED. */
enum { UFP4_E1M2 = 0, UFP4_INT4 = 1, UFP4_E2M1 = 2, UFP4_E4M3 = 3 };
/* Rounding ([UFP4] formats section; [2DFP4] 2D section, E[roundS(x)] = x). */
enum { UFP4_RTNE = 0, UFP4_SR = 1 };
/* Scale rule: s_B = absmax / qmax in fp32 ([UFP4] formats section), or the
 * truncation-free power of two S = 2^ceil(log2(2M / (Qp - Qn))) ([2DFP4]). */
enum { UFP4_SCALE_F32 = 0, UFP4_SCALE_POW2 = 1 };

enum {
  UFP4_OK = 0,
  UFP4_ERR_INVALID_ARG = -1,  /* null pointer, negative size, bad enum     */
  UFP4_ERR_SHAPE = -2,        /* sizes not divisible by rht_n / blocks      */
  UFP4_ERR_MISMATCH = -3,     /* GEMM operands disagree (K, rotation, grid) */
  UFP4_ERR_UNSUPPORTED = -4,  /* valid but not implemented combination      */
  UFP4_ERR_HIP = -5           /* the HIP runtime reported an error          */
};

/* Parameters of one quantization.
 *   grid, rounding, scale_mode : the enums above.
 *   block_rows x block_cols    : 1 x 16 or 1 x 32 (1D groups along K,
 *                                [2DFP4] root cause), or 16 x 16 or 32 x 32
 *                                square blocks ([2DFP4] 2D section; its
 *                                block-size comparison favours 16 to 32).
 *                                Power-of-two scales go with square blocks
 *                                or 1 x 32 blocks (the OCP-MX block: one
 *                                E8M0 byte per row and 32 elements); fp32
 *                                scales with 1 x 16 or 1 x 32 blocks; any
 *                                other pairing is UFP4_ERR_UNSUPPORTED.
 *   rht_n     : Hadamard size along K, a power of two in [1, 128]; 1 = no
 *               rotation ([UFP4] Method, Sylvester recursion).  Square
 *               blocks accept rht_n up to their size.
 *   sign_seed : seed of the random sign diagonal S_n ([UFP4] Method, H' = S H).
 *               Both operands of a GEMM must use the same sign_seed and rht_n.
 *   sr_seed, sr_stream : key and stream of the stochastic-rounding draws;
 *               stream 0xFFFFFFFF is reserved.
 *   tensor_scale : 0 for single-level scaling, or (power-of-two scales only)
 *               a per-tensor fp32 factor s_T > 0, finite and normal, over
 *               the block scales -- two-level scaling ([UFP4] Method: the
 *               scaling hierarchy is orthogonal to the format).  The rotated
 *               values are multiplied by m_T = RN_fp32(1 / s_T) before the
 *               block exponents are chosen, and an element then stands for
 *               level * 2^e * s_T (dequantization and the GEMMs apply s_T;
 *               the E8M0 bytes are stored as without it).  Anything else is
 *               UFP4_ERR_INVALID_ARG, a nonzero s_T with fp32 scales
 *               UFP4_ERR_UNSUPPORTED. */
typedef struct ufp4_quant_cfg {
  int32_t grid;
  int32_t rounding;
  int32_t scale_mode;
  int32_t block_rows;
  int32_t block_cols;
  int32_t rht_n;
  uint64_t sign_seed;
  uint64_t sr_seed;
  uint32_t sr_stream;
  float tensor_scale;
} ufp4_quant_cfg;

/* A quantized logical operand (device codes and scales, layout above). */
typedef struct ufp4_qtensor {
  const uint8_t* codes;
  const void* scales;
  int64_t P;
  int64_t K;
  ufp4_quant_cfg cfg;
} ufp4_qtensor;

/* Fused RHT + blockwise 4-bit (or MXFP8) quantization of a bf16 matrix.
 * [UFP4] formats section (block absmax scale, RTNE / SR onto G) and Method
 * (X H'_n with H'_n = S_n H_n along the shared GEMM dimension).
 *   x        : bf16 [rows][ld] row-major, ld >= cols.
 *   along    : 0 -> A = x (P = rows, K = cols), row-wise;
 *              1 -> A = x^T (P = cols, K = rows), column-wise: the output is
 *                   the transposed operand, written K-contiguous.
 *   codes    : uint8 [P][K/2] ([P][K] for E4M3);  scales : see the layout above.
 *   rotated  : optional fp32 [P][K] copy of the rotated values y = RN(c_n *
 *              FWHT(S x)) (NULL to skip; not part of the fast path).
 * The rotation is block-diagonal along K in chunks of rht_n; each chunk and
 * block lies inside the operand (K % rht_n == 0, K % block_cols == 0,
 * P % block_rows == 0, else UFP4_ERR_SHAPE).  Stochastic-rounding draw of
 * element (p, k) is keyed by its index p*K + k.  rows == 0 or cols == 0 is a
 * no-op. */
int ufp4_rht_quant(const void* x, int64_t rows, int64_t cols, int64_t ld, int32_t along,
                   const ufp4_quant_cfg* cfg, uint8_t* codes, void* scales, float* rotated,
                   void* stream);

/* Both quantizations of one tensor X [rows][ld] from a single read: the
 * row-wise one (A = X, K = cols; as ufp4_rht_quant with along = 0 and
 * cfg_row) and the column-wise one (A = X^T, K = rows; as ufp4_rht_quant with
 * along = 1 and cfg_col, or as ufp4_rht_quant_segmented when row_offsets is
 * given).  [UFP4] Method: the recipe quantizes X, W and dY along both axes,
 * since each takes part in two GEMMs with different shared dimensions.
 * Outputs are bit-identical to the single-axis calls.  cfg_row and cfg_col
 * must be 1D and agree in grid, rounding, scale mode, block_cols and rht_n;
 * they may differ in sign_seed, sr_seed and sr_stream (else
 * UFP4_ERR_UNSUPPORTED).  rows (or every segment) and cols must be multiples
 * of lcm(rht_n, block_cols) (UFP4_ERR_SHAPE).  row_offsets: HOST int64
 * [num_segments+1] or NULL; 1 <= num_segments <= 128.  Buffers: codes_row
 * [rows][cols/2], scales_row [rows][cols/block_cols], codes_col /
 * scales_col as the column-wise call; device pointers, codes 16-byte and
 * scales 4-byte aligned, x 16-byte aligned with ld % 8 == 0. */
int ufp4_rht_quant_dual(const void* x, int64_t rows, int64_t cols, int64_t ld,
                        const int64_t* row_offsets, int32_t num_segments,
                        const ufp4_quant_cfg* cfg_row, const ufp4_quant_cfg* cfg_col,
                        uint8_t* codes_row, void* scales_row, uint8_t* codes_col,
                        void* scales_col, void* stream);

/* Size in bytes of the device workspace ufp4_quant_diag takes (the partial
 * sums of its workgroups). */
#define UFP4_DIAG_WORKSPACE_BYTES 8192

/* Level statistics of a row-wise quantization (diagnostics): the same
 * transform, scale and rounding as ufp4_rht_quant with along = 0 and cfg, but
 * nothing is stored except, for each magnitude level index k = 0..7 of the
 * codebook, stats[k] = the number of elements rounded to level k and
 * stats[8 + k] = the sum over those elements of rint((L_k - |t|) * 2^28) as a
 * two's-complement int64, t the clamped normalized value the rounding acts on
 * and L_k the level's magnitude in grid units.  stats[8+k] / stats[k] * 2^-28
 * is then the per-level mean rounding error E[rho(t) - t] that [UFP4]'s
 * bin-asymmetry equation (Method, Shrinkage Bias) predicts -- zero for the
 * uniform grids, negative at E2M1's spacing changes under RTNE -- and the
 * counts are the bucket utilisation the Method section attributes to the RHT.
 * The sums are exact integers, so the result does not depend on launch order.
 * stats: DEVICE uint64 [16], 8-byte aligned, overwritten.  workspace:
 * DEVICE buffer of UFP4_DIAG_WORKSPACE_BYTES, 8-byte aligned, owned by the
 * caller; the call clears it and keeps the workgroups' partial sums there,
 * so calls that overlap in time need workspaces of their own (its contents
 * after the call mean nothing).  cfg must be 1D (block_rows == 1) with a
 * 4-bit codebook; shapes and errors as ufp4_rht_quant; a null or misaligned
 * workspace is UFP4_ERR_INVALID_ARG. */
int ufp4_quant_diag(const void* x, int64_t rows, int64_t cols, int64_t ld,
                    const ufp4_quant_cfg* cfg, uint64_t* stats, void* workspace,
                    void* stream);

/* ufp4_quant_diag without the workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, statistics and errors as
 * ufp4_quant_diag; the partial sums live in a scratch array of
 * UFP4_DIAG_WORKSPACE_BYTES that the library holds on each GPU it runs on
 * until the process ends (its address is looked up on the first call on a
 * device).  The scratch does not grow with the input, so no size is refused
 * for it.  The call allocates nothing; each call clears the scratch before
 * use, and calls that overlap on one GPU (different streams or host threads)
 * race on it -- order them on one stream. */
int ufp4_quant_diag_noalloc(const void* x, int64_t rows, int64_t cols, int64_t ld,
                            const ufp4_quant_cfg* cfg, uint64_t* stats, void* stream);

/* Column-wise quantization of row segments (per-expert transposed operands):
 * the quantizer of ufp4_rht_quant ([UFP4] formats section; Method: X H'
 * along the shared dimension) applied to each expert's token range on its
 * own, since in an MoE layer ([UFP4] abstract: the MoE 7.9B and 124B runs)
 * WGRAD contracts over the tokens routed to one expert.
 * Segment g is rows [row_offsets[g], row_offsets[g+1]) of x [rows][ld]; it
 * yields A_g = x[seg]^T of shape [cols][L_g], L_g = segment length, which is
 * stored at codes + cols*row_offsets[g]/2 as [cols][L_g/2] and at scales +
 * cols*row_offsets[g]/block_cols elements as [cols][L_g/block_cols].  Draw
 * indices continue across segments (segment g starts at cols*row_offsets[g]).
 * row_offsets: HOST int64 [num_segments+1], ascending, 0 .. rows, each
 * segment length a multiple of lcm(rht_n, block_cols).  1D blocks only;
 * 1 <= num_segments <= 128 (else UFP4_ERR_INVALID_ARG). */
int ufp4_rht_quant_segmented(const void* x, int64_t rows, int64_t cols, int64_t ld,
                             const int64_t* row_offsets, int32_t num_segments,
                             const ufp4_quant_cfg* cfg, uint8_t* codes, void* scales,
                             void* stream);

/* Dequantization Q_G(T) ([UFP4] formats section: a quantized tensor stands
 * for level * block scale), in the rotated basis: out[p][k] =
 * RN_fp32(level(code) * s_B), written to out [P][ldo] (ldo >= K). */
int ufp4_dequant(const ufp4_qtensor* q, float* out, int64_t ldo, void* stream);

/* Block-scaled 4-bit GEMMs ([UFP4] Method: Y^ = Q(X H') Q(W H')^T, the
 * rotation cancels on the shared dimension; [2DFP4] root cause: dX = dY W,
 * dW = dY^T X).  Each computes C[p][q] = sum_k A[p][k] * B[q][k] over the
 * dequantized codes, accumulating in fp32, and writes fp32 C [P_A][ldc].
 *   fprop: A = X  (M x K_in),  B = W   (N x K_in)    -> Y  [M][N]
 *   dgrad: A = dY (M x N),     B = W^T (K_in x N)    -> dX [M][K_in]
 *   wgrad: A = dY^T (N x M),   B = X^T (K_in x M)    -> dW [N][K_in]
 * Operands must agree on K, grid, scale_mode, rht_n and sign_seed
 * (UFP4_ERR_MISMATCH otherwise).  Block shapes may differ between operands.
 * With fp32 block scales, a launch whose last round of workgroups (one per
 * compute unit) would be at most half full computes those tiles as two K
 * halves added into C, zeroed first by the same call (two addends on zero:
 * the same result whatever the timing).  This and the grouped forms.  C
 * must be ordinary device memory (hipMalloc, torch's CUDA tensors): those
 * additions are the hardware's fp32 atomics. */
int ufp4_gemm_fprop(const ufp4_qtensor* X, const ufp4_qtensor* W, float* Y, int64_t ldy,
                    void* stream);
int ufp4_gemm_dgrad(const ufp4_qtensor* dY, const ufp4_qtensor* Wt, float* dX, int64_t ldx,
                    void* stream);
int ufp4_gemm_wgrad(const ufp4_qtensor* dYt, const ufp4_qtensor* Xt, float* dW, int64_t ldw,
                    void* stream);

/* Grouped (MoE expert) GEMMs in one launch: one FPROP / DGRAD / WGRAD of
 * [UFP4] Method (Y^ = Q(X H') Q(W H')^T per expert) for each expert of an
 * MoE layer ([UFP4] abstract: MoE 7.9B and 124B pretraining).
 * offsets: HOST int64 [G+1], the padded token offsets of the experts in
 * the expert-sorted token matrix (0 = offsets[0] <= ... <= offsets[G] = T);
 * G <= 64.
 *   fprop_grouped: A = X_perm [T][K_in], B = W stacked [G*N][K_in]
 *                  (expert g = rows g*N ..), Y [T][ldy]: Y_g = X_g W_g^T.
 *   dgrad_grouped: A = dY_perm [T][N], B = W^T stacked [G*K_in][N] (the
 *                  segmented column-wise quantization of W [G*N][K_in] with
 *                  offsets g*N), dX [T][ldx]: dX_g = dY_g W_g.
 *   wgrad_grouped: A = dY^T segments (ufp4_rht_quant_segmented of dY_perm,
 *                  P = N, K = T), B = X^T segments (of X_perm, P = K_in,
 *                  K = T), dW stacked [G*N][ldw]: dW_g = dY_g^T X_g.
 * The per-group B row count is B->P / G. */
int ufp4_gemm_fprop_grouped(const ufp4_qtensor* Xp, const ufp4_qtensor* W, int32_t G,
                            const int64_t* offsets, float* Y, int64_t ldy, void* stream);
int ufp4_gemm_dgrad_grouped(const ufp4_qtensor* dYp, const ufp4_qtensor* Wt, int32_t G,
                            const int64_t* offsets, float* dX, int64_t ldx, void* stream);
int ufp4_gemm_wgrad_grouped(const ufp4_qtensor* dYt, const ufp4_qtensor* Xt, int32_t G,
                            const int64_t* offsets, float* dW, int64_t ldw, void* stream);

/* The three GEMMs above with a caller workspace.  op: UFP4_GEMM_FPROP,
 * UFP4_GEMM_DGRAD or UFP4_GEMM_WGRAD; G = 0 for the dense call (offsets may
 * be NULL), G >= 1 for the grouped one (same arguments and rules as above).
 * Same operation, result contract and errors as the call without a
 * workspace.  The uniform grids (E1M2, INT4) with power-of-two scales on
 * 32-element K blocks (1 x 32 or 32 x 32) are contracted on the scaled
 * matrix cores as FP6 E2M3 operands -- every E1M2 level k/4 and every INT4
 * level n in -7..7 is an E2M3 value ([UFP4] chatpaper abstract: uniform grids as
 * first-class hardware primitives; [UFP4] Method: the GEMM contracts the
 * quantized operands): both operands are first expanded from their codes
 * into `workspace` (device memory, 256-byte aligned, at least
 * ufp4_gemm_workspace_bytes(op, A, B, G) bytes; its contents on entry do not
 * matter and are overwritten).  A smaller or misaligned workspace for such
 * a call is UFP4_ERR_INVALID_ARG; workspace = NULL (workspace_bytes 0) or
 * any other operand kind runs the call without it.  Calls that share a
 * workspace must be ordered on one stream. */
#define UFP4_GEMM_FPROP 0
#define UFP4_GEMM_DGRAD 1
#define UFP4_GEMM_WGRAD 2
size_t ufp4_gemm_workspace_bytes(int32_t op, const ufp4_qtensor* A, const ufp4_qtensor* B,
                                 int32_t G);
int ufp4_gemm_ws(int32_t op, const ufp4_qtensor* A, const ufp4_qtensor* B, int32_t G,
                 const int64_t* offsets, float* C, int64_t ldc, void* workspace,
                 size_t workspace_bytes, void* stream);

/* Transpose of a quantized operand whose blocks are square (2D mode): the
 * codes of A^T are the transposed codes and, because S(B) = S(B^T) for
 * square blocks ([2DFP4] 2D section), its scale grid is the transposed grid.
 * dst_codes [K][P/2], dst_scales [K/b][P/b].  P and K must be multiples of
 * the block size and of 2; rht_n must be 1. */
int ufp4_transpose_qtensor(const ufp4_qtensor* src, uint8_t* dst_codes, void* dst_scales,
                           void* stream);

/* Size helpers (bytes) for caller allocation. */
size_t ufp4_codes_bytes(int64_t P, int64_t K);
size_t ufp4_scales_bytes(int64_t P, int64_t K, const ufp4_quant_cfg* cfg);

/* The 16-bit stochastic-rounding draws for elements first .. first+n-1 under
 * (seed, stream), written to out [n] (device uint16).  Exposes the device
 * generator so it can be checked on its own: stochastic rounding ([UFP4]
 * formats section; [2DFP4] 2D section, E[roundS(x)] = x) rounds up when the
 * element's draw falls below its fractional position between two levels. */
int ufp4_philox_fill(uint64_t seed, uint32_t stream_id, uint64_t first, int64_t n,
                     uint16_t* out, void* stream);

/* Device-to-device copy of nbytes bytes from src to dst, written as a
 * streaming kernel (one 16-byte vector per thread over a grid that covers
 * the buffer, non-temporal loads and stores; bytes past the last whole vector
 * copied one by one).  A
 * measurement aid: the HBM bandwidth a pass that reads and writes every byte
 * once reaches, the yardstick for the quantizers, which read their input once
 * and write their outputs once (the pages put the cost of fusing the
 * rotation into the quantizer at a modest overhead, [UFP4] experiments
 * section).  src and dst are
 * device pointers, 16-byte aligned, whose ranges do not overlap; the caller
 * owns both.  nbytes = 0 does nothing.  Errors (no launch):
 * UFP4_ERR_INVALID_ARG for nbytes < 0, a null pointer with nbytes > 0,
 * misalignment or overlapping ranges.  Asynchronous on `stream`. */
int ufp4_stream_copy(const void* src, void* dst, int64_t nbytes, void* stream);

/* Name of a status code (static string). */
const char* ufp4_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* UFP4_H */
