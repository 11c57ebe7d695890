/*
 * bsq.h -- C ABI of libbsq.so: block-scaled MoE expert grouped GEMM on
 * AMD Instinct MI355X (gfx950).
 *
 * What the library computes (the pages describe the method, not an API):
 *   "Composer 2 Technical Report" (papercache.org summary), section 6.1
 *   "Training infrastructure": the MoE forward quantizes BF16 activations and
 *   weights to an NVFP4 variant -- FP4 E2M1 values, one FP8 E4M3 scale per
 *   16-element block and one FP32 scale per token (instead of a per-tensor
 *   FP32 scale), with IEEE-compliant division; the MoE backward runs in
 *   standard MXFP8 -- FP8 E4M3 values with one E8M0 scale per 32 elements; the
 *   expert computation is a grouped GEMM whose efficiency grows with the tokens
 *   per rank.  "Cursor Composer 2 report deep dive" (machinelearningatscale),
 *   section 1 "The kernel section", gives the same recipe and notes the
 *   per-token scale costs latency in the quantize and in the GEMM epilogue.
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless marked (host).  The caller owns all
 *    memory; the library never allocates, frees or synchronizes, and enqueues
 *    its kernels on `stream` only (0 = the null stream).
 *  - bf16 inputs are raw IEEE bfloat16 bit patterns (uint16).  Non-finite
 *    inputs are outside the contract.
 *  - Matrices are row-major; "ld" is the row pitch in elements.
 *  - `offsets` is a device array of num_groups+1 int32 exclusive prefix sums:
 *    offsets[0] = 0, non-decreasing, offsets[num_groups] = rows (m_total).
 *    Group g (an expert) owns rows [offsets[g], offsets[g+1]).  It stays on
 *    the device; it is read by the kernels, never by the host.  Its validity
 *    is a precondition: a violation found on the device makes the GEMMs skip
 *    all work and is reported by bsq_debug_status().
 *  - Argument errors are detected on the host before anything is enqueued
 *    and returned as a status; a launch failure returns BSQ_ERR_HIP.
 *  - Calls are reentrant; kernels of calls on different streams may overlap
 *    as long as their output and workspace buffers do not.
 *
 * Data layouts (bytes are compared bit-exactly against the CPU oracle):
 *  NVFP4-variant (NVFP4v), rows x cols, cols % 16 == 0:
 *    codes  [rows][cols/2] u8: element 2j in the LOW nibble of byte j; nibble =
 *           sign (bit 3) | E2M1 magnitude code (bits 0-2, values
 *           0,.5,1,1.5,2,3,4,6).
 *    bscale [rows][cols/16] u8: E4M3 (OCP E4M3FN) block scale S_b.
 *    rscale [rows] f32: per-row (per-token) decode scale s_row = A / 2688.
 *    Decoded element: e2m1(code) * S_b * s_row.
 *  MXFP8 scales are stored BLOCK-MAJOR: for a matrix of R rows whose blocks
 *    of 32 run along its rows, the E8M0 byte (2^(byte-127)) of row r, block b
 *    is at scale[b * R + r].  (The GEMMs fetch the scales of 256 consecutive
 *    rows of one block as one contiguous run.)
 *  MXFP8 ROWWISE, rows x cols, cols % 32 == 0:
 *    codes [rows][cols] u8 E4M3; scale [cols/32][rows].
 *  MXFP8 COLWISE_T of an input [rows][cols] with groups `offsets`:
 *    blocks of 32 run DOWN the rows of each group and restart at each group;
 *    the output is transposed: codes [cols][P], scale [P/32][cols] with
 *    P = bsq_colwise_padded_cols(num_groups, rows) = 128*(num_groups +
 *    ceil(rows/128)).  Group g starts at column c0(g) = 128*(g +
 *    offsets[g]/128) (integer division), so every group's code rows begin on
 *    a 128-byte line (one L2 request per line for the GEMMs), and spans
 *    32*ceil(M_g/32) columns; every byte not holding a real element (tails,
 *    gaps, the end) is 0.
 */
#ifndef BSQ_H_
#define BSQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

/* 3: COLWISE_T segments start on 128-column boundaries (P changed);
 * added bsq_quantize_mxfp8_dual and bsq_grouped_gemm_w4a16.
 * 4: added bsq_grouped_gemm_fwd_noalloc.
 * 5: added bsq_grouped_gemm_fwd_swiglu; the SwiGLU activation's reciprocal
 *    (1 + e^-|g|)^-1 comes from the hardware reciprocal. */
#define BSQ_ABI_VERSION 5

typedef enum {
    BSQ_OK = 0,
    BSQ_ERR_INVALID_ARG = 1,         /* null pointer, negative size, bad enum     */
    BSQ_ERR_UNSUPPORTED = 2,         /* valid but unsupported shape or alignment  */
    BSQ_ERR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes < bsq_workspace_size(...) */
    BSQ_ERR_HIP = 4                  /* a HIP runtime call or launch failed       */
} bsq_status;

typedef enum { BSQ_BF16 = 0, BSQ_F32 = 1 } bsq_dtype;

typedef enum {
    BSQ_ROWWISE = 0,   /* blocks of 32 along each row (the contiguous dim)      */
    BSQ_COLWISE_T = 1  /* blocks of 32 down each group's rows, output transposed */
} bsq_axis;

/* Flags of bsq_grouped_gemm_bwd. */
#define BSQ_DGRAD 1u
#define BSQ_WGRAD 2u

/* Operation ids of bsq_workspace_size. */
#define BSQ_OP_GEMM_FWD 0
#define BSQ_OP_GEMM_BWD 1

/*
 * bsq_quantize_nvfp4v -- NVFP4-variant quantization of each row of a bf16
 * matrix ("Composer 2 Technical Report", section 6.1, NVFP4 variant in the
 * MoE forward; per-token instead of per-tensor scale).  Per row: A = max|x|;
 * A == 0 gives all-zero outputs; else s_row = RN32(A/2688); per 16-block b with
 * a_b = max|x|: S_b = E4M3_RNE(RN32(448*a_b/A)); d_b = RN32(S_b*s_row); codes
 * sign(x) | E2M1_RNE_sat(RN32(x/d_b)) (IEEE division), all-zero when d_b == 0.
 * Row-local: a row's bytes never depend on other rows (batch invariant).
 *   x_bf16 [rows][ld_x] bf16, 16-byte aligned, ld_x % 8 == 0, ld_x >= cols.
 *   cols % 16 == 0 (cols == 0 or rows == 0: nothing to do).
 *   offsets/num_groups: accepted for a uniform interface; the operation is
 *   row-local so they change no output byte (may be NULL / 0).
 *   codes [rows][cols/2], bscale [rows][cols/16], rscale [rows]: outputs.
 * Errors: INVALID_ARG (null pointer with rows*cols > 0, negative sizes),
 *   UNSUPPORTED (cols % 16, alignment), HIP.
 */
bsq_status bsq_quantize_nvfp4v(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                               const int32_t* offsets, int32_t num_groups,
                               uint8_t* codes, uint8_t* bscale, float* rscale, hipStream_t stream);

/*
 * bsq_quantize_mxfp8_gather -- MXFP8 ROWWISE quantization fused with the
 * token permutation of an expert dispatch: output row i is the quantization
 * of source row row_index[i] ("Composer 2 Technical Report", section 6.1,
 * and "Cursor Composer 2 report deep dive", section 2: tokens are quantized
 * to MXFP8 before the expert-parallel dispatch, since the experts compute in
 * MXFP8 anyway; this is the one-GPU half, the permute into expert-sorted
 * order, with top-k duplicates as repeated indices).
 *   x_bf16 [src_rows][ld_x] bf16, 16-byte aligned, ld_x % 8 == 0,
 *   ld_x >= cols, src_rows * ld_x * 2 < 2^31; cols % 32 == 0.
 *   row_index [rows] int32 (device): an index outside [0, src_rows) gives an
 *   all-zero output row (codes 0, scale bytes 0).
 *   codes [rows][cols] (16-byte aligned), scale [cols/32][rows] block-major:
 *   the bytes bsq_quantize_mxfp8(BSQ_ROWWISE) gives for the gathered rows.
 * Errors: INVALID_ARG, UNSUPPORTED (cols multiple, alignment, source size),
 *   HIP.
 */
bsq_status bsq_quantize_mxfp8_gather(const void* x_bf16, int64_t src_rows, int64_t cols, int64_t ld_x,
                                    const int32_t* row_index, int64_t rows, uint8_t* codes, uint8_t* scale,
                                    hipStream_t stream);

/*
 * bsq_swiglu_quantize_nvfp4v -- the activation between the two forward
 * expert GEMMs fused with the NVFP4-variant quantization of its output, so
 * the down projection's input is quantized without another pass over H
 * ("Composer 2 Technical Report", section 6.1: NVFP4 variant on the MoE
 * forward activations; the per-token absmax is fused into the quantizer as
 * in "Cursor Composer 2 report deep dive", section 1).  The activation itself
 * is not on the pages; this library takes SwiGLU: for each row of
 * [gate | up] (2 * inter bf16), H[c] = bf16_RNE(silu(g) * u), g = row[c],
 * u = row[inter + c], with silu evaluated in binary32 from t = e^-|g|:
 * g / (1 + t) for g >= 0, (g * t) / (1 + t) for g < 0 (IEEE division, expf).  H is then quantized exactly as
 * bsq_quantize_nvfp4v quantizes a bf16 row (same bytes).
 *   gu_bf16 [rows][ld_gu] bf16, 16-byte aligned, ld_gu % 8 == 0,
 *   ld_gu >= 2 * inter; inter % 16 == 0, inter <= 16384.
 *   h_bf16 [rows][ld_h] (optional, may be NULL): receives H; 16-byte aligned,
 *   ld_h % 8 == 0, ld_h >= inter.
 *   codes [rows][inter/2], bscale [rows][inter/16], rscale [rows]: outputs.
 * Row-local, batch invariant.  rows == 0 or inter == 0: nothing to do.
 * Errors: INVALID_ARG (null pointers, negative sizes, short leading
 *   dimensions), UNSUPPORTED (inter multiple or size, alignment), HIP.
 */
bsq_status bsq_swiglu_quantize_nvfp4v(const void* gu_bf16, int64_t rows, int64_t inter, int64_t ld_gu,
                                      void* h_bf16, int64_t ld_h,
                                      uint8_t* codes, uint8_t* bscale, float* rscale, hipStream_t stream);

/*
 * bsq_debug_quantize_nvfp4v_fastdiv -- ABLATION, not the method: the NVFP4
 * variant quantizer of bsq_quantize_nvfp4v with every division (A/2688,
 * 448*a_b/A and x/d_b) replaced by a fast approximate divide, numerator times
 * the hardware reciprocal approximation (v_rcp_f32).  "Composer 2 Technical
 * Report", section 6.1, reports that such a fast divide in NVFP4 quantization
 * made RL training diverge after about a hundred steps and that IEEE
 * division is required; this entry point exists to count how many codes,
 * block scales and row scales the approximation changes.  Same arguments,
 * layouts and errors as bsq_quantize_nvfp4v (no offsets).
 */
bsq_status bsq_debug_quantize_nvfp4v_fastdiv(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                                             uint8_t* codes, uint8_t* bscale, float* rscale, hipStream_t stream);

/*
 * bsq_quantize_mxfp8 -- MXFP8 quantization ("Composer 2 Technical Report",
 * section 6.1, MXFP8 in the MoE backward: E4M3 values, E8M0 scale per 32).
 * Per block of 32: A = max|x|; A == 0 gives scale byte 0 and codes 0; else
 * sh = clamp(floor(log2 A) - 8, -127, 127), scale byte sh+127, codes
 * sign(x) | E4M3_RNE_sat(x * 2^-sh) (exact power-of-two scaling).
 *   x_bf16 [rows][ld_x] bf16, 16-byte aligned, ld_x % 8 == 0, ld_x >= cols.
 *   BSQ_ROWWISE: cols % 32 == 0; codes [rows][cols], scale [cols/32][rows];
 *     offsets may be NULL.
 *   BSQ_COLWISE_T: cols % 8 == 0; offsets required (num_groups >= 1),
 *     device int32 [num_groups + 1] with 0 = offsets[0] <= ... <=
 *     offsets[num_groups] = rows; offsets breaking this give unspecified
 *     bytes but no access outside the buffers (segments are clamped to the
 *     rows).  codes [cols][P], scale [P/32][cols], P = bsq_colwise_padded_cols(
 *     num_groups, rows); every output byte is written (padding = 0).
 *     Quantizing expert weights W [E][N][K] as rows = E*N with offsets
 *     {0, N, 2N, ...} gives the dgrad operand Wt: codes [K][P_w].
 * Errors: INVALID_ARG, UNSUPPORTED (cols multiple, alignment), HIP.
 */
bsq_status bsq_quantize_mxfp8(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                              bsq_axis axis, const int32_t* offsets, int32_t num_groups,
                              uint8_t* codes, uint8_t* scale, hipStream_t stream);

/*
 * bsq_quantize_mxfp8_dual -- both MXFP8 layouts of one bf16 tensor from a
 * single read ("Composer 2 Technical Report", section 6.1, MXFP8 in the MoE
 * backward: an activation gradient feeds dgrad along its rows and wgrad
 * along each expert's token dimension, so it is needed blocked both ways).
 * Writes exactly the bytes of bsq_quantize_mxfp8(BSQ_ROWWISE) into
 * row_codes/row_scale and of bsq_quantize_mxfp8(BSQ_COLWISE_T, offsets)
 * into t_codes/t_scale.
 *   x_bf16 [rows][ld_x] bf16, 16-byte aligned, ld_x % 8 == 0, ld_x >= cols,
 *   258 * ld_x * 2 < 2^31; cols % 32 == 0.
 *   offsets [num_groups + 1] int32 (device), num_groups >= 1, as for
 *   BSQ_COLWISE_T; every row must lie in some group (offsets[0] == 0,
 *   offsets[num_groups] == rows) or its ROWWISE bytes are not written.
 *   row_codes [rows][cols] (16-byte aligned), row_scale [cols/32][rows];
 *   t_codes [cols][P] (16-byte aligned), t_scale [P/32][cols],
 *   P = bsq_colwise_padded_cols(num_groups, rows).
 * rows == 0 or cols == 0: nothing to do.
 * Errors: INVALID_ARG (null pointers, negative sizes, short ld_x),
 *   UNSUPPORTED (cols multiple, alignment, sizes), HIP.
 */
bsq_status bsq_quantize_mxfp8_dual(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                                  const int32_t* offsets, int32_t num_groups,
                                  uint8_t* row_codes, uint8_t* row_scale,
                                  uint8_t* t_codes, uint8_t* t_scale, hipStream_t stream);

/*
 * bsq_grouped_gemm_fwd -- forward expert grouped GEMM over NVFP4v operands
 * ("Composer 2 Technical Report", section 6.1: grouped GEMM of the MoE
 * layer; per-token scale applied in the GEMM epilogue):
 *   y[m][n] = s_a[m] * s_w[e*n_ + n] * sum_k (q_a S_a)[m][k] * (q_w S_w)[e*n_ + n][k]
 * for every row m of expert e's segment.  The E2M1 x E4M3 products are
 * dequantized exactly and accumulated in fp32; each output element is
 * produced by one workgroup in a fixed k order (deterministic, no split-K).
 *   a_*: NVFP4v of the expert-sorted activations, [m_total][k].
 *   w_*: NVFP4v of the weights [num_experts][n][k] (rows e*n + j).
 *   y [m_total][n] in y_dtype (bf16 round-to-nearest-even, or f32).
 *   k % 64 == 0, n % 8 == 0, num_experts >= 1.
 *   workspace >= bsq_workspace_size(BSQ_OP_GEMM_FWD, ...) bytes, 256-byte
 *   aligned; its contents are scratch (no state kept between calls).
 * Errors: INVALID_ARG, UNSUPPORTED (k/n multiples), WORKSPACE_TOO_SMALL, HIP.
 */
bsq_status bsq_grouped_gemm_fwd(const uint8_t* a_codes, const uint8_t* a_bscale, const float* a_rscale,
                                const uint8_t* w_codes, const uint8_t* w_bscale, const float* w_rscale,
                                const int32_t* offsets, int32_t num_experts, int64_t m_total, int64_t n,
                                int64_t k, void* y, bsq_dtype y_dtype, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/*
 * bsq_grouped_gemm_fwd_swiglu -- the gate/up projection of the MoE forward
 * with the activation in the GEMM epilogue ("Cursor Composer 2 report deep
 * dive", section 1: the per-token scale is applied in the GEMM epilogue;
 * "Composer 2 Technical Report", section 6.1).  With gu = the bf16 output
 * bsq_grouped_gemm_fwd would write for these operands ([gate | up] columns,
 * 2*inter of them), it writes only
 *   h[m][j] = bf16_RNE(silu(gu[m][j]) * gu[m][inter + j]),   j < inter,
 * with silu evaluated in binary32 (within one bf16 ulp of the exact value;
 * bit for bit what bsq_swiglu_quantize_nvfp4v writes as h from that gu).  gu
 * itself never reaches memory.  Quantize h with bsq_quantize_nvfp4v for the
 * down projection.
 *   a_*: NVFP4v of the expert-sorted activations [m_total][k].
 *   w_*: NVFP4v of the gate/up weights [num_experts][2*inter][k]: rows
 *   e*2*inter + j are gate row j, rows e*2*inter + inter + j up row j.
 *   h_bf16 [m_total][ld_h] bf16, ld_h >= inter, ld_h % 8 == 0, 16-byte aligned.
 *   inter % 128 == 0, k % 64 == 0, num_experts >= 1.
 *   workspace >= bsq_workspace_size(BSQ_OP_GEMM_FWD, num_experts, m_total,
 *   2*inter, k) bytes, 256-byte aligned.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE_TOO_SMALL, HIP.
 */
bsq_status bsq_grouped_gemm_fwd_swiglu(const uint8_t* a_codes, const uint8_t* a_bscale, const float* a_rscale,
                                       const uint8_t* w_codes, const uint8_t* w_bscale, const float* w_rscale,
                                       const int32_t* offsets, int32_t num_experts, int64_t m_total, int64_t inter,
                                       int64_t k, void* h_bf16, int64_t ld_h, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream);

/*
 * bsq_grouped_gemm_fwd_noalloc -- bsq_grouped_gemm_fwd without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).  Same
 * operands, outputs, results (bit for bit) and errors as bsq_grouped_gemm_fwd;
 * the planner tables and claim counters live in a device array inside the
 * library, one per GPU, sized for num_experts <= 4096 (33,280 bytes, held
 * until the process ends).  Allocates nothing: no hipMalloc, no allocating
 * library call.  Every call on one GPU uses that GPU's single array, so calls
 * that may overlap on one GPU (other streams, other host threads) race and
 * must be serialized by the caller; each call's planner rewrites every word
 * its GEMM reads, so no clearing is needed between calls.
 * Errors: as bsq_grouped_gemm_fwd, plus UNSUPPORTED for num_experts > 4096.
 */
bsq_status bsq_grouped_gemm_fwd_noalloc(const uint8_t* a_codes, const uint8_t* a_bscale, const float* a_rscale,
                                        const uint8_t* w_codes, const uint8_t* w_bscale, const float* w_rscale,
                                        const int32_t* offsets, int32_t num_experts, int64_t m_total, int64_t n,
                                        int64_t k, void* y, bsq_dtype y_dtype, hipStream_t stream);

/*
 * bsq_grouped_gemm_bwd -- backward expert grouped GEMMs in MXFP8
 * ("Composer 2 Technical Report", section 6.1, MXFP8 in the MoE backward; the
 * three GEMMs of training are forward, dgrad and wgrad).  With the forward
 * y = x W_e^T (x [m_total][k], W [E][n][k]) and the incoming gradient dy:
 *   BSQ_DGRAD: dx[m][j] = sum_i dy[m][i] * W_e[i][j]   (reduction over n)
 *     dy_codes/dy_scale: MXFP8 ROWWISE of dy [m_total][n];
 *     wt_codes/wt_scale: MXFP8 COLWISE_T of W viewed as [E*n][k] with offsets
 *     {0, n, 2n, ...}: codes [k][P_w], scale [P_w/32][k],
 *     P_w = bsq_colwise_padded_cols(E, E*n).
 *     dx [m_total][k] in dx_dtype.
 *   BSQ_WGRAD: dW_e[i][j] = sum_{m in segment e} dy[m][i] * x[m][j]
 *     dyt_*: MXFP8 COLWISE_T of dy with `offsets` (codes [n][P], scale [P/32][n]);
 *     xt_*:  MXFP8 COLWISE_T of x with `offsets` (codes [k][P], scale [P/32][k]),
 *     P = bsq_colwise_padded_cols(num_experts, m_total).
 *     dw [num_experts][n][k] in dw_dtype; an empty expert gets zeros.
 * Products are formed by the block-scaled MFMA (E8M0 scales applied inside
 * the matrix core), accumulated in fp32 in a fixed order per element.
 *   n % 64 == 0, k % 64 == 0, num_experts >= 1, flags a non-empty subset of
 *   BSQ_DGRAD | BSQ_WGRAD (operands of an unrequested GEMM may be NULL).
 *   workspace >= bsq_workspace_size(BSQ_OP_GEMM_BWD, ...) bytes.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE_TOO_SMALL, HIP.
 */
bsq_status bsq_grouped_gemm_bwd(const uint8_t* dy_codes, const uint8_t* dy_scale,
                                const uint8_t* wt_codes, const uint8_t* wt_scale,
                                const uint8_t* dyt_codes, const uint8_t* dyt_scale,
                                const uint8_t* xt_codes, const uint8_t* xt_scale,
                                const int32_t* offsets, int32_t num_experts, int64_t m_total, int64_t n,
                                int64_t k, void* dx, bsq_dtype dx_dtype, void* dw, bsq_dtype dw_dtype,
                                unsigned flags, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * bsq_grouped_gemm_fwd_mxfp8 -- forward expert grouped GEMM over MXFP8
 * operands: y[m][j] = sum_k x[m][k] * W_e[j][k] for every row m of expert e's
 * segment, with x and W quantized to MXFP8 along k.  This is the all-MXFP8
 * expert GEMM ("Composer 2 Technical Report", section 3.1: continued
 * pretraining runs in MXFP8; "Scaling and Optimizing Frontier Model
 * Training", MXFP8 expert kernels: MXFP8 grouped GEMMs in forward and
 * backward), next to the NVFP4-variant forward of bsq_grouped_gemm_fwd.
 *   x_codes/x_scale: MXFP8 ROWWISE of x [m_total][k] (scale [k/32][m_total]).
 *   w_codes/w_scale: MXFP8 ROWWISE of W viewed as [num_experts*n][k] (rows
 *   e*n + j; scale [k/32][num_experts*n]).
 *   y [m_total][n] in y_dtype (bf16 round-to-nearest-even, or f32).
 * Products are formed by the block-scaled MFMA and accumulated in fp32 in a
 * fixed order per element (the same kernel and tolerance as BSQ_DGRAD).
 *   n % 64 == 0, k % 64 == 0, num_experts >= 1.
 *   workspace >= bsq_workspace_size(BSQ_OP_GEMM_FWD, ...) bytes, 256-byte
 *   aligned; its contents are scratch.
 * Errors: INVALID_ARG, UNSUPPORTED (multiples, alignment, sizes beyond the
 *   kernel's 32-bit offsets), WORKSPACE_TOO_SMALL, HIP.
 */
bsq_status bsq_grouped_gemm_fwd_mxfp8(const uint8_t* x_codes, const uint8_t* x_scale,
                                      const uint8_t* w_codes, const uint8_t* w_scale,
                                      const int32_t* offsets, int32_t num_experts, int64_t m_total, int64_t n,
                                      int64_t k, void* y, bsq_dtype y_dtype, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream);

/*
 * bsq_grouped_gemm_bf16 -- the bf16 baseline of the forward expert grouped
 * GEMM: y[m][j] = sum_k x[m][k] * W_e[j][k] for every row m of expert e's
 * segment, on plain bf16 operands with the same tiles, DMA pipeline and tile
 * scheduler as the block-scaled kernels ("Scaling and Optimizing Frontier
 * Model Training", MXFP8 expert kernels: the block-scaled grouped GEMMs are
 * measured against BF16 on the 32-expert, 7168/2048 shapes).  bf16 MFMA,
 * fp32 accumulation in a fixed order per element.
 *   x_bf16 [m_total][k], w_bf16 [num_experts*n][k] (rows e*n + j), row-major,
 *   16-byte aligned; y [m_total][n] in y_dtype.
 *   n % 64 == 0, k % 64 == 0, num_experts >= 1; workspace as for
 *   bsq_grouped_gemm_fwd (BSQ_OP_GEMM_FWD).
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE_TOO_SMALL, HIP.
 */
bsq_status bsq_grouped_gemm_bf16(const void* x_bf16, const void* w_bf16, const int32_t* offsets,
                                 int32_t num_experts, int64_t m_total, int64_t n, int64_t k, void* y,
                                 bsq_dtype y_dtype, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * bsq_grouped_gemm_w4a16 -- forward expert grouped GEMM over frozen experts
 * kept in packed form ("Scaling and Optimizing Frontier Model Training",
 * low-precision expert quantization: frozen expert weights stored in a
 * packed low-precision format, about 4x smaller than bf16, and dequantized to
 * bf16 on the fly in the forward).  The pages do not name the packed format;
 * this library takes its NVFP4 variant (4.5 bits per weight, 3.56x smaller
 * than bf16), as written by bsq_quantize_nvfp4v for W viewed as [E*n][k]:
 *   y[m][j] = s_w[e*n + j] * sum_k x[m][k] * (e2m1(q_w) * S_w)[e*n + j][k]
 * for every row m of expert e's segment.  Each E2M1 x E4M3 product is exact
 * in bf16, so the weights reach the bf16 MFMA undistorted; fp32 accumulation
 * in a fixed order per element; the fp32 row scale s_w is applied to the
 * fp32 sum before the output rounding.
 *   x_bf16 [m_total][k] row-major, 16-byte aligned.
 *   w_codes [num_experts*n][k/2] (16-byte aligned), w_bscale
 *   [num_experts*n][k/16] E4M3, w_rscale [num_experts*n] fp32 (4-byte
 *   aligned): the three outputs of bsq_quantize_nvfp4v.
 *   y [m_total][n] in y_dtype.  n % 64 == 0, k % 64 == 0, num_experts >= 1;
 *   workspace as for bsq_grouped_gemm_fwd (BSQ_OP_GEMM_FWD).
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE_TOO_SMALL, HIP.
 */
bsq_status bsq_grouped_gemm_w4a16(const void* x_bf16, const uint8_t* w_codes, const uint8_t* w_bscale,
                                  const float* w_rscale, const int32_t* offsets, int32_t num_experts,
                                  int64_t m_total, int64_t n, int64_t k, void* y, bsq_dtype y_dtype,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace the GEMM entry points need (host function, no GPU use).
 * op is BSQ_OP_GEMM_FWD or BSQ_OP_GEMM_BWD; returns 0 for invalid arguments. */
size_t bsq_workspace_size(int op, int32_t num_experts, int64_t m_total, int64_t n, int64_t k);

/* P of the COLWISE_T layout: 128 * (num_groups + ceil(rows / 128)) (host). */
int64_t bsq_colwise_padded_cols(int32_t num_groups, int64_t rows);

/* Static description of a status code (host). */
const char* bsq_status_string(bsq_status s);

/* BSQ_ABI_VERSION of the built library (host). */
int bsq_abi_version(void);

/*
 * bsq_debug_status -- synchronizes `stream`, then reads the device error word
 * that the GEMM planners write into `workspace` (host-visible result):
 * 0 = the last GEMM call on this workspace saw valid offsets; 1 = offsets[0]
 * != 0, a decreasing pair, or offsets[E] != m_total (that call did no work).
 * Returns BSQ_ERR_HIP on a runtime failure.
 */
bsq_status bsq_debug_status(const void* workspace, hipStream_t stream, int32_t* error_word_host);

/*
 * Element encoders exposed for exhaustive verification of the device
 * conversion paths the quantizers use: out[i] = sign(in[i]) |
 * E2M1_RNE_sat(|in[i]|) (codes 0..15), resp. E4M3_RNE_sat (bytes), for any
 * non-NaN float.  in/out are device arrays of n elements.
 */
bsq_status bsq_debug_encode_e2m1(const float* in, uint8_t* out, int64_t n, hipStream_t stream);
bsq_status bsq_debug_encode_e4m3(const float* in, uint8_t* out, int64_t n, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BSQ_H_ */
