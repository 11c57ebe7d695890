// C ABI of libbsq.so: argument validation and kernel launches.  Every entry
// point checks what the host can know (pointers, sizes, multiples, alignment,
// workspace size) before enqueueing anything, never allocates and never
// synchronizes (bsq_debug_status excepted, by contract).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "../../include/bsq.h"
#include "gemm_common.h"

namespace bsq {
hipError_t launch_quantize_nvfp4v(const uint16_t*, int64_t, int, int64_t, uint8_t*, uint8_t*, float*, hipStream_t);
hipError_t launch_swiglu_quantize_nvfp4v(const uint16_t*, int64_t, int, int64_t, uint16_t*, int64_t, uint8_t*, uint8_t*,
                                         float*, hipStream_t);
hipError_t launch_quantize_mxfp8_gather(const uint16_t*, int64_t, int, int64_t, const int32_t*, int64_t, uint8_t*,
                                        uint8_t*, hipStream_t);
hipError_t launch_quantize_nvfp4v_fastdiv(const uint16_t*, int64_t, int, int64_t, uint8_t*, uint8_t*, float*,
                                          hipStream_t);
hipError_t launch_quantize_mxfp8_rowwise(const uint16_t*, int64_t, int, int64_t, uint8_t*, uint8_t*, hipStream_t);
hipError_t launch_quantize_mxfp8_colwise_t(const uint16_t*, int64_t, int, int64_t, const int32_t*, int, int64_t,
                                           uint8_t*, uint8_t*, hipStream_t);
hipError_t launch_quantize_mxfp8_dual(const uint16_t*, int64_t, int, int64_t, const int32_t*, int, int64_t, uint8_t*,
                                      uint8_t*, uint8_t*, uint8_t*, hipStream_t);
hipError_t launch_debug_encode(int, const float*, uint8_t*, int64_t, hipStream_t);
}  // namespace bsq

namespace {

constexpr int64_t kMaxBufferOffset = (int64_t)1 << 31;  // 32-bit buffer offsets
// A dispatch counts its work-items in 32 bits (workgroups x 256 threads <
// 2^32).  Row quantizers run one wave per row, four rows per workgroup of 256
// threads; the debug encoders one element per thread.
constexpr int64_t kMaxNvfp4vRows = ((int64_t)1 << 26) - 4;
constexpr int64_t kMaxDebugElems = ((int64_t)1 << 32) - 256;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Persistent-grid size: one workgroup per compute unit, a multiple of the 8
// XCDs.  The CU count is read once per device.
int persistent_grid() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        v = ((cus + 7) / 8) * 8;
        cache[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

bsq_status from_hip(hipError_t e) { return e == hipSuccess ? BSQ_OK : BSQ_ERR_HIP; }

size_t plan_bytes(int E) { return (size_t)((bsq::plan_words(E) * 4 + 255) / 256 * 256); }

}  // namespace

extern "C" {

int bsq_abi_version(void) { return BSQ_ABI_VERSION; }

const char* bsq_status_string(bsq_status s) {
    switch (s) {
        case BSQ_OK: return "ok";
        case BSQ_ERR_INVALID_ARG: return "invalid argument";
        case BSQ_ERR_UNSUPPORTED: return "unsupported shape or alignment";
        case BSQ_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case BSQ_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

int64_t bsq_colwise_padded_cols(int32_t num_groups, int64_t rows) {
    if (num_groups < 0 || rows < 0) return -1;
    return 128 * ((int64_t)num_groups + (rows + 127) / 128);
}

size_t bsq_workspace_size(int op, int32_t num_experts, int64_t m_total, int64_t n, int64_t k) {
    (void)m_total; (void)n; (void)k;
    if (num_experts < 1 || num_experts > bsq::MAX_EXPERTS) return 0;
    if (op == BSQ_OP_GEMM_FWD) return plan_bytes(num_experts) + 256;
    if (op == BSQ_OP_GEMM_BWD) return 2 * plan_bytes(num_experts) + 256;
    return 0;
}

bsq_status bsq_quantize_nvfp4v(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                               const int32_t* offsets, int32_t num_groups, uint8_t* codes, uint8_t* bscale,
                               float* rscale, hipStream_t stream) {
    (void)offsets;
    if (rows < 0 || cols < 0 || num_groups < 0) return BSQ_ERR_INVALID_ARG;
    if (rows == 0 || cols == 0) return BSQ_OK;
    if (!x_bf16 || !codes || !bscale || !rscale || ld_x < cols) return BSQ_ERR_INVALID_ARG;
    if (cols % 16 || cols > 16384 || ld_x % 8 || !aligned(x_bf16, 16) || !aligned(codes, 8) || !aligned(rscale, 4))
        return BSQ_ERR_UNSUPPORTED;
    if (rows > kMaxNvfp4vRows) return BSQ_ERR_UNSUPPORTED;
    return from_hip(bsq::launch_quantize_nvfp4v(static_cast<const uint16_t*>(x_bf16), rows, (int)cols, ld_x, codes,
                                                bscale, rscale, stream));
}

bsq_status bsq_debug_quantize_nvfp4v_fastdiv(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                                             uint8_t* codes, uint8_t* bscale, float* rscale, hipStream_t stream) {
    if (rows < 0 || cols < 0) return BSQ_ERR_INVALID_ARG;
    if (rows == 0 || cols == 0) return BSQ_OK;
    if (!x_bf16 || !codes || !bscale || !rscale || ld_x < cols) return BSQ_ERR_INVALID_ARG;
    if (cols % 16 || cols > 16384 || ld_x % 8 || !aligned(x_bf16, 16) || !aligned(codes, 8) || !aligned(rscale, 4))
        return BSQ_ERR_UNSUPPORTED;
    if (rows > kMaxNvfp4vRows) return BSQ_ERR_UNSUPPORTED;
    return from_hip(bsq::launch_quantize_nvfp4v_fastdiv(static_cast<const uint16_t*>(x_bf16), rows, (int)cols, ld_x,
                                                        codes, bscale, rscale, stream));
}

bsq_status bsq_quantize_mxfp8_gather(const void* x_bf16, int64_t src_rows, int64_t cols, int64_t ld_x,
                                    const int32_t* row_index, int64_t rows, uint8_t* codes, uint8_t* scale,
                                    hipStream_t stream) {
    if (src_rows < 0 || cols < 0 || rows < 0) return BSQ_ERR_INVALID_ARG;
    if (rows == 0 || cols == 0) return BSQ_OK;
    if (!row_index || !codes || !scale || (src_rows > 0 && !x_bf16) || ld_x < cols) return BSQ_ERR_INVALID_ARG;
    if (cols % 32 || ld_x % 8 || (x_bf16 && !aligned(x_bf16, 16)) || !aligned(codes, 16)) return BSQ_ERR_UNSUPPORTED;
    // source offsets are 32-bit: src_rows * ld_x * 2 bytes must stay below 2^31
    if (src_rows * ld_x * 2 >= kMaxBufferOffset || rows > ((int64_t)1 << 40)) return BSQ_ERR_UNSUPPORTED;
    return from_hip(bsq::launch_quantize_mxfp8_gather(static_cast<const uint16_t*>(x_bf16), src_rows, (int)cols, ld_x,
                                                      row_index, rows, codes, scale, stream));
}

bsq_status bsq_swiglu_quantize_nvfp4v(const void* gu_bf16, int64_t rows, int64_t inter, int64_t ld_gu, void* h_bf16,
                                      int64_t ld_h, uint8_t* codes, uint8_t* bscale, float* rscale,
                                      hipStream_t stream) {
    if (rows < 0 || inter < 0) return BSQ_ERR_INVALID_ARG;
    if (rows == 0 || inter == 0) return BSQ_OK;
    if (!gu_bf16 || !codes || !bscale || !rscale || ld_gu < 2 * inter) return BSQ_ERR_INVALID_ARG;
    if (h_bf16 && ld_h < inter) return BSQ_ERR_INVALID_ARG;
    if (inter % 16 || inter > 16384 || ld_gu % 8 || !aligned(gu_bf16, 16) || !aligned(codes, 8) ||
        !aligned(rscale, 4))
        return BSQ_ERR_UNSUPPORTED;
    if (h_bf16 && (ld_h % 8 || !aligned(h_bf16, 16))) return BSQ_ERR_UNSUPPORTED;
    if (rows > kMaxNvfp4vRows) return BSQ_ERR_UNSUPPORTED;
    return from_hip(bsq::launch_swiglu_quantize_nvfp4v(static_cast<const uint16_t*>(gu_bf16), rows, (int)inter, ld_gu,
                                                       static_cast<uint16_t*>(h_bf16), ld_h, codes, bscale, rscale,
                                                       stream));
}

bsq_status bsq_quantize_mxfp8(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x, bsq_axis axis,
                              const int32_t* offsets, int32_t num_groups, uint8_t* codes, uint8_t* scale,
                              hipStream_t stream) {
    if (rows < 0 || cols < 0 || num_groups < 0) return BSQ_ERR_INVALID_ARG;
    if (axis != BSQ_ROWWISE && axis != BSQ_COLWISE_T) return BSQ_ERR_INVALID_ARG;
    if (axis == BSQ_ROWWISE && (rows == 0 || cols == 0)) return BSQ_OK;  // nothing to write
    if (!codes || !scale) return BSQ_ERR_INVALID_ARG;
    if (axis == BSQ_COLWISE_T && (!offsets || num_groups < 1)) return BSQ_ERR_INVALID_ARG;
    if (cols > ((int64_t)1 << 30)) return BSQ_ERR_UNSUPPORTED;
    if (axis == BSQ_ROWWISE) {
        if (rows == 0 || cols == 0) return BSQ_OK;
        if (!x_bf16 || ld_x < cols) return BSQ_ERR_INVALID_ARG;
        if (cols % 32 || ld_x % 8 || !aligned(x_bf16, 16) || !aligned(codes, 16)) return BSQ_ERR_UNSUPPORTED;
        if (256 * ld_x >= kMaxBufferOffset) return BSQ_ERR_UNSUPPORTED;  // 32-bit offsets within a 128-row tile
        return from_hip(bsq::launch_quantize_mxfp8_rowwise(static_cast<const uint16_t*>(x_bf16), rows, (int)cols,
                                                           ld_x, codes, scale, stream));
    }
    if (cols == 0) return BSQ_OK;
    if (rows > 0 && (!x_bf16 || ld_x < cols)) return BSQ_ERR_INVALID_ARG;
    if (cols % 8 || ld_x % 8 || !aligned(x_bf16, 16) || !aligned(codes, 16)) return BSQ_ERR_UNSUPPORTED;
    if (num_groups > (1 << 30)) return BSQ_ERR_UNSUPPORTED;
    // per-tile load offsets are 32-bit: 128 token rows of ld_x bf16 elements
    if (258 * ld_x >= kMaxBufferOffset) return BSQ_ERR_UNSUPPORTED;
    const int64_t P = bsq_colwise_padded_cols(num_groups, rows);
    return from_hip(bsq::launch_quantize_mxfp8_colwise_t(static_cast<const uint16_t*>(x_bf16), rows, (int)cols, ld_x,
                                                         offsets, num_groups, P, codes, scale, stream));
}

bsq_status bsq_quantize_mxfp8_dual(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                                   const int32_t* offsets, int32_t num_groups, uint8_t* row_codes,
                                   uint8_t* row_scale, uint8_t* t_codes, uint8_t* t_scale, hipStream_t stream) {
    if (rows < 0 || cols < 0 || num_groups < 1 || !offsets) return BSQ_ERR_INVALID_ARG;
    if (rows == 0 || cols == 0) return BSQ_OK;
    if (!x_bf16 || ld_x < cols || !row_codes || !row_scale || !t_codes || !t_scale) return BSQ_ERR_INVALID_ARG;
    if (cols > ((int64_t)1 << 30) || num_groups > (1 << 30)) return BSQ_ERR_UNSUPPORTED;
    if (cols % 32 || ld_x % 8 || !aligned(x_bf16, 16) || !aligned(row_codes, 16) || !aligned(t_codes, 16))
        return BSQ_ERR_UNSUPPORTED;
    if (258 * ld_x >= kMaxBufferOffset) return BSQ_ERR_UNSUPPORTED;
    const int64_t P = bsq_colwise_padded_cols(num_groups, rows);
    return from_hip(bsq::launch_quantize_mxfp8_dual(static_cast<const uint16_t*>(x_bf16), rows, (int)cols, ld_x,
                                                    offsets, num_groups, P, t_codes, t_scale, row_codes, row_scale,
                                                    stream));
}

bsq_status bsq_grouped_gemm_fwd(const uint8_t* a_codes, const uint8_t* a_bscale, const float* a_rscale,
                                const uint8_t* w_codes, const uint8_t* w_bscale, const float* w_rscale,
                                const int32_t* offsets, int32_t num_experts, int64_t m_total, int64_t n, int64_t k,
                                void* y, bsq_dtype y_dtype, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
    if (num_experts < 1 || m_total < 0 || n < 0 || k < 0) return BSQ_ERR_INVALID_ARG;
    if (y_dtype != BSQ_BF16 && y_dtype != BSQ_F32) return BSQ_ERR_INVALID_ARG;
    if (!offsets || !workspace || !w_codes || !w_bscale || !w_rscale) return BSQ_ERR_INVALID_ARG;
    if (m_total > 0 && (!a_codes || !a_bscale || !a_rscale || !y)) return BSQ_ERR_INVALID_ARG;
    if (num_experts > bsq::MAX_EXPERTS) return BSQ_ERR_UNSUPPORTED;
    if (k == 0 || n == 0 || k % 64 || n % 8) return BSQ_ERR_UNSUPPORTED;
    if (!aligned(a_codes, 16) || !aligned(w_codes, 16) || !aligned(a_bscale, 4) || !aligned(w_bscale, 4) ||
        !aligned(workspace, 256))
        return BSQ_ERR_UNSUPPORTED;
    // per-tile buffer offsets are 32-bit: 256 rows of codes/scales
    if (256 * (k / 2) >= kMaxBufferOffset || m_total >= (int64_t)1 << 31) return BSQ_ERR_UNSUPPORTED;
    // per-tile output offsets are 32-bit: 256 rows of n outputs
    if (256 * n * (y_dtype == BSQ_F32 ? 4 : 2) >= kMaxBufferOffset) return BSQ_ERR_UNSUPPORTED;
    if (workspace_bytes < bsq_workspace_size(BSQ_OP_GEMM_FWD, num_experts, m_total, n, k))
        return BSQ_ERR_WORKSPACE_TOO_SMALL;
    return from_hip(bsq::launch_gemm_fwd_nvfp4v(a_codes, a_bscale, a_rscale, w_codes, w_bscale, w_rscale, offsets,
                                                num_experts, m_total, n, k, y, y_dtype == BSQ_F32 ? 1 : 0, 0, n,
                                                static_cast<int32_t*>(workspace), persistent_grid(), stream));
}

bsq_status bsq_grouped_gemm_fwd_swiglu(const uint8_t* a_codes, const uint8_t* a_bscale, const float* a_rscale,
                                       const uint8_t* w_codes, const uint8_t* w_bscale, const float* w_rscale,
                                       const int32_t* offsets, int32_t num_experts, int64_t m_total, int64_t inter,
                                       int64_t k, void* h_bf16, int64_t ld_h, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
    if (num_experts < 1 || m_total < 0 || inter < 0 || k < 0) return BSQ_ERR_INVALID_ARG;
    if (!offsets || !workspace || !w_codes || !w_bscale || !w_rscale) return BSQ_ERR_INVALID_ARG;
    if (m_total > 0 && (!a_codes || !a_bscale || !a_rscale || !h_bf16 || ld_h < inter)) return BSQ_ERR_INVALID_ARG;
    if (num_experts > bsq::MAX_EXPERTS) return BSQ_ERR_UNSUPPORTED;
    // a 256-column output tile holds 128 gate and the matching 128 up columns
    if (k == 0 || inter == 0 || k % 64 || inter % 128) return BSQ_ERR_UNSUPPORTED;
    if (!aligned(a_codes, 16) || !aligned(w_codes, 16) || !aligned(a_bscale, 4) || !aligned(w_bscale, 4) ||
        !aligned(workspace, 256) || (m_total > 0 && (!aligned(h_bf16, 16) || ld_h % 8)))
        return BSQ_ERR_UNSUPPORTED;
    // 32-bit per-tile offsets: 256 rows of codes / scales, 256 rows of H
    if (256 * (k / 2) >= kMaxBufferOffset || m_total >= (int64_t)1 << 31 || 256 * ld_h * 2 >= kMaxBufferOffset)
        return BSQ_ERR_UNSUPPORTED;
    if (workspace_bytes < bsq_workspace_size(BSQ_OP_GEMM_FWD, num_experts, m_total, 2 * inter, k))
        return BSQ_ERR_WORKSPACE_TOO_SMALL;
    return from_hip(bsq::launch_gemm_fwd_nvfp4v(a_codes, a_bscale, a_rscale, w_codes, w_bscale, w_rscale, offsets,
                                                num_experts, m_total, 2 * inter, k, h_bf16, 0, 1, ld_h,
                                                static_cast<int32_t*>(workspace), persistent_grid(), stream));
}

bsq_status bsq_grouped_gemm_bwd(const uint8_t* dy_codes, const uint8_t* dy_scale, const uint8_t* wt_codes,
                                const uint8_t* wt_scale, const uint8_t* dyt_codes, const uint8_t* dyt_scale,
                                const uint8_t* xt_codes, const uint8_t* xt_scale, const int32_t* offsets,
                                int32_t num_experts, int64_t m_total, int64_t n, int64_t k, void* dx,
                                bsq_dtype dx_dtype, void* dw, bsq_dtype dw_dtype, unsigned flags, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
    if (num_experts < 1 || m_total < 0 || n < 0 || k < 0) return BSQ_ERR_INVALID_ARG;
    if (flags == 0 || (flags & ~(BSQ_DGRAD | BSQ_WGRAD))) return BSQ_ERR_INVALID_ARG;
    if (!offsets || !workspace) return BSQ_ERR_INVALID_ARG;
    const bool dg = flags & BSQ_DGRAD, wg = flags & BSQ_WGRAD;
    if (dg && (dx_dtype != BSQ_BF16 && dx_dtype != BSQ_F32)) return BSQ_ERR_INVALID_ARG;
    if (wg && (dw_dtype != BSQ_BF16 && dw_dtype != BSQ_F32)) return BSQ_ERR_INVALID_ARG;
    if (dg && (!wt_codes || !wt_scale || (m_total > 0 && (!dy_codes || !dy_scale || !dx))))
        return BSQ_ERR_INVALID_ARG;
    if (wg && (!dyt_codes || !dyt_scale || !xt_codes || !xt_scale || !dw)) return BSQ_ERR_INVALID_ARG;
    if (num_experts > bsq::MAX_EXPERTS) return BSQ_ERR_UNSUPPORTED;
    if (n == 0 || k == 0 || n % 64 || k % 64) return BSQ_ERR_UNSUPPORTED;
    if (!aligned(workspace, 256)) return BSQ_ERR_UNSUPPORTED;
    if (dg && (!aligned(dy_codes, 16) || !aligned(wt_codes, 16))) return BSQ_ERR_UNSUPPORTED;
    if (wg && (!aligned(dyt_codes, 16) || !aligned(xt_codes, 16))) return BSQ_ERR_UNSUPPORTED;
    const int64_t P = bsq_colwise_padded_cols(num_experts, m_total);
    const int64_t Pw = bsq_colwise_padded_cols(num_experts, (int64_t)num_experts * n);
    // per-tile buffer offsets are 32-bit: 256 rows of codes, and block-major
    // scale runs (block index x rows of the scale matrix)
    if (256 * Pw + Pw >= kMaxBufferOffset || 256 * P + P >= kMaxBufferOffset || 256 * n >= kMaxBufferOffset ||
        m_total >= (int64_t)1 << 31 || (n / 32 + 1) * (m_total + 256) >= kMaxBufferOffset ||
        (P / 32 + 1) * (n + k) >= kMaxBufferOffset || (Pw / 32 + 1) * k >= kMaxBufferOffset)
        return BSQ_ERR_UNSUPPORTED;
    // per-tile output offsets are 32-bit: 256 rows of k outputs (dx and dw)
    if ((dg && 256 * k * (dx_dtype == BSQ_F32 ? 4 : 2) >= kMaxBufferOffset) ||
        (wg && 256 * k * (dw_dtype == BSQ_F32 ? 4 : 2) >= kMaxBufferOffset))
        return BSQ_ERR_UNSUPPORTED;
    if (workspace_bytes < bsq_workspace_size(BSQ_OP_GEMM_BWD, num_experts, m_total, n, k))
        return BSQ_ERR_WORKSPACE_TOO_SMALL;
    int32_t* plan0 = static_cast<int32_t*>(workspace);
    int32_t* plan1 = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + plan_bytes(num_experts));
    const int grid = persistent_grid();
    if (dg && m_total > 0) {
        bsq::BwdArgs a{dy_codes, dy_scale, wt_codes, wt_scale, nullptr, nullptr, nullptr, nullptr,
                       offsets, num_experts, m_total, n, k, P, Pw, dx, dx_dtype == BSQ_F32 ? 1 : 0, 0, plan0, 0, 0};
        const hipError_t e = bsq::launch_gemm_bwd_mxfp8(a, grid, stream);
        if (e != hipSuccess) return BSQ_ERR_HIP;
    }
    if (wg) {
        bsq::BwdArgs a{nullptr, nullptr, nullptr, nullptr, dyt_codes, dyt_scale, xt_codes, xt_scale,
                       offsets, num_experts, m_total, n, k, P, Pw, dw, dw_dtype == BSQ_F32 ? 1 : 0, 1, plan1, 0, 0};
        const hipError_t e = bsq::launch_gemm_bwd_mxfp8(a, grid, stream);
        if (e != hipSuccess) return BSQ_ERR_HIP;
    }
    return BSQ_OK;
}

bsq_status bsq_grouped_gemm_fwd_mxfp8(const uint8_t* x_codes, const uint8_t* x_scale, const uint8_t* w_codes,
                                      const uint8_t* w_scale, const int32_t* offsets, int32_t num_experts,
                                      int64_t m_total, int64_t n, int64_t k, void* y, bsq_dtype y_dtype,
                                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (num_experts < 1 || m_total < 0 || n < 0 || k < 0) return BSQ_ERR_INVALID_ARG;
    if (y_dtype != BSQ_BF16 && y_dtype != BSQ_F32) return BSQ_ERR_INVALID_ARG;
    if (!offsets || !workspace || !w_codes || !w_scale) return BSQ_ERR_INVALID_ARG;
    if (m_total > 0 && (!x_codes || !x_scale || !y)) return BSQ_ERR_INVALID_ARG;
    if (num_experts > bsq::MAX_EXPERTS) return BSQ_ERR_UNSUPPORTED;
    if (n == 0 || k == 0 || n % 64 || k % 64) return BSQ_ERR_UNSUPPORTED;
    if (!aligned(workspace, 256) || !aligned(w_codes, 16) || (m_total > 0 && !aligned(x_codes, 16)))
        return BSQ_ERR_UNSUPPORTED;
    // 32-bit per-tile offsets: 256 rows of codes; block-major scale runs
    const int64_t wrows = (int64_t)num_experts * n;
    if (256 * k >= kMaxBufferOffset || m_total >= (int64_t)1 << 31 ||
        (k / 32 + 1) * (m_total + 256) >= kMaxBufferOffset || (k / 32 + 1) * (wrows + 256) >= kMaxBufferOffset)
        return BSQ_ERR_UNSUPPORTED;
    // per-tile output offsets are 32-bit: 256 rows of n outputs
    if (256 * n * (y_dtype == BSQ_F32 ? 4 : 2) >= kMaxBufferOffset) return BSQ_ERR_UNSUPPORTED;
    if (workspace_bytes < bsq_workspace_size(BSQ_OP_GEMM_FWD, num_experts, m_total, n, k))
        return BSQ_ERR_WORKSPACE_TOO_SMALL;
    if (m_total == 0) return BSQ_OK;
    // the dgrad tile path with a row-major weight stack as B: reduction k,
    // output width n
    bsq::BwdArgs a{x_codes, x_scale, w_codes, w_scale, nullptr, nullptr, nullptr, nullptr,
                   offsets, num_experts, m_total, k, n, 0, 0, y, y_dtype == BSQ_F32 ? 1 : 0, 0,
                   static_cast<int32_t*>(workspace), 1, 0};
    return bsq::launch_gemm_bwd_mxfp8(a, persistent_grid(), stream) == hipSuccess ? BSQ_OK : BSQ_ERR_HIP;
}

bsq_status bsq_grouped_gemm_bf16(const void* x_bf16, const void* w_bf16, const int32_t* offsets,
                                 int32_t num_experts, int64_t m_total, int64_t n, int64_t k, void* y,
                                 bsq_dtype y_dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (num_experts < 1 || m_total < 0 || n < 0 || k < 0) return BSQ_ERR_INVALID_ARG;
    if (y_dtype != BSQ_BF16 && y_dtype != BSQ_F32) return BSQ_ERR_INVALID_ARG;
    if (!offsets || !workspace || !w_bf16) return BSQ_ERR_INVALID_ARG;
    if (m_total > 0 && (!x_bf16 || !y)) return BSQ_ERR_INVALID_ARG;
    if (num_experts > bsq::MAX_EXPERTS) return BSQ_ERR_UNSUPPORTED;
    if (n == 0 || k == 0 || n % 64 || k % 64) return BSQ_ERR_UNSUPPORTED;
    if (!aligned(workspace, 256) || !aligned(w_bf16, 16) || (m_total > 0 && !aligned(x_bf16, 16)))
        return BSQ_ERR_UNSUPPORTED;
    if (256 * 2 * k >= kMaxBufferOffset || m_total >= (int64_t)1 << 31) return BSQ_ERR_UNSUPPORTED;
    // per-tile output offsets are 32-bit: 256 rows of n outputs
    if (256 * n * (y_dtype == BSQ_F32 ? 4 : 2) >= kMaxBufferOffset) return BSQ_ERR_UNSUPPORTED;
    if (workspace_bytes < bsq_workspace_size(BSQ_OP_GEMM_FWD, num_experts, m_total, n, k))
        return BSQ_ERR_WORKSPACE_TOO_SMALL;
    if (m_total == 0) return BSQ_OK;
    bsq::BwdArgs a{static_cast<const uint8_t*>(x_bf16), nullptr, static_cast<const uint8_t*>(w_bf16), nullptr,
                   nullptr, nullptr, nullptr, nullptr, offsets, num_experts, m_total, k, n, 0, 0, y,
                   y_dtype == BSQ_F32 ? 1 : 0, 0, static_cast<int32_t*>(workspace), 1, 1};
    return bsq::launch_gemm_bwd_mxfp8(a, persistent_grid(), stream) == hipSuccess ? BSQ_OK : BSQ_ERR_HIP;
}

bsq_status bsq_grouped_gemm_w4a16(const void* x_bf16, const uint8_t* w_codes, const uint8_t* w_bscale,
                                  const float* w_rscale, const int32_t* offsets, int32_t num_experts,
                                  int64_t m_total, int64_t n, int64_t k, void* y, bsq_dtype y_dtype,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (num_experts < 1 || m_total < 0 || n < 0 || k < 0) return BSQ_ERR_INVALID_ARG;
    if (y_dtype != BSQ_BF16 && y_dtype != BSQ_F32) return BSQ_ERR_INVALID_ARG;
    if (!offsets || !workspace || !w_codes || !w_bscale || !w_rscale) return BSQ_ERR_INVALID_ARG;
    if (m_total > 0 && (!x_bf16 || !y)) return BSQ_ERR_INVALID_ARG;
    if (num_experts > bsq::MAX_EXPERTS) return BSQ_ERR_UNSUPPORTED;
    if (n == 0 || k == 0 || n % 64 || k % 64) return BSQ_ERR_UNSUPPORTED;
    if (!aligned(workspace, 256) || !aligned(w_codes, 16) || !aligned(w_bscale, 4) || !aligned(w_rscale, 4) ||
        (m_total > 0 && !aligned(x_bf16, 16)))
        return BSQ_ERR_UNSUPPORTED;
    if (256 * 2 * k >= kMaxBufferOffset || m_total >= (int64_t)1 << 31) return BSQ_ERR_UNSUPPORTED;
    // per-tile output offsets are 32-bit: 256 rows of n outputs
    if (256 * n * (y_dtype == BSQ_F32 ? 4 : 2) >= kMaxBufferOffset) return BSQ_ERR_UNSUPPORTED;
    if (workspace_bytes < bsq_workspace_size(BSQ_OP_GEMM_FWD, num_experts, m_total, n, k))
        return BSQ_ERR_WORKSPACE_TOO_SMALL;
    if (m_total == 0) return BSQ_OK;
    // dgrad-style tiles: reduction k, output width n, B the packed rows of W_e
    bsq::BwdArgs a{static_cast<const uint8_t*>(x_bf16), nullptr, w_codes, w_bscale, nullptr, nullptr, nullptr,
                   nullptr, offsets, num_experts, m_total, k, n, 0, 0, y, y_dtype == BSQ_F32 ? 1 : 0, 0,
                   static_cast<int32_t*>(workspace), 1, 0, 1, w_rscale};
    return bsq::launch_gemm_bwd_mxfp8(a, persistent_grid(), stream) == hipSuccess ? BSQ_OK : BSQ_ERR_HIP;
}

bsq_status bsq_debug_status(const void* workspace, hipStream_t stream, int32_t* error_word_host) {
    if (!workspace || !error_word_host) return BSQ_ERR_INVALID_ARG;
    if (hipStreamSynchronize(stream) != hipSuccess) return BSQ_ERR_HIP;
    int32_t v = 0;
    if (hipMemcpy(&v, static_cast<const int32_t*>(workspace) + bsq::PLAN_ERR, 4, hipMemcpyDeviceToHost) !=
        hipSuccess)
        return BSQ_ERR_HIP;
    *error_word_host = v;
    return BSQ_OK;
}

bsq_status bsq_debug_encode_e2m1(const float* in, uint8_t* out, int64_t n, hipStream_t stream) {
    if (n < 0) return BSQ_ERR_INVALID_ARG;
    if (n == 0) return BSQ_OK;
    if (!in || !out) return BSQ_ERR_INVALID_ARG;
    if (n > kMaxDebugElems) return BSQ_ERR_UNSUPPORTED;
    return from_hip(bsq::launch_debug_encode(0, in, out, n, stream));
}

bsq_status bsq_debug_encode_e4m3(const float* in, uint8_t* out, int64_t n, hipStream_t stream) {
    if (n < 0) return BSQ_ERR_INVALID_ARG;
    if (n == 0) return BSQ_OK;
    if (!in || !out) return BSQ_ERR_INVALID_ARG;
    if (n > kMaxDebugElems) return BSQ_ERR_UNSUPPORTED;
    return from_hip(bsq::launch_debug_encode(1, in, out, n, stream));
}

}  // extern "C"
