// Allocation-free form of the forward expert grouped GEMM.
//
// bsq_grouped_gemm_fwd needs a small device workspace: the tile planner's
// per-expert tile prefix and expert order, the per-XCD tile-claim counters,
// the tile total and the error word.  Callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid allocation) use bsq_grouped_gemm_fwd_noalloc instead, which keeps
// that workspace in a file-scope device array, one copy per GPU, sized for
// the largest expert count the GEMM accepts.
//
// Every call on a GPU shares that GPU's array.  The planner kernel, enqueued
// first on the call's stream, rewrites every word the GEMM kernel reads
// (claim counters included), so nothing has to start at zero and nothing is
// cleared here; but calls that overlap on one GPU (different streams, or host
// threads) race on the array and must be serialized by the caller.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "../../include/bsq.h"
#include "gemm_common.h"

namespace {

// Same layout and size as the caller-provided workspace of
// bsq_grouped_gemm_fwd for bsq::MAX_EXPERTS experts: the plan's int32 words
// rounded up to 256 bytes, plus 256 bytes.
constexpr int64_t kNoAllocMaxExperts = bsq::MAX_EXPERTS;
constexpr int64_t kPlanWords = bsq::PLAN_HDR + 2 * kNoAllocMaxExperts + 1;
constexpr size_t kScratchBytes = (size_t)((kPlanWords * 4 + 255) / 256 * 256 + 256);

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// Device address of `scratch` on each GPU, looked up once per device with
// that device current (host code never passes the array's name to a kernel:
// on the host it is only a stand-in for the device symbol).
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];

bsq_status scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return BSQ_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return BSQ_ERR_UNSUPPORTED;
    void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return BSQ_ERR_HIP;
        g_scratch_addr[dev].store(p, std::memory_order_release);  // racing threads store the same address
    }
    *out = p;
    return BSQ_OK;
}

}  // namespace

extern "C" bsq_status bsq_grouped_gemm_fwd_noalloc(const uint8_t* a_codes, const uint8_t* a_bscale,
                                                   const float* a_rscale, const uint8_t* w_codes,
                                                   const uint8_t* w_bscale, const float* w_rscale,
                                                   const int32_t* offsets, int32_t num_experts, int64_t m_total,
                                                   int64_t n, int64_t k, void* y, bsq_dtype y_dtype,
                                                   hipStream_t stream) {
    if (num_experts < 1) return BSQ_ERR_INVALID_ARG;
    if (num_experts > kNoAllocMaxExperts) return BSQ_ERR_UNSUPPORTED;  // beyond what `scratch` holds
    if (bsq_workspace_size(BSQ_OP_GEMM_FWD, num_experts, m_total, n, k) > kScratchBytes) return BSQ_ERR_UNSUPPORTED;
    void* ws = nullptr;
    const bsq_status st = scratch_address(&ws);
    if (st != BSQ_OK) return st;
    return bsq_grouped_gemm_fwd(a_codes, a_bscale, a_rscale, w_codes, w_bscale, w_rscale, offsets, num_experts,
                                m_total, n, k, y, y_dtype, ws, kScratchBytes, stream);
}
