// Device tile planner (see gemm_common.h for the scheduling scheme).
#include "gemm_common.h"

namespace bsq {

// One workgroup of 256 threads.  Tile counts per expert:
//  PLAN_RAGGED_ROWS:      ceil(M_e / bm) * nt   (forward, dgrad: tiles along the
//                         expert's tokens times tiles along the output width)
//  PLAN_RAGGED_REDUCTION: nt * kt               (wgrad: fixed output tiles
//                         per expert, each costing M_e; ordered largest M_e
//                         first so the long tiles start early).
__global__ __launch_bounds__(256) void k_plan(const int32_t* __restrict__ offsets, int E, int64_t m_total,
                                              int mode, int bm, int nt, int kt, int32_t* __restrict__ plan) {
    __shared__ int32_t s_m[MAX_EXPERTS];
    __shared__ int32_t s_order[MAX_EXPERTS];
    __shared__ int32_t s_part[256];
    __shared__ int s_err;
    const int t = threadIdx.x;
    if (t == 0) s_err = (offsets[0] != 0 || (int64_t)offsets[E] != m_total) ? 1 : 0;
    __syncthreads();
    for (int e = t; e < E; e += 256) {
        const int32_t m = offsets[e + 1] - offsets[e];
        if (m < 0) s_err = 1;
        s_m[e] = m < 0 ? 0 : m;
    }
    __syncthreads();
    for (int e = t; e < E; e += 256) {
        if (mode == PLAN_RAGGED_REDUCTION) {
            // rank = number of experts ordered before e (larger M, ties by id)
            const int32_t me = s_m[e];
            int r = 0;
            for (int f = 0; f < E; ++f) r += (s_m[f] > me) || (s_m[f] == me && f < e);
            s_order[r] = e;
        } else {
            s_order[e] = e;
        }
    }
    __syncthreads();
    // tile counts in order position, then an exclusive scan: each thread owns
    // a contiguous chunk of positions.
    const int chunk = (E + 255) / 256;
    const int i0 = t * chunk, i1 = min(E, i0 + chunk);
    int32_t local = 0;
    for (int i = i0; i < i1; ++i) {
        const int e = s_order[i];
        const int32_t c = (mode == PLAN_RAGGED_REDUCTION) ? nt * kt : ((s_m[e] + bm - 1) / bm) * nt;
        local += c;
    }
    s_part[t] = local;
    __syncthreads();
    if (t == 0) {
        int32_t acc = 0;
        for (int i = 0; i < 256; ++i) { const int32_t v = s_part[i]; s_part[i] = acc; acc += v; }
        plan[PLAN_TOTAL] = s_err ? 0 : acc;
        plan[PLAN_ERR] = s_err;
        plan[PLAN_HDR + E] = acc;
    }
    __syncthreads();
    int32_t run = s_part[t];
    for (int i = i0; i < i1; ++i) {
        const int e = s_order[i];
        plan[PLAN_HDR + i] = run;
        plan[PLAN_HDR + E + 1 + i] = e;
        run += (mode == PLAN_RAGGED_REDUCTION) ? nt * kt : ((s_m[e] + bm - 1) / bm) * nt;
    }
    if (t < 8) plan[PLAN_CTR + t] = 0;
}

hipError_t launch_plan(const int32_t* offsets, int E, int64_t m_total, int mode, int bm, int nt, int kt,
                       int32_t* plan, hipStream_t s) {
    hipLaunchKernelGGL(k_plan, dim3(1), dim3(256), 0, s, offsets, E, m_total, mode, bm, nt, kt, plan);
    return hipGetLastError();
}

}  // namespace bsq
