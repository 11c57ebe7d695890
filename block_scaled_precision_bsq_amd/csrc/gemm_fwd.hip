// Forward expert grouped GEMM over NVFP4-variant operands (gfx950).
//
//   y[m][n] = s_a[m] * s_w[n] * sum_k (q_a * S_a)[m][k] * (q_w * S_w)[n][k]
//
// "Composer 2 Technical Report" (papercache.org summary), section 6.1: the
// MoE forward runs its grouped GEMM on the NVFP4 variant and applies the
// per-token FP32 scale in the GEMM epilogue; on the pages' hardware the block
// scales are dequantized inside the tensor-core MMA.
//
// gfx950 design.  The block-scaled f8f6f4 MFMA takes one power-of-two (E8M0)
// scale per 32 elements, while this format has an arbitrary E4M3 scale per 16
// elements, so it cannot carry S_b exactly.  Every E2M1 x E4M3 product q*S_b
// is exact in fp16 (at most 6 significant bits, magnitude in [2^-10, 2688]),
// so the kernel dequantizes in registers -- one v_cvt_scalef32_pk_f16_fp4
// (two E2M1 codes -> two fp16, unit scale) and one packed fp16 multiply by S_b
// per pair of elements -- and feeds exact fp16 operands to the dense
// v_mfma_f32_32x32x16_f16 with fp32 accumulation.  HBM and LDS only ever see
// the 4.5-bit encoding (codes + scale bytes).
//
// Tiling: 256 x 256 output tile per workgroup of 4 waves (2 x 2, 128 x 128
// per wave = 4 x 4 MFMA 32x32 tiles, fp32 accumulators in AGPRs).  K runs in
// stages of 128 elements (64 code bytes + 8 scale bytes per row), double
// buffered in LDS with the next stage prefetched into registers while the
// current one is multiplied.  LDS rows are padded to 80 bytes so the 16-byte
// fragment reads of 16 consecutive rows hit distinct banks.
#include "device_common.h"
#include "gemm_common.h"

namespace bsq {

constexpr int FWD_BM = 256;
constexpr int FWD_BN = 256;
constexpr int FWD_BK = 128;              // K elements per stage
constexpr int FWD_KB = FWD_BK / 2;       // code bytes per row per stage
constexpr int FWD_SB = FWD_BK / 16;      // scale bytes per row per stage
constexpr int FWD_PITCH = FWD_KB + 16;   // padded LDS row (bytes)

struct FwdSmem {
    uint8_t a[2][FWD_BM * FWD_PITCH];
    uint8_t b[2][FWD_BN * FWD_PITCH];
    uint32_t sa[2][FWD_BM * 2];
    uint32_t sb[2][FWD_BN * 2];
};

// Eight E2M1 codes (one 32-bit word, element 0 in the low nibble) times the
// block scale -> eight exact fp16 values.
__device__ __forceinline__ half8 dequant8(uint32_t w, half2v s) {
    half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s;
    half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s;
    half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s;
    half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s;
    half8 r;
    r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
    r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
    return r;
}

__device__ __forceinline__ half2v scale_pair(uint32_t byte) {
    const _Float16 h = (_Float16)e4m3_value(byte & 0x7Fu);
    half2v r;
    r[0] = h;
    r[1] = h;
    return r;
}

struct FwdArgs {
    const uint8_t* a_codes; const uint8_t* a_bscale; const float* a_rscale;
    const uint8_t* w_codes; const uint8_t* w_bscale; const float* w_rscale;
    const int32_t* offsets; int E; int64_t N; int64_t K;
    void* y; int y_f32; int32_t* plan;
};

__global__ __launch_bounds__(256, 1) void k_gemm_fwd_nvfp4v(FwdArgs p) {
    extern __shared__ __align__(16) uint8_t smem_raw[];
    FwdSmem& sm = *reinterpret_cast<FwdSmem*>(smem_raw);
    __shared__ int s_tile;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int lr = lane & 31, h = lane >> 5;
    const int xcd = blockIdx.x & 7;
    const int64_t KB = p.K / 2, KS = p.K / 16;  // row pitch of codes and scales (bytes)
    const int nstages = (int)((p.K + FWD_BK - 1) / FWD_BK);
    const int NT = (int)((p.N + FWD_BN - 1) / FWD_BN);
    const int total = p.plan[PLAN_TOTAL];
    const int32_t* start = plan_start(p.plan);
    const int32_t* order = plan_order(p.plan, p.E);
    int dq = 0;

    for (;;) {
        if (tid == 0) s_tile = claim_tile(p.plan, xcd, total, dq);
        __syncthreads();
        const int tile = __builtin_amdgcn_readfirstlane(s_tile);  // uniform: keeps tile state in SGPRs
        __syncthreads();
        if (tile < 0) break;

        // Tile decode; readfirstlane marks the results wave-uniform so that
        // addresses and buffer resources stay in SGPRs.
        const int pos = find_position(start, p.E, tile);
        const int e = __builtin_amdgcn_readfirstlane(order[pos]);
        const int local = __builtin_amdgcn_readfirstlane(tile - start[pos]);
        const int64_t off0 = __builtin_amdgcn_readfirstlane(p.offsets[e]);
        const int64_t off1 = __builtin_amdgcn_readfirstlane(p.offsets[e + 1]);
        int mt, nt;
        grouped_tile(local, (int)((off1 - off0 + FWD_BM - 1) / FWD_BM), NT, mt, nt);
        const int64_t m_base = off0 + (int64_t)mt * FWD_BM;
        const int rows_a = (int)min((int64_t)FWD_BM, off1 - m_base);
        const int64_t n_base = (int64_t)nt * FWD_BN;
        const int rows_b = (int)min((int64_t)FWD_BN, p.N - n_base);
        const uint8_t* ga = p.a_codes + m_base * KB;
        const uint8_t* gsa = p.a_bscale + m_base * KS;
        const uint8_t* gb = p.w_codes + ((int64_t)e * p.N + n_base) * KB;
        const uint8_t* gsb = p.w_bscale + ((int64_t)e * p.N + n_base) * KS;

        // Global -> register staging for one stage (buffer loads: 32-bit
        // offsets, out-of-range rows and k tails read as zero codes).
        uint4 ra[4], rb[4];
        uint32_t rsa[2], rsb[2];
        const __amdgpu_buffer_rsrc_t rA = make_rsrc(ga, 0x7FFFFFFFu);
        const __amdgpu_buffer_rsrc_t rB = make_rsrc(gb, 0x7FFFFFFFu);
        const __amdgpu_buffer_rsrc_t rAs = make_rsrc(gsa, 0x7FFFFFFFu);
        const __amdgpu_buffer_rsrc_t rBs = make_rsrc(gsb, 0x7FFFFFFFu);
        const uint32_t kb32 = (uint32_t)KB, ks32 = (uint32_t)KS;
        auto load_stage = [&](int s) {
            const uint32_t q = tid & 3;
            const uint32_t kb = (uint32_t)s * FWD_KB + 16 * q;
            const bool okk = kb < kb32;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = (tid >> 2) + 64 * i;
                ra[i] = buf_load16(rA, (okk & (r < rows_a)) ? r * kb32 + kb : OOB);
                rb[i] = buf_load16(rB, (okk & (r < rows_b)) ? r * kb32 + kb : OOB);
            }
            const uint32_t ks = (uint32_t)s * FWD_SB;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const bool okj = ks + 4 * j < ks32;
                rsa[j] = buf_load4(rAs, (okj & (tid < rows_a)) ? tid * ks32 + ks + 4 * j : OOB);
                rsb[j] = buf_load4(rBs, (okj & (tid < rows_b)) ? tid * ks32 + ks + 4 * j : OOB);
            }
        };
        auto store_stage = [&](int buf) {
            const int q = tid & 3;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = (tid >> 2) + 64 * i;
                *reinterpret_cast<uint4*>(&sm.a[buf][r * FWD_PITCH + 16 * q]) = ra[i];
                *reinterpret_cast<uint4*>(&sm.b[buf][r * FWD_PITCH + 16 * q]) = rb[i];
            }
            sm.sa[buf][2 * tid] = rsa[0];
            sm.sa[buf][2 * tid + 1] = rsa[1];
            sm.sb[buf][2 * tid] = rsb[0];
            sm.sb[buf][2 * tid + 1] = rsb[1];
        };

        float16v acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

        load_stage(0);
        store_stage(0);
        __syncthreads();
        for (int s = 0; s < nstages; ++s) {
            const int buf = s & 1;
            // Prefetch the next stage (out-of-range offsets past the last stage
            // read zeros: the loop body stays one basic block).
            load_stage(s + 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll 1
            for (int c = 0; c < 2; ++c) {  // 64-element chunks of the stage
                uint4 qa[4], qb[4];
                uint32_t sca[4], scb[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int ra_ = wm * 128 + 32 * i + lr;
                    const int rb_ = wn * 128 + 32 * i + lr;
                    qa[i] = *reinterpret_cast<const uint4*>(&sm.a[buf][ra_ * FWD_PITCH + 32 * c + 16 * h]);
                    qb[i] = *reinterpret_cast<const uint4*>(&sm.b[buf][rb_ * FWD_PITCH + 32 * c + 16 * h]);
                    // scale bytes of blocks 4c+2h and 4c+2h+1 of the stage
                    sca[i] = (sm.sa[buf][2 * ra_ + c] >> (16 * h)) & 0xFFFFu;
                    scb[i] = (sm.sb[buf][2 * rb_ + c] >> (16 * h)) & 0xFFFFu;
                }
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    half8 fa[4], fb[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t wa = kk == 0 ? qa[i].x : kk == 1 ? qa[i].y : kk == 2 ? qa[i].z : qa[i].w;
                        const uint32_t wb = kk == 0 ? qb[i].x : kk == 1 ? qb[i].y : kk == 2 ? qb[i].z : qb[i].w;
                        fa[i] = dequant8(wa, scale_pair(sca[i] >> (8 * (kk >> 1))));
                        fb[i] = dequant8(wb, scale_pair(scb[i] >> (8 * (kk >> 1))));
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            store_stage(buf ^ 1);
            __syncthreads();
        }

        // Epilogue: per-token and per-output-channel fp32 scales, then store.
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = wn * 128 + 32 * j + lr;
            if (col >= rows_b) continue;
            const float sw = p.w_rscale[(int64_t)e * p.N + n_base + col];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int row = wm * 128 + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
                    if (row >= rows_a) continue;
                    const float val = (acc[i][j][v] * p.a_rscale[m_base + row]) * sw;
                    const int64_t off = (m_base + row) * p.N + n_base + col;
                    if (p.y_f32)
                        reinterpret_cast<float*>(p.y)[off] = val;
                    else
                        reinterpret_cast<uint16_t*>(p.y)[off] = (uint16_t)f32_to_bf16_rne(val);
                }
            }
        }
    }
}

size_t fwd_smem_bytes() { return sizeof(FwdSmem); }

hipError_t launch_gemm_fwd_nvfp4v(const uint8_t* a_codes, const uint8_t* a_bscale, const float* a_rscale,
                                  const uint8_t* w_codes, const uint8_t* w_bscale, const float* w_rscale,
                                  const int32_t* offsets, int E, int64_t m_total, int64_t N, int64_t K, void* y,
                                  int y_f32, int32_t* plan, int grid, hipStream_t s) {
    const int NT = (int)((N + FWD_BN - 1) / FWD_BN);
    hipError_t err = launch_plan(offsets, E, m_total, PLAN_RAGGED_ROWS, FWD_BM, NT, 1, plan, s);
    if (err != hipSuccess) return err;
    static bool attr_set = false;  // idempotent; racing writers set the same value
    if (!attr_set) {
        err = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_fwd_nvfp4v),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(FwdSmem));
        if (err != hipSuccess) return err;
        attr_set = true;
    }
    FwdArgs p{a_codes, a_bscale, a_rscale, w_codes, w_bscale, w_rscale, offsets, E, N, K, y, y_f32, plan};
    hipLaunchKernelGGL(k_gemm_fwd_nvfp4v, dim3(grid), dim3(256), sizeof(FwdSmem), s, p);
    return hipGetLastError();
}

}  // namespace bsq
