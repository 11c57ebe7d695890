// Backward expert grouped GEMMs in MXFP8 on gfx950 (dgrad and wgrad).
//
// "Composer 2 Technical Report" (papercache.org summary), section 6.1: the MoE
// backward uses standard MXFP8 (E4M3 elements, E8M0 scale per 32); training
// runs three GEMMs per expert and layer (forward, dgrad, wgrad).  gfx950's
// v_mfma_scale_f32_32x32x64_f8f6f4 consumes exactly this format: E4M3
// operands plus one E8M0 scale per row and 32-element k block, applied inside
// the matrix core, so the kernel never dequantizes.
//
// Both GEMMs are "reduction-contiguous" (TN) products C[i][j] = sum_r
// A[i][r] B[j][r] with scales per 32 r:
//   dgrad  A = dY rows of expert e (ROWWISE codes), B = rows of W_e^T
//          (COLWISE_T codes of the weights), r = the n dimension;
//   wgrad  A = dY^T rows, B = X^T rows, both COLWISE_T over the tokens of
//          expert e, r = the expert's (32-padded) tokens.
//
// MFMA operand layout (measured on gfx950): for 32x32x64, lane l supplies row
// l%32; its first 16 bytes hold k in [16g, 16g+16) and its last 16 bytes
// k in [32+16g, 32+16g+16), g = l/32; the E8M0 scale of k-block b (k in
// [32b, 32b+32)) is taken from lane-group b.  A lane therefore reads bytes
// [16g, +16) and [32+16g, +16) of each 64-byte k step and the scale of block
// g: memory order is the hardware k order.
//
// Tiling: 256 x 256 outputs per workgroup (4 waves, 2 x 2, 128 x 128 each:
// 4 x 4 MFMA tiles, fp32 accumulators in AGPRs); 128-byte k stages double
// buffered in LDS, rows padded to 144 bytes (16-lane 16-byte reads hit
// distinct banks), next stage prefetched into registers during the MFMAs.
#include "device_common.h"
#include "gemm_common.h"

namespace bsq {

constexpr int BWD_BM = 256;
constexpr int BWD_BN = 256;
constexpr int BWD_BK = 128;             // k bytes (= elements) per stage
constexpr int BWD_PITCH = BWD_BK + 16;  // padded LDS row (bytes)

struct BwdSmem {
    uint8_t a[2][BWD_BM * BWD_PITCH];
    uint8_t b[2][BWD_BN * BWD_PITCH];
    uint32_t sa[2][BWD_BM];  // 4 scale bytes (blocks of the stage) per row
    uint32_t sb[2][BWD_BN];
};


// One output tile of C[i][j] = sum_r A[i][r] B[j][r].
struct TileOps {
    const uint8_t* a; const uint8_t* as; int64_t lda, ldas; int rows_a;
    const uint8_t* b; const uint8_t* bs; int64_t ldb, ldbs; int rows_b;
    int64_t R;  // reduction length (multiple of 32)
    char* c; int64_t ldc;
};

__global__ __launch_bounds__(256, 1) void k_gemm_bwd_mxfp8(BwdArgs p) {
    extern __shared__ __align__(16) uint8_t smem_raw[];
    BwdSmem& sm = *reinterpret_cast<BwdSmem*>(smem_raw);
    __shared__ int s_tile;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int lr = lane & 31, g = lane >> 5;
    const int xcd = blockIdx.x & 7;
    const int esz = p.out_f32 ? 4 : 2;
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
        TileOps op;
        if (!p.wgrad) {
            // dX[m][k] = sum_n dY[m][n] Wt_e[k][n]
            const int KT = (int)((p.K + BWD_BN - 1) / BWD_BN);
            const int mt = local / KT, kt = local % KT;
            const int64_t m0 = off0 + (int64_t)mt * BWD_BM, k0 = (int64_t)kt * BWD_BN;
            const int64_t cw = (int64_t)e * (p.N + 32);  // 32*(e + e*N/32): segment start of W_e
            op.a = p.dy_codes + m0 * p.N; op.as = p.dy_scale + m0 * (p.N / 32);
            op.lda = p.N; op.ldas = p.N / 32; op.rows_a = (int)min((int64_t)BWD_BM, off1 - m0);
            op.b = p.wt_codes + k0 * p.Pw + cw; op.bs = p.wt_scale + k0 * (p.Pw / 32) + cw / 32;
            op.ldb = p.Pw; op.ldbs = p.Pw / 32; op.rows_b = (int)min((int64_t)BWD_BN, p.K - k0);
            op.R = p.N;
            op.c = reinterpret_cast<char*>(p.out) + (m0 * p.K + k0) * esz; op.ldc = p.K;
        } else {
            // dW_e[n][k] = sum_{m in e} dY^T[n][m] X^T[k][m]
            const int KT = (int)((p.K + BWD_BN - 1) / BWD_BN);
            const int nt = local / KT, kt = local % KT;
            const int64_t n0 = (int64_t)nt * BWD_BM, k0 = (int64_t)kt * BWD_BN;
            const int64_t c0 = 32 * ((int64_t)e + off0 / 32);  // segment start column
            op.a = p.dyt_codes + n0 * p.P + c0; op.as = p.dyt_scale + n0 * (p.P / 32) + c0 / 32;
            op.lda = p.P; op.ldas = p.P / 32; op.rows_a = (int)min((int64_t)BWD_BM, p.N - n0);
            op.b = p.xt_codes + k0 * p.P + c0; op.bs = p.xt_scale + k0 * (p.P / 32) + c0 / 32;
            op.ldb = p.P; op.ldbs = p.P / 32; op.rows_b = (int)min((int64_t)BWD_BN, p.K - k0);
            op.R = 32 * ((off1 - off0 + 31) / 32);
            op.c = reinterpret_cast<char*>(p.out) + (((int64_t)e * p.N + n0) * p.K + k0) * esz; op.ldc = p.K;
        }
        op.a = uniform_ptr(op.a); op.as = uniform_ptr(op.as);
        op.b = uniform_ptr(op.b); op.bs = uniform_ptr(op.bs);
        op.c = uniform_ptr(op.c);
        op.lda = uniform_i64(op.lda); op.ldas = uniform_i64(op.ldas);
        op.ldb = uniform_i64(op.ldb); op.ldbs = uniform_i64(op.ldbs);
        op.ldc = uniform_i64(op.ldc); op.R = uniform_i64(op.R);
        op.rows_a = __builtin_amdgcn_readfirstlane(op.rows_a);
        op.rows_b = __builtin_amdgcn_readfirstlane(op.rows_b);
        const int nstages = (int)((op.R + BWD_BK - 1) / BWD_BK);

        uint4 ra[8], rb[8];
        uint32_t rsa, rsb;
        const __amdgpu_buffer_rsrc_t rA = make_rsrc(op.a, 0x7FFFFFFFu);
        const __amdgpu_buffer_rsrc_t rB = make_rsrc(op.b, 0x7FFFFFFFu);
        const __amdgpu_buffer_rsrc_t rAs = make_rsrc(op.as, 0x7FFFFFFFu);
        const __amdgpu_buffer_rsrc_t rBs = make_rsrc(op.bs, 0x7FFFFFFFu);
        const uint32_t lda = (uint32_t)op.lda, ldb = (uint32_t)op.ldb;
        const uint32_t ldas = (uint32_t)op.ldas, ldbs = (uint32_t)op.ldbs;
        const uint32_t R = (uint32_t)op.R;
        auto load_stage = [&](int s) {
            const uint32_t q = tid & 7;
            const uint32_t kb = (uint32_t)s * BWD_BK + 16 * q;
            const bool okk = kb < R;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = (tid >> 3) + 32 * i;
                ra[i] = buf_load16(rA, (okk && r < op.rows_a) ? r * lda + kb : OOB);
                rb[i] = buf_load16(rB, (okk && r < op.rows_b) ? r * ldb + kb : OOB);
            }
            // 4 scale bytes per row (row = tid); byte loads: the scale row
            // pitch need not be 4-byte aligned.
            const uint32_t sblk = (uint32_t)s * (BWD_BK / 32);
            const uint32_t nblk = R / 32;
            uint32_t va = 0, vb = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bool okb = sblk + j < nblk;
                va |= buf_load1(rAs, (okb && tid < op.rows_a) ? tid * ldas + sblk + j : OOB) << (8 * j);
                vb |= buf_load1(rBs, (okb && tid < op.rows_b) ? tid * ldbs + sblk + j : OOB) << (8 * j);
            }
            rsa = va;
            rsb = vb;
        };
        auto store_stage = [&](int buf) {
            const int q = tid & 7;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = (tid >> 3) + 32 * i;
                *reinterpret_cast<uint4*>(&sm.a[buf][r * BWD_PITCH + 16 * q]) = ra[i];
                *reinterpret_cast<uint4*>(&sm.b[buf][r * BWD_PITCH + 16 * q]) = rb[i];
            }
            sm.sa[buf][tid] = rsa;
            sm.sb[buf][tid] = rsb;
        };

        float16v acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

        if (nstages > 0) {
            load_stage(0);
            store_stage(0);
        }
        __syncthreads();
        for (int s = 0; s < nstages; ++s) {
            const int buf = s & 1;
            if (s + 1 < nstages) load_stage(s + 1);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {  // 64-byte MFMA k steps
                int8v fa[4], fb[4];
                int sca[4], scb[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int ra_ = wm * 128 + 32 * i + lr;
                    const int rb_ = wn * 128 + 32 * i + lr;
                    const uint8_t* pa = &sm.a[buf][ra_ * BWD_PITCH + 64 * kk + 16 * g];
                    const uint8_t* pb = &sm.b[buf][rb_ * BWD_PITCH + 64 * kk + 16 * g];
                    const uint4 a0 = *reinterpret_cast<const uint4*>(pa);
                    const uint4 a1 = *reinterpret_cast<const uint4*>(pa + 32);
                    const uint4 b0 = *reinterpret_cast<const uint4*>(pb);
                    const uint4 b1 = *reinterpret_cast<const uint4*>(pb + 32);
                    fa[i] = int8v{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
                    fb[i] = int8v{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
                    sca[i] = (int)((sm.sa[buf][ra_] >> (8 * (2 * kk + g))) & 0xFFu);
                    scb[i] = (int)((sm.sb[buf][rb_] >> (8 * (2 * kk + g))) & 0xFFu);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            fa[i], fb[j], acc[i][j], 0, 0, 0, sca[i], 0, scb[j]);
            }
            if (s + 1 < nstages) store_stage(buf ^ 1);
            __syncthreads();
        }

        // Epilogue: fp32 accumulators -> f32 or bf16 (round to nearest even).
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = wn * 128 + 32 * j + lr;
            if (col >= op.rows_b) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int row = wm * 128 + 32 * i + 8 * (v >> 2) + 4 * g + (v & 3);
                    if (row >= op.rows_a) continue;
                    const int64_t o = (int64_t)row * op.ldc + col;
                    if (p.out_f32)
                        reinterpret_cast<float*>(op.c)[o] = acc[i][j][v];
                    else
                        reinterpret_cast<uint16_t*>(op.c)[o] = (uint16_t)f32_to_bf16_rne(acc[i][j][v]);
                }
            }
        }
    }
}

size_t bwd_smem_bytes() { return sizeof(BwdSmem); }

hipError_t launch_gemm_bwd_mxfp8(const BwdArgs& args, int grid, hipStream_t s) {
    const int KT = (int)((args.K + BWD_BN - 1) / BWD_BN);
    hipError_t err;
    if (args.wgrad) {
        const int NTn = (int)((args.N + BWD_BM - 1) / BWD_BM);
        err = launch_plan(args.offsets, args.E, args.m_total, PLAN_RAGGED_REDUCTION, 1, NTn, KT, args.plan, s);
    } else {
        err = launch_plan(args.offsets, args.E, args.m_total, PLAN_RAGGED_ROWS, BWD_BM, KT, 1, args.plan, s);
    }
    if (err != hipSuccess) return err;
    static bool attr_set = false;  // idempotent; racing writers set the same value
    if (!attr_set) {
        err = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_bwd_mxfp8),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(BwdSmem));
        if (err != hipSuccess) return err;
        attr_set = true;
    }
    hipLaunchKernelGGL(k_gemm_bwd_mxfp8, dim3(grid), dim3(256), sizeof(BwdSmem), s, args);
    return hipGetLastError();
}

}  // namespace bsq
