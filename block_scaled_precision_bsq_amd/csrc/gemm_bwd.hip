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
// 4 x 4 MFMA tiles, fp32 accumulators in AGPRs).  k runs in 64-byte stages
// (one MFMA k step) through a 4-deep LDS ring filled by buffer-to-LDS DMA
// (gemm_pipe.h): three stages are in flight while one is multiplied, and the
// fragments of stage s+1 are read from LDS into a second register set while
// the MFMAs of stage s run.
#include "device_common.h"
#include "gemm_common.h"
#include "gemm_pipe.h"

#include <type_traits>
#include <stddef.h>

namespace bsq {

constexpr int BWD_BM = 256;
constexpr int BWD_BN = 256;
constexpr int BWD_DMA_PER_STAGE = 12;  // DMA instructions per wave per stage

struct BwdSmem {
    uint8_t a[PIPE_NST][PIPE_STAGE_BYTES];
    uint8_t b[PIPE_NST][PIPE_STAGE_BYTES];
    uint32_t sa[PIPE_NST][PIPE_ROWS * 2];  // E8M0 byte of (block, row) in dword block*256 + row
    uint32_t sb[PIPE_NST][PIPE_ROWS * 2];
};

// One output tile of C[i][j] = sum_r A[i][r] B[j][r].
struct TileOps {
    const uint8_t* a; const uint8_t* as; int64_t lda, ldas; int rows_a;
    const uint8_t* b; const uint8_t* bs; int64_t ldb, ldbs; int rows_b;
    int64_t R;  // reduction length (multiple of 32)
    char* c; int64_t ldc;
};

struct BwdFrag {
    int8v a[4], b[4];
    int sa[4], sb[4];
};

template <int V> using IC = std::integral_constant<int, V>;

template <bool OUT_F32>
__global__ __launch_bounds__(256, 1) void k_gemm_bwd_mxfp8(BwdArgs p) {
    extern __shared__ __align__(16) uint8_t smem_raw[];
    __shared__ int s_tile;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave-uniform by construction; readfirstlane lets the compiler keep
    // everything derived from it in SGPRs
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int lr = lane & 31, g = lane >> 5;
    const int xcd = blockIdx.x & 7;
    constexpr int esz = OUT_F32 ? 4 : 2;
    const int total = p.plan[PLAN_TOTAL];
    const int32_t* start = plan_start(p.plan);
    const int32_t* order = plan_order(p.plan, p.E);
    int dq = 0;

    // 32-bit LDS byte addresses of the ring buffers
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem_raw));
    const uint32_t LA = lds0 + offsetof(BwdSmem, a), LB = lds0 + offsetof(BwdSmem, b);
    const uint32_t LSA = lds0 + offsetof(BwdSmem, sa), LSB = lds0 + offsetof(BwdSmem, sb);
    // fragment reads address the same buffers relative to smem_raw
    const __attribute__((address_space(3))) uint8_t* lds =
        (const __attribute__((address_space(3))) uint8_t*)(smem_raw);

    // DMA lane geometry (tile-invariant): instruction i of this wave covers
    // rows 16 * (4 * wave + i) + lane / 4; the lane fetches logical chunk
    // (lane & 3) ^ swz(row) of its row into slot lane & 3.  swz(row) depends
    // only on bits 1..3 of the row, i.e. on lane / 4.
    const int drow0 = 64 * wave + (lane >> 2);
    const uint32_t dchunk = (uint32_t)((lane & 3) ^ swz(lane >> 2));
    const bool dlow = dchunk < 2;  // chunk lies in the first 32-byte k block
    // Fragment read geometry: lane (lr, g) reads chunks g and g + 2 of row
    // lr of each 32-row group; swz(row) = swz(lr) for every such row.
    const uint32_t fr0 = (uint32_t)(lr * PIPE_BK + 16 * (g ^ swz(lr)));
    const uint32_t fr1 = fr0 ^ 32u;  // chunk g + 2
    const uint32_t fa = offsetof(BwdSmem, a) + (uint32_t)(wm * 128 * PIPE_BK);
    const uint32_t fb = offsetof(BwdSmem, b) + (uint32_t)(wn * 128 * PIPE_BK);
    const uint32_t fsa = offsetof(BwdSmem, sa) + 4u * (uint32_t)(256 * g + wm * 128 + lr);
    const uint32_t fsb = offsetof(BwdSmem, sb) + 4u * (uint32_t)(256 * g + wn * 128 + lr);

    for (;;) {
        if (tid == 0) s_tile = claim_tile(p.plan, xcd, total, dq);
        __syncthreads();
        const int tile = __builtin_amdgcn_readfirstlane(s_tile);  // uniform: keeps tile state in SGPRs
        __syncthreads();
        if (tile < 0) break;

        // Tile decode; readfirstlane marks the results wave-uniform so that
        // addresses and buffer descriptors stay in SGPRs.
        const int pos = find_position(start, p.E, tile);
        const int e = __builtin_amdgcn_readfirstlane(order[pos]);
        const int local = __builtin_amdgcn_readfirstlane(tile - start[pos]);
        const int64_t off0 = __builtin_amdgcn_readfirstlane(p.offsets[e]);
        const int64_t off1 = __builtin_amdgcn_readfirstlane(p.offsets[e + 1]);
        TileOps op;
        if (!p.wgrad) {
            // dX[m][k] = sum_n dY[m][n] Wt_e[k][n]
            const int KT = (int)((p.K + BWD_BN - 1) / BWD_BN);
            int mt, kt;
            grouped_tile(local, (int)((off1 - off0 + BWD_BM - 1) / BWD_BM), KT, mt, kt);
            const int64_t m0 = off0 + (int64_t)mt * BWD_BM, k0 = (int64_t)kt * BWD_BN;
            const int64_t cw = (int64_t)e * (p.N + 32);  // 32*(e + e*N/32): segment start of W_e
            // block-major scales: block j of rows r0.. starts at base + j * rows_total + r0
            op.a = p.dy_codes + m0 * p.N; op.as = p.dy_scale + m0;
            op.lda = p.N; op.ldas = p.m_total; op.rows_a = (int)min((int64_t)BWD_BM, off1 - m0);
            op.b = p.wt_codes + k0 * p.Pw + cw; op.bs = p.wt_scale + (cw / 32) * p.K + k0;
            op.ldb = p.Pw; op.ldbs = p.K; op.rows_b = (int)min((int64_t)BWD_BN, p.K - k0);
            op.R = p.N;
            op.c = reinterpret_cast<char*>(p.out) + (m0 * p.K + k0) * esz; op.ldc = p.K;
        } else {
            // dW_e[n][k] = sum_{m in e} dY^T[n][m] X^T[k][m]
            const int KT = (int)((p.K + BWD_BN - 1) / BWD_BN);
            int nt, kt;
            grouped_tile(local, (int)((p.N + BWD_BM - 1) / BWD_BM), KT, nt, kt);
            const int64_t n0 = (int64_t)nt * BWD_BM, k0 = (int64_t)kt * BWD_BN;
            const int64_t c0 = 32 * ((int64_t)e + off0 / 32);  // segment start column
            op.a = p.dyt_codes + n0 * p.P + c0; op.as = p.dyt_scale + (c0 / 32) * p.N + n0;
            op.lda = p.P; op.ldas = p.N; op.rows_a = (int)min((int64_t)BWD_BM, p.N - n0);
            op.b = p.xt_codes + k0 * p.P + c0; op.bs = p.xt_scale + (c0 / 32) * p.K + k0;
            op.ldb = p.P; op.ldbs = p.K; op.rows_b = (int)min((int64_t)BWD_BN, p.K - k0);
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
        const int nstages = (int)((op.R + PIPE_BK - 1) / PIPE_BK);

        const i32x4 dA = make_desc(op.a), dB = make_desc(op.b);
        const i32x4 dAs = make_desc(op.as), dBs = make_desc(op.bs);
        const uint32_t lda = (uint32_t)op.lda, ldb = (uint32_t)op.ldb;
        const uint32_t ldas = (uint32_t)op.ldas, ldbs = (uint32_t)op.ldbs;
        const uint32_t R = (uint32_t)op.R;

        // Per-tile lane offsets at k = 0; rows past the tile read as zero.
        uint32_t va[4], vb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = drow0 + 16 * i;
            va[i] = row < op.rows_a ? (uint32_t)row * lda + 16 * dchunk : OOB;
            vb[i] = row < op.rows_b ? (uint32_t)row * ldb + 16 * dchunk : OOB;
        }
        // scales: instruction i (of 2) covers k block (2 * wave + i) >> 2 of
        // the stage, rows 64 * ((2 * wave + i) & 3) + lane
        uint32_t vsa[2], vsb[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int ins = 2 * wave + i;
            const int row = 64 * (ins & 3) + lane;
            const uint32_t kb = (uint32_t)(ins >> 2);
            vsa[i] = row < op.rows_a ? kb * ldas + row : OOB;
            vsb[i] = row < op.rows_b ? kb * ldbs + row : OOB;
        }

        // DMA of stage st into ring slot st % 4: 12 instructions per wave,
        // issued in 5 parts (part i < 4: A and B rows of instruction i; part
        // 4: the four scale instructions).  Stages past the end land as
        // zeros, which keeps the per-stage instruction count, and so the
        // vmcnt bookkeeping, uniform.  R is a multiple of 32: a stage is
        // either whole, half (its first k block only) or past the end.
        auto issue_part = [&](int st, int part) {
            const uint32_t q = (uint32_t)st & (PIPE_NST - 1);
            const uint32_t kbase = (uint32_t)st * PIPE_BK;
            if (part < 4) {
                const bool full = kbase + PIPE_BK <= R;
                const bool half = kbase + 32 == R;
                const bool okc = full | (half & dlow);
                const uint32_t ldst = q * PIPE_STAGE_BYTES + 1024u * (uint32_t)(4 * wave + part);
                dma16(dA, okc ? va[part] + kbase : OOB, LA + ldst);
                dma16(dB, okc ? vb[part] + kbase : OOB, LB + ldst);
            } else {
                const uint32_t sblk = 2 * (uint32_t)st;  // first k block of the stage
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int ins = 2 * wave + i;
                    const bool oks = (sblk + (uint32_t)(ins >> 2)) * 32 < R;
                    const uint32_t ldst = 4u * (q * 512u + 64u * (uint32_t)ins);
                    dma1(dAs, oks ? vsa[i] + sblk * ldas : OOB, LSA + ldst);
                    dma1(dBs, oks ? vsb[i] + sblk * ldbs : OOB, LSB + ldst);
                }
            }
        };
        auto issue = [&](int st) {
#pragma unroll
            for (int part = 0; part < 5; ++part) issue_part(st, part);
        };
        // Fragments of the stage in ring slot Q: lane (row, g) takes logical
        // chunks g and g+2 of its row (k bytes [16g, +16) and [32+16g, +16):
        // the MFMA's k order) and the scale of block g.  Part 2i reads the A
        // rows of group i, part 2i+1 the B rows.
        auto read_part = [&](uint32_t Q, BwdFrag& f, int part) {
            const int i = part >> 1;
            const uint32_t so = ((part & 1) ? fsb : fsa) + Q * 2048u + 128u * i;
            const uint32_t o = ((part & 1) ? fb : fa) + Q * PIPE_STAGE_BYTES + (uint32_t)(32 * i * PIPE_BK);
            const u32x4 x0 = *(const __attribute__((address_space(3))) u32x4*)(lds + o + fr0);
            const u32x4 x1 = *(const __attribute__((address_space(3))) u32x4*)(lds + o + fr1);
            const int sc = *(const __attribute__((address_space(3))) int*)(lds + so);
            const int8v v = int8v{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
            if (part & 1) { f.b[i] = v; f.sb[i] = sc; } else { f.a[i] = v; f.sa[i] = sc; }
        };
        auto read = [&](uint32_t Q, BwdFrag& f) {
#pragma unroll
            for (int part = 0; part < 8; ++part) read_part(Q, f, part);
        };

        float16v acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

        auto mma = [&](const BwdFrag& f) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[i], f.b[j], acc[i][j], 0, 0, 0,
                                                                              f.sa[i], 0, f.sb[j]);
        };
        // One pipeline step at stage s (fragments in cur): wait until stage
        // s+1 has landed and every wave holds stage s in registers, then run
        // the 16 MFMAs of stage s with the refill of ring slot s % 4 (stage
        // s+4) and the reads of stage s+1 into nxt slotted in between them.
        // sched_barrier pins the interleave: the memory work issues in the
        // shadow of the matrix core instead of in front of it.
        auto step = [&](int s, const BwdFrag& cur, BwdFrag& nxt) {
            wait_vmcnt<2 * BWD_DMA_PER_STAGE>();
            wait_lgkmcnt0();
            block_barrier();
            const uint32_t qn = (uint32_t)(s + 1) & (PIPE_NST - 1);
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const int i = k >> 2, j = k & 3;
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cur.a[i], cur.b[j], acc[i][j], 0, 0, 0,
                                                                          cur.sa[i], 0, cur.sb[j]);
                if (k < 5) issue_part(s + 4, k);
                else if (k >= 6 && k < 14) read_part(qn, nxt, k - 6);
                __builtin_amdgcn_sched_barrier(0);
            }
        };

        // Prologue: stages 0..3 in flight, stage 0 read into X.
        issue(0); issue(1); issue(2); issue(3);
        wait_vmcnt<3 * BWD_DMA_PER_STAGE>();
        block_barrier();
        BwdFrag X, Y;
        read(0, X);
        int s = 0;
        for (; s + 1 < nstages; s += 2) {
            step(s, X, Y);
            step(s + 1, Y, X);
        }
        if (s < nstages) {
            wait_lgkmcnt0();
            mma(X);
        }
        // drain every DMA of this tile before the ring is reused
        wait_vmcnt<0>();
        wait_lgkmcnt0();
        block_barrier();

        // Epilogue: fp32 accumulators -> f32 or bf16 (round to nearest even)
        // through buffer stores.  Lane (lr, g) holds column wn*128 + 32j + lr
        // of rows wm*128 + 32i + 8(v/4) + 4g + v%4; a running row offset
        // walks the rows and the column tile goes into the immediate offset.
        // Lanes outside a partial tile get an out-of-range offset and store
        // nothing.
        {
            const __amdgpu_buffer_rsrc_t rc = make_rsrc(op.c, 0x7FFFFFFFu);
            const uint32_t ldcb = (uint32_t)op.ldc * (uint32_t)esz;
            const int lcol = wn * 128 + lr;
            int row = wm * 128 + 4 * g;
            uint32_t vrow = (uint32_t)row * ldcb + (uint32_t)lcol * (uint32_t)esz;
            const bool whole = (op.rows_a == BWD_BM) & (op.rows_b == BWD_BN);
            bool okc[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) okc[j] = lcol + 32 * j < op.rows_b;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int vq = 0; vq < 4; ++vq) {
#pragma unroll
                    for (int vr = 0; vr < 4; ++vr) {
                        const bool okr = whole | (row < op.rows_a);
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const float x = acc[i][j][4 * vq + vr];
                            const uint32_t vo = (whole | (okr & okc[j])) ? vrow + (uint32_t)(32 * j * esz) : OOB;
                            if constexpr (OUT_F32)
                                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), rc, (int)vo, 0, 0);
                            else
                                __builtin_amdgcn_raw_buffer_store_b16((uint16_t)f32_to_bf16_rne(x), rc, (int)vo, 0, 0);
                        }
                        row += 1;
                        vrow += ldcb;
                    }
                    row += 4;
                    vrow += 4 * ldcb;
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
        err = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_bwd_mxfp8<true>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(BwdSmem));
        if (err != hipSuccess) return err;
        err = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_bwd_mxfp8<false>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(BwdSmem));
        if (err != hipSuccess) return err;
        attr_set = true;
    }
    if (args.out_f32)
        hipLaunchKernelGGL(k_gemm_bwd_mxfp8<true>, dim3(grid), dim3(256), sizeof(BwdSmem), s, args);
    else
        hipLaunchKernelGGL(k_gemm_bwd_mxfp8<false>, dim3(grid), dim3(256), sizeof(BwdSmem), s, args);
    return hipGetLastError();
}

}  // namespace bsq
