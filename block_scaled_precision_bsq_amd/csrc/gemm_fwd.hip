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
// so the kernel dequantizes in registers -- v_cvt_scalef32_pk_f16_fp4 (two
// E2M1 codes -> two fp16, unit scale) and one packed fp16 multiply by S_b per
// pair of elements, S_b itself converted by v_cvt_scalef32_pk_f16_fp8 -- and
// feeds exact fp16 operands to the dense v_mfma_f32_32x32x16_f16 with fp32
// accumulation.  HBM and LDS only ever see the 4.5-bit encoding.
//
// Tiling: 256 x 256 outputs per workgroup (4 waves, 2 x 2, 128 x 128 each:
// 4 x 4 MFMA tiles, fp32 accumulators in AGPRs).  K runs in super-stages of
// 256 elements: 128 code bytes + 16 scale bytes per row, moved by
// buffer-to-LDS DMA (whole 128-byte lines) into a 2-slot ring, refilled once
// per super-stage with 15 MFMA k steps of latency to spare.
//
// k order inside a 64-element group: the MFMA takes 8 k values per lane from
// lane group g = lane / 32.  Lane g of a row takes the group's code bytes
// [16g, 16g + 16) -- k in [32g, 32g + 32) -- and feeds dword j of them to k
// step j; A and B use the same assignment, so every product pairs equal k.
// The two 16-element scale blocks a lane touches in a group are bytes 2g and
// 2g + 1 of the row's scale dword for that group.
//
// Schedule: each k step issues its 16 MFMAs with the dequantization of the
// next step (8 fragments, half a fragment per MFMA), the LDS reads of the
// next group and, once per super-stage, the ring refill pinned between them
// by sched_barrier, so VALU, LDS and DMA work runs in the matrix core's
// shadow.
//
// SWIGLU (the gate/up projection with the activation in its epilogue): the
// weight stack holds [gate; up] rows per expert (N = 2 I, I % 128 == 0), and
// output tile nt takes gate rows [128 nt, +128) as its columns 0..127 and the
// matching up rows [I + 128 nt, +128) as columns 128..255 (waves 0-1 and 2-3
// load the two halves from their own base rows).  The epilogue rounds each
// scaled gate and up value to bf16 -- the values the plain GEMM would store --
// and writes H = swiglu_pair(gate, up) for H columns [128 nt, +128): the
// gate/up output itself never reaches memory.  The "Cursor Composer 2 report
// deep dive", section 1, places the per-token scaling cost in the quantize
// and GEMM epilogue; here the activation joins it.
#include "device_common.h"
#include "gemm_common.h"
#include "gemm_pipe.h"

#include <stddef.h>

namespace bsq {

constexpr int FWD_BM = 256;
constexpr int FWD_BN = 256;
constexpr int FS_K = 256;                 // K elements per super-stage
constexpr int FS_CB = FS_K / 2;           // code bytes per row per super-stage
constexpr int FS_SB = FS_K / 16;          // scale bytes per row per super-stage
constexpr int FS_CODE_TILE = 256 * FS_CB; // one operand's codes (32 KB)
constexpr int FS_SCALE_TILE = 256 * FS_SB;
constexpr int FS_DMA = 24;                // DMA instructions per wave per super-stage

struct FwdSmem {
    uint8_t a[2][FS_CODE_TILE];
    uint8_t b[2][FS_CODE_TILE];
    uint8_t sa[2][FS_SCALE_TILE];
    uint8_t sb[2][FS_SCALE_TILE];
    float rs_a[FWD_BM];  // per-token decode scales of the tile's rows
    float rs_w[FWD_BN];  // per-output-channel decode scales of the tile's columns
};

struct FwdArgs {
    const uint8_t* a_codes; const uint8_t* a_bscale; const float* a_rscale;
    const uint8_t* w_codes; const uint8_t* w_bscale; const float* w_rscale;
    const int32_t* offsets; int E; int64_t N; int64_t K;
    void* y; int y_f32; int32_t* plan;
    int64_t ldo;  // SWIGLU: row pitch (elements) of the bf16 H output
};

// Raw LDS data of one 64-element group: 16 code bytes and one scale dword per
// 32-row fragment (A rows i = 0..3, B rows i = 0..3).
struct FwdRaw {
    u32x4 c[8];
    uint32_t s[8];
};

// Dequantized operands of one 16-element k step.
struct FwdOps {
    half8 f[8];
};

// Elements [4H, 4H + 4) of the eight codes in w, times s.
template <int H>
__device__ __forceinline__ void dequant_half(half8& out, uint32_t w, _Float16 s) {
    half2v ss;
    ss[0] = s;
    ss[1] = s;
    const half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2 * H) * ss;
    const half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2 * H + 1) * ss;
    out[4 * H] = p0[0];
    out[4 * H + 1] = p0[1];
    out[4 * H + 2] = p1[0];
    out[4 * H + 3] = p1[1];
}

template <bool OUT_F32, bool SWIGLU>
__global__ __launch_bounds__(256, 1) void k_gemm_fwd_nvfp4v(FwdArgs p) {
    static_assert(!(OUT_F32 && SWIGLU), "the activation output is bf16");
    extern __shared__ __align__(16) uint8_t smem_raw[];
    __shared__ int s_tile;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int lr = lane & 31, g = lane >> 5;
    const int xcd = blockIdx.x & 7;
    constexpr int esz = OUT_F32 ? 4 : 2;
    const uint32_t KB = (uint32_t)(p.K / 2), KS = (uint32_t)(p.K / 16);
    const int nsup = (int)((p.K + FS_K - 1) / FS_K);
    const int NT = (int)((p.N + FWD_BN - 1) / FWD_BN);
    const int total = p.plan[PLAN_TOTAL];
    int dq = 0;

    // 32-bit LDS byte addresses (DMA targets go through M0)
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem_raw));
    const uint32_t LA = lds0 + offsetof(FwdSmem, a), LB = lds0 + offsetof(FwdSmem, b);
    const uint32_t LSA = lds0 + offsetof(FwdSmem, sa), LSB = lds0 + offsetof(FwdSmem, sb);
    const uint32_t LRA = lds0 + offsetof(FwdSmem, rs_a), LRW = lds0 + offsetof(FwdSmem, rs_w);
    const __attribute__((address_space(3))) uint8_t* lds = (const __attribute__((address_space(3))) uint8_t*)(smem_raw);

    // Code DMA: instruction i (0..7) of this wave covers rows 64 * wave + 8i +
    // lane / 8; the lane fetches logical chunk (lane & 7) ^ swz8(row) into
    // slot lane & 7 (swz8(row) depends on lane / 8 and the parity of i).
    const int drow0 = 64 * wave + (lane >> 3);
    const uint32_t dch0 = (uint32_t)((lane & 7) ^ swz8(lane >> 3));
    const uint32_t dch1 = (uint32_t)((lane & 7) ^ swz8(8 + (lane >> 3)));
    // Scale DMA: instruction i (0..3) covers rows 64 * wave + 16i + lane / 4,
    // dword lane & 3 of the row's 16 scale bytes.
    const int srow0 = 64 * wave + (lane >> 2);
    const uint32_t sdw = (uint32_t)(lane & 3);
    // Fragment reads: lane (lr, g) of group gg takes logical chunk 2gg + g of
    // row lr of each 32-row group: slot (2gg + g) ^ swz8(lr).
    const uint32_t fr = (uint32_t)(lr * FS_CB + 16 * (g ^ swz8(lr)));
    const uint32_t fa = offsetof(FwdSmem, a) + (uint32_t)(wm * 128 * FS_CB);
    const uint32_t fb = offsetof(FwdSmem, b) + (uint32_t)(wn * 128 * FS_CB);
    const uint32_t fsa = offsetof(FwdSmem, sa) + (uint32_t)((wm * 128 + lr) * FS_SB);
    const uint32_t fsb = offsetof(FwdSmem, sb) + (uint32_t)((wn * 128 + lr) * FS_SB);

    // decode tables in LDS behind the staging buffers (when they fit)
    __attribute__((address_space(3))) int32_t* tab =
        (__attribute__((address_space(3))) int32_t*)(smem_raw + sizeof(FwdSmem));
    const bool tab_lds = p.E <= LDS_TABLE_MAX_E;
    if (tab_lds) fill_lds_tables(tab, p.plan, p.offsets, p.E);
    if (tid == 0) s_tile = claim_tile(p.plan, xcd, total, dq);
    __syncthreads();
    int tile = __builtin_amdgcn_readfirstlane(s_tile);  // uniform: keeps tile state in SGPRs

    for (;;) {
        if (tile < 0) break;
        // claim the next tile now; the atomic's latency hides behind this one
        int next_tile = 0;
        if (tid == 0) next_tile = claim_tile(p.plan, xcd, total, dq);

        const TileRef tr = decode_tile_any(tab_lds, tab, p.plan, p.offsets, p.E, tile, lane);
        const int e = tr.e;
        const int local = tr.local;
        const int64_t off0 = tr.off0;
        const int64_t off1 = tr.off1;
        int mt, nt;
        grouped_tile(local, (int)((off1 - off0 + FWD_BM - 1) / FWD_BM), NT, mt, nt);
        const int64_t m_base = uniform_i64(off0 + (int64_t)mt * FWD_BM);
        const int rows_a = __builtin_amdgcn_readfirstlane((int)min((int64_t)FWD_BM, off1 - m_base));
        const int64_t n_base = uniform_i64((int64_t)nt * FWD_BN);
        // first weight row of this wave's B rows (SWIGLU: waves 2-3 take the up half)
        const int64_t wrow = SWIGLU ? uniform_i64((int64_t)e * p.N + 128 * (int64_t)nt + (wave >= 2 ? p.N / 2 - 128 : 0))
                                    : uniform_i64((int64_t)e * p.N + n_base);
        const int rows_b = SWIGLU ? FWD_BN : __builtin_amdgcn_readfirstlane((int)min((int64_t)FWD_BN, p.N - n_base));
        const i32x4 dA = make_desc(uniform_ptr(p.a_codes + m_base * (int64_t)KB));
        const i32x4 dB = make_desc(uniform_ptr(p.w_codes + wrow * (int64_t)KB));
        const i32x4 dAs = make_desc(uniform_ptr(p.a_bscale + m_base * (int64_t)KS));
        const i32x4 dBs = make_desc(uniform_ptr(p.w_bscale + wrow * (int64_t)KS));

        const uint32_t vra = (uint32_t)drow0 * KB, vrb = (uint32_t)drow0 * KB;
        const uint32_t vsa = (uint32_t)srow0 * KS + 4 * sdw, vsb = vsa;

        // DMA of super-stage S into ring slot S % 2 in 12 parts of 2
        // instructions: parts 0..7 code rows (A and B of instruction i),
        // parts 8..11 scale rows.  Chunks past K read as zero.
        auto issue_part = [&](int S, int part) {
            const uint32_t q = (uint32_t)S & 1;
            if (part < 8) {
                const int i = part;
                const int row = drow0 + 8 * i;
                const uint32_t ko = (uint32_t)S * FS_CB + 16 * ((i & 1) ? dch1 : dch0);
                const bool okk = ko < KB;
                const uint32_t ldst = q * FS_CODE_TILE + 1024u * (uint32_t)(8 * wave + i);
                dma16(dA, (okk & (row < rows_a)) ? vra + (uint32_t)(8 * i) * KB + ko : OOB, LA + ldst);
                dma16(dB, (okk & (row < rows_b)) ? vrb + (uint32_t)(8 * i) * KB + ko : OOB, LB + ldst);
            } else {
                const int i = part - 8;
                const int row = srow0 + 16 * i;
                const uint32_t so = (uint32_t)S * FS_SB;
                const bool oks = so + 4 * sdw < KS;
                const uint32_t ldst = q * FS_SCALE_TILE + 256u * (uint32_t)(4 * wave + i);
                dma4(dAs, (oks & (row < rows_a)) ? vsa + (uint32_t)(16 * i) * KS + so : OOB, LSA + ldst);
                dma4(dBs, (oks & (row < rows_b)) ? vsb + (uint32_t)(16 * i) * KS + so : OOB, LSB + ldst);
            }
        };
        // LDS reads of group G (super-stage G / 4, group G % 4 of it); part f
        // (0..7) reads fragment f: A rows of group f, or B rows of group f - 4.
        auto read_part = [&](int G, FwdRaw& r, int f) {
            const uint32_t q = ((uint32_t)G >> 2) & 1, gg = (uint32_t)G & 3;
            const int i = f & 3;
            const uint32_t co = ((f < 4) ? fa : fb) + q * FS_CODE_TILE + (uint32_t)(32 * i * FS_CB);
            const uint32_t so = ((f < 4) ? fsa : fsb) + q * FS_SCALE_TILE + (uint32_t)(32 * i * FS_SB) + 4 * gg;
            r.c[f] = *(const __attribute__((address_space(3))) u32x4*)(lds + co + (fr ^ (32u * gg)));
            r.s[f] = *(const __attribute__((address_space(3))) uint32_t*)(lds + so);
        };
        // this lane's two block scales of fragment f in the group, as fp16
        auto conv_scale = [&](const FwdRaw& r, int f) -> half2v {
            return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.s[f] >> (16 * g), 1.0f, false);
        };

        float16v acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

        // Prologue: the tile's row and column scales, super-stages 0 and 1.
        {
            const int r = 64 * wave + lane;
            dma4(make_desc(uniform_ptr(p.a_rscale + m_base)), r < rows_a ? 4u * (uint32_t)r : OOB, LRA + 256u * wave);
            dma4(make_desc(uniform_ptr(p.w_rscale + wrow)), r < rows_b ? 4u * (uint32_t)r : OOB, LRW + 256u * wave);
        }
#pragma unroll
        for (int part = 0; part < 12; ++part) issue_part(0, part);
#pragma unroll
        for (int part = 0; part < 12; ++part) issue_part(1, part);
        wait_vmcnt<FS_DMA>();
        block_barrier();

        FwdRaw raw[2];
        FwdOps ops[2];
        half2v sh[8];
#pragma unroll
        for (int f = 0; f < 8; ++f) read_part(0, raw[0], f);
        wait_lgkmcnt0();
#pragma unroll
        for (int f = 0; f < 8; ++f) {
            sh[f] = conv_scale(raw[0], f);
            dequant_half<0>(ops[0].f[f], raw[0].c[f][0], sh[f][0]);
            dequant_half<1>(ops[0].f[f], raw[0].c[f][0], sh[f][0]);
        }

        // One super-stage: 4 groups x 4 k steps, fully unrolled so ring
        // slots, register buffers and schedule slots are compile-time.
        auto superstage = [&](int S) {
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                const int G = 4 * S + gg;
                FwdRaw& cur = raw[gg & 1];
                FwdRaw& nxt = raw[(gg + 1) & 1];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const FwdOps& o = ops[j & 1];
                    FwdOps& on = ops[(j + 1) & 1];
                    if (j == 0 && gg == 3) {
                        // super-stage S+1 has landed (the only DMA in flight)
                        // and every wave is done reading slot S % 2
                        wait_vmcnt<0>();
                        wait_lgkmcnt0();
                        block_barrier();
                    }
                    if (j == 3) wait_lgkmcnt0();  // next group's raw data
#pragma unroll
                    for (int k = 0; k < 16; ++k) {
                        const int i = k >> 2, jj = k & 3;
                        acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(o.f[i], o.f[4 + jj], acc[i][jj], 0, 0, 0);
                        // dequantize half a fragment of the next k step
                        const int f = k >> 1;
                        const uint32_t w = j < 3 ? cur.c[f][(j + 1) & 3] : nxt.c[f][0];
                        if (j == 3 && (k & 1) == 0) sh[f] = conv_scale(nxt, f);
                        const _Float16 sc = (j < 3 && (j + 1) >= 2) ? sh[f][1] : sh[f][0];
                        if (k & 1)
                            dequant_half<1>(on.f[f], w, sc);
                        else
                            dequant_half<0>(on.f[f], w, sc);
                        // LDS reads of the next group
                        if (j == 0 && k < 8) read_part(G + 1, nxt, k);
                        // refill of the slot just freed with super-stage S+2
                        if (gg == 3 && j == 1 && k < 12 && S + 2 < nsup) issue_part(S + 2, k);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
        };
        for (int S = 0; S < nsup; ++S) superstage(S);

        // drain every DMA of this tile before the ring is reused
        wait_vmcnt<0>();
        wait_lgkmcnt0();
        block_barrier();

        // Epilogue: the fp32 tile goes through the idle ring in two passes of
        // 128 rows, scaled by s_a[row] and then s_w[col] when it leaves as
        // whole rows in 16-byte stores (bf16 rounded to nearest even).  Lane
        // (lr, g) holds column wn*128 + 32j + lr of rows
        // wm*128 + 32i + 8(v/4) + 4g + v%4; the staging pitch of 1056 bytes
        // puts the two lane halves on disjoint banks.
        {
            constexpr uint32_t EP = 1056;
            // SWIGLU: the tile's H columns start at 128 nt of rows of p.ldo elements
            const __amdgpu_buffer_rsrc_t rc =
                make_rsrc(uniform_ptr(reinterpret_cast<char*>(p.y) +
                                      (SWIGLU ? (m_base * p.ldo + 128 * (int64_t)nt) * 2 : (m_base * p.N + n_base) * esz)),
                          0x7FFFFFFFu);
            const uint32_t ldcb = SWIGLU ? (uint32_t)p.ldo * 2u : (uint32_t)p.N * (uint32_t)esz;
            __attribute__((address_space(3))) uint8_t* st = (__attribute__((address_space(3))) uint8_t*)(smem_raw);
            const __attribute__((address_space(3))) float* rsa =
                (const __attribute__((address_space(3))) float*)(st + offsetof(FwdSmem, rs_a));
            const __attribute__((address_space(3))) float* rsw =
                (const __attribute__((address_space(3))) float*)(st + offsetof(FwdSmem, rs_w));
            const uint32_t wbase = (uint32_t)(wm * 64 + 4 * g) * EP + (uint32_t)(wn * 128 + lr) * 4u;
#pragma unroll
            for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
                for (int ii = 0; ii < 2; ++ii) {
                    const int i = 2 * pass + ii;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
#pragma unroll
                        for (int v = 0; v < 16; ++v) {
                            const uint32_t o = wbase + (uint32_t)(32 * ii + 8 * (v >> 2) + (v & 3)) * EP + 128u * j;
                            *(__attribute__((address_space(3))) float*)(st + o) = acc[i][j][v];
                        }
                }
                wait_lgkmcnt0();
                block_barrier();
                // staged row r (0..127) is tile row (r / 64) * 128 + 64 * pass + r % 64
                if constexpr (SWIGLU) {
#pragma unroll 2
                    for (int it = 0; it < 8; ++it) {
                        const int c = it * 256 + tid;  // 16 chunks of 8 H columns per row
                        const int r = c >> 4, cc = c & 15;
                        const int row = (r >> 6) * 128 + 64 * pass + (r & 63);
                        const uint32_t ro = (uint32_t)r * EP + 32u * cc;
                        const u32x4 g0 = *(const __attribute__((address_space(3))) u32x4*)(st + ro);
                        const u32x4 g1 = *(const __attribute__((address_space(3))) u32x4*)(st + ro + 16u);
                        const u32x4 u0 = *(const __attribute__((address_space(3))) u32x4*)(st + ro + 512u);
                        const u32x4 u1 = *(const __attribute__((address_space(3))) u32x4*)(st + ro + 528u);
                        const float sa = rsa[row];
                        float gv[8], uv[8];
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            gv[q] = (__uint_as_float(g0[q]) * sa) * rsw[8 * cc + q];
                            gv[4 + q] = (__uint_as_float(g1[q]) * sa) * rsw[8 * cc + 4 + q];
                            uv[q] = (__uint_as_float(u0[q]) * sa) * rsw[128 + 8 * cc + q];
                            uv[4 + q] = (__uint_as_float(u1[q]) * sa) * rsw[128 + 8 * cc + 4 + q];
                        }
                        u32x4 y;
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            y[q] = swiglu_pair(pack_bf16x2(gv[2 * q], gv[2 * q + 1]), pack_bf16x2(uv[2 * q], uv[2 * q + 1]));
                        __builtin_amdgcn_raw_buffer_store_b128(y, rc, row < rows_a ? (int)((uint32_t)row * ldcb + 16u * cc) : (int)OOB,
                                                               0, OUT_STORE_NT);
                    }
                } else if constexpr (OUT_F32) {
#pragma unroll 4
                    for (int it = 0; it < 32; ++it) {
                        const int c = it * 256 + tid;  // 64 chunks of 4 columns per row
                        const int r = c >> 6, cc = c & 63;
                        const int row = (r >> 6) * 128 + 64 * pass + (r & 63);
                        const u32x4 x = *(const __attribute__((address_space(3))) u32x4*)(st + (uint32_t)r * EP + 16u * cc);
                        const float sa = rsa[row];
                        u32x4 y;
#pragma unroll
                        for (int q = 0; q < 4; ++q) y[q] = __float_as_uint((__uint_as_float(x[q]) * sa) * rsw[4 * cc + q]);
                        const bool ok = (row < rows_a) & (4 * cc < rows_b);
                        __builtin_amdgcn_raw_buffer_store_b128(y, rc, ok ? (int)((uint32_t)row * ldcb + 16u * cc) : (int)OOB, 0,
                                                               OUT_STORE_NT);
                    }
                } else {
#pragma unroll 4
                    for (int it = 0; it < 16; ++it) {
                        const int c = it * 256 + tid;  // 32 chunks of 8 columns per row
                        const int r = c >> 5, cc = c & 31;
                        const int row = (r >> 6) * 128 + 64 * pass + (r & 63);
                        const u32x4 x0 = *(const __attribute__((address_space(3))) u32x4*)(st + (uint32_t)r * EP + 32u * cc);
                        const u32x4 x1 = *(const __attribute__((address_space(3))) u32x4*)(st + (uint32_t)r * EP + 32u * cc + 16u);
                        const float sa = rsa[row];
                        float v[8];
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            v[q] = (__uint_as_float(x0[q]) * sa) * rsw[8 * cc + q];
                            v[4 + q] = (__uint_as_float(x1[q]) * sa) * rsw[8 * cc + 4 + q];
                        }
                        u32x4 y;
#pragma unroll
                        for (int q = 0; q < 4; ++q) y[q] = pack_bf16x2(v[2 * q], v[2 * q + 1]);
                        const bool ok = (row < rows_a) & (8 * cc < rows_b);
                        __builtin_amdgcn_raw_buffer_store_b128(y, rc, ok ? (int)((uint32_t)row * ldcb + 16u * cc) : (int)OOB, 0,
                                                               OUT_STORE_NT);
                    }
                }
                // every wave's reads of this pass are done before the next
                // pass (or the next tile's DMA) overwrites the staging area;
                // the last barrier also publishes the next tile
                if (pass == 1 && tid == 0) s_tile = next_tile;
                wait_lgkmcnt0();
                block_barrier();
            }
        }
        tile = __builtin_amdgcn_readfirstlane(s_tile);
    }
}

size_t fwd_smem_bytes() { return sizeof(FwdSmem); }

hipError_t launch_gemm_fwd_nvfp4v(const uint8_t* a_codes, const uint8_t* a_bscale, const float* a_rscale,
                                  const uint8_t* w_codes, const uint8_t* w_bscale, const float* w_rscale,
                                  const int32_t* offsets, int E, int64_t m_total, int64_t N, int64_t K, void* y,
                                  int y_f32, int swiglu, int64_t ldo, int32_t* plan, int grid, hipStream_t s) {
    const int NT = (int)((N + FWD_BN - 1) / FWD_BN);
    hipError_t err = launch_plan(offsets, E, m_total, PLAN_RAGGED_ROWS, FWD_BM, NT, 1, plan, s);
    if (err != hipSuccess) return err;
    static bool attr_set = false;  // idempotent; racing writers set the same value
    if (!attr_set) {
        const void* ks[3] = {reinterpret_cast<const void*>(&k_gemm_fwd_nvfp4v<true, false>),
                             reinterpret_cast<const void*>(&k_gemm_fwd_nvfp4v<false, false>),
                             reinterpret_cast<const void*>(&k_gemm_fwd_nvfp4v<false, true>)};
        for (const void* k : ks) {
            err = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                      (int)(sizeof(FwdSmem) + lds_table_bytes(LDS_TABLE_MAX_E)));
            if (err != hipSuccess) return err;
        }
        attr_set = true;
    }
    FwdArgs p{a_codes, a_bscale, a_rscale, w_codes, w_bscale, w_rscale, offsets, E, N, K, y, y_f32, plan, ldo};
    const size_t lds = sizeof(FwdSmem) + lds_table_bytes(E);
    if (swiglu)
        hipLaunchKernelGGL((k_gemm_fwd_nvfp4v<false, true>), dim3(grid), dim3(256), lds, s, p);
    else if (y_f32)
        hipLaunchKernelGGL((k_gemm_fwd_nvfp4v<true, false>), dim3(grid), dim3(256), lds, s, p);
    else
        hipLaunchKernelGGL((k_gemm_fwd_nvfp4v<false, false>), dim3(grid), dim3(256), lds, s, p);
    return hipGetLastError();
}

}  // namespace bsq
