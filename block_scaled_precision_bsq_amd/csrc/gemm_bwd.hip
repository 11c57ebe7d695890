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
// Tiling: 256 x 256 outputs per workgroup.  k runs in 128-byte super-stages
// (two MFMA k steps) through a 2-slot LDS ring filled by buffer-to-LDS DMA
// (gemm_pipe.h).  One DMA instruction moves 8 rows x 128 bytes, i.e. whole
// 128-byte cache lines: fetching half lines (64-byte rows) caps the L2-to-CU
// stream near half of what full lines reach.
//
// Every operand mode runs in k_gemm_bwd_ws: 8 waves, two per SIMD, each
// owning 128 x 64 outputs (4 x 2 MFMA tiles).  The operand stream is bound by
// the latency of the CU's outstanding L2 requests, and a DMA instruction that
// finds the memory queue full stalls the wave that issues it.  Waves 4..7
// issue every DMA instruction and waves 0..3 none, so each SIMD always holds
// one wave whose MFMAs never wait behind a DMA issue, and the DMA waves place
// one MFMA between consecutive DMA instructions so that their own MFMAs run
// while they stall.  Two super-stages are in flight (see the kernel).
//
// Operand modes (OPS): MXFP8 (the backward GEMMs and the MXFP8 forward),
// plain bf16 operands (the bf16 baseline; a k step is 32 elements, 64 bytes,
// run as two bf16 MFMAs) and bf16 activations against packed NVFP4-variant
// weights (frozen expert storage): B fragments arrive as E2M1 codes plus E4M3
// block scales and are dequantized to bf16 in registers -- every E2M1 x E4M3
// product is exact in bf16 -- and the weight rows' fp32 scales are applied in
// the epilogue.
#include "device_common.h"
#include "gemm_common.h"
#include "gemm_pipe.h"

#include <type_traits>
#include <stddef.h>

namespace bsq {

constexpr int BWD_BM = 256;
constexpr int BWD_BN = 256;
constexpr int SS_BK = 128;                       // bytes of k per row per super-stage
constexpr int SS_TILE = PIPE_ROWS * SS_BK;       // one operand's super-stage (32 KB)

// One ring slot: codes of both operands and their scale bytes (one dword per
// (k block, row): block * 256 + row).  Slot-major so that a whole slot is
// one contiguous region: the epilogue stages its output through slot 1.
struct BwdSlot {
    uint8_t a[SS_TILE];
    uint8_t b[SS_TILE];
    uint32_t sa[4 * PIPE_ROWS];  // dgrad: one dword per (block, row); wgrad: packed bytes [block][row]
    uint8_t sb[4 * PIPE_ROWS];   // packed bytes [block][row]
};
struct BwdSmem {
    BwdSlot slot[2];
    float rs[256];  // packed-weight mode: fp32 scales of the tile's output columns
};
constexpr uint32_t SLOT_BYTES = sizeof(BwdSlot);
static_assert(SLOT_BYTES >= 128 * 512, "a bf16 epilogue pass stages 128 rows of 512 bytes in one slot");



// Per-tile DMA state: buffer descriptors, leading dimensions and the lane
// offsets at k = 0 (rows past the tile read as zero).
struct BwdTile {
    i32x4 dA, dB, dAs, dBs;
    const float* rs;  // packed-weight mode: fp32 scales of the tile's output columns
    uint32_t lda, ldb, ldas, ldbs, R;
    int rows_a, rows_b, nsteps;
    char* c;
    uint32_t ldcb;
    uint32_t vra, vrb;
    uint32_t vsa[4];  // dgrad A scale rows (one byte per lane)
};

// Operand modes of the tile loop.
constexpr int OPS_MX = 0;    // MXFP8 codes and E8M0 scales on both sides
constexpr int OPS_BF16 = 1;  // bf16 on both sides
constexpr int OPS_W4 = 2;    // bf16 A, NVFP4-variant B dequantized in registers

// Packed-weight B fragment of one k step: the lane's code dword for the
// step's first 16 elements sits in f[0], the one for the second 16 in f[4]
// (elements 8g.. of each half, row lr), and byte HF of s is the E4M3 scale
// of half HF.  Half HF becomes the four bf16 dwords f[4HF .. 4HF+3] the
// bf16 MFMA of that half takes: E2M1 pairs to fp32 (exact), times the block
// scale in fp32 (exact: at most 6 significant bits), high halves packed (the
// products are bf16 values, so nothing is rounded).
template <int HF>
__device__ __forceinline__ void w4_dequant_half(int8v& f, uint32_t s) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const uint32_t w = (uint32_t)f[4 * HF];
    const float sc = __builtin_amdgcn_cvt_f32_fp8((int)s, HF);
    // byte q of w holds elements 2q (low nibble) and 2q + 1
    const f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    const f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    const f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    const f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    auto pk = [&](const f32x2 v) {
        return (int)__builtin_amdgcn_perm(__float_as_uint(v[1] * sc), __float_as_uint(v[0] * sc), 0x07060302u);
    };
    const int o0 = pk(v0), o1 = pk(v1), o2 = pk(v2), o3 = pk(v3);
    f[4 * HF] = o0;
    f[4 * HF + 1] = o1;
    f[4 * HF + 2] = o2;
    f[4 * HF + 3] = o3;
}

// One 64-byte k step of fragments for output block (i, j): a single
// block-scaled fp8 MFMA (64 k), or for bf16 operands two bf16 MFMAs (16 k
// each) on the same 32 bytes per lane -- bytes [16g, +16) then [32+16g, +16),
// i.e. elements 8g.. and 16+8g.. of the 32 the step holds, the bf16 MFMA's
// k order for lane group g.
template <bool BF16>
__device__ __forceinline__ float16v mfma_step(const int8v& a, const int8v& b, int sa, int sb, float16v c) {
    if constexpr (BF16) {
        typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
        typedef int int4v __attribute__((ext_vector_type(4)));
        const int4v alo = {a[0], a[1], a[2], a[3]}, ahi = {a[4], a[5], a[6], a[7]};
        const int4v blo = {b[0], b[1], b[2], b[3]}, bhi = {b[4], b[5], b[6], b[7]};
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, alo), __builtin_bit_cast(bf16x8, blo),
                                                    c, 0, 0, 0);
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ahi),
                                                       __builtin_bit_cast(bf16x8, bhi), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
    }
}

// Number of DMA instructions in issue part `part` of a DMA wave's refills
// (super-stages 2 onwards; part 12 of packed weights loads only with the
// tile's second super-stage), and of LDS reads after MFMA m of a k step
// (refill order: B 0 after MFMA 3, A m - 4 after MFMA m >= 4, B 1 after
// MFMA 7; two 16-byte reads per fragment plus a scale read with MXFP8
// operands, three 4-byte reads per packed weight fragment).
template <bool WGRAD, int OPS>
constexpr int ws_part_dma(int part) {
    return OPS == OPS_W4     ? (part < 11 ? 1 : 0)
           : OPS == OPS_BF16 ? (part < 8 ? 2 : 0)
                             : (part < 8 ? 2 : (part < 12 ? (WGRAD ? 0 : 1) : (WGRAD ? 2 : 1)));
}
// RA / RB: LDS reads per A / B fragment
template <int RA, int RB>
constexpr int ws_reads_after(int m) { return m < 3 ? 0 : (m == 3 ? RB : (m < 7 ? RA : RA + RB)); }
// Pins NM MFMAs, then NV DMA instructions, then ND LDS reads, in order.
template <int NM, int NV, int ND>
__device__ __forceinline__ void ws_sched_step() {
    __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
    if constexpr (NV > 0) __builtin_amdgcn_sched_group_barrier(0x010, NV, 0);
    if constexpr (ND > 0) __builtin_amdgcn_sched_group_barrier(0x100, ND, 0);
}

// The tile loop: 8 waves (two per SIMD), each owning a 128 x 64 block of the
// 256 x 256 tile (4 x 2 MFMA tiles, 128 accumulators).  Waves 4..7 also issue
// every DMA instruction, so a DMA issue that stalls on the CU's full memory
// queue holds up only the matrix-core work of its own wave; waves 0..3 never
// enter that queue.  Two super-stages are in flight: the refill of a ring
// slot starts as soon as every wave holds the slot's data in registers
// (barrier X), and the wait for the next super-stage (barrier Y) comes after
// the first refill instructions.
template <bool OUT_F32, bool WGRAD, int OPS>
__global__ __launch_bounds__(512, 1) void k_gemm_bwd_ws(BwdArgs p) {
    constexpr bool BF16 = OPS != OPS_MX;  // bf16 A rows and bf16 MFMAs
    constexpr bool W4 = OPS == OPS_W4;
    static_assert(!(BF16 && WGRAD), "the bf16 modes run the row-ragged tiles only");
    // DMA instructions per DMA wave per super-stage, and per code part
    constexpr int SS_DMA = W4 ? 11 : (BF16 ? 16 : (WGRAD ? 18 : 21));
    constexpr int CP = W4 ? 1 : 2;
    constexpr int P1 = 3;                    // code parts issued before barrier Y
    extern __shared__ __align__(16) uint8_t smem_raw[];
    __shared__ int s_tile;

    const int tid0 = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid0 >> 6);
    const bool dwave = wave >= 4;
    const int dw = wave & 3;
    // When both waves of a SIMD are ready to issue an MFMA, the DMA wave's
    // goes first, so it returns sooner to its next DMA instruction.
    if (dwave) __builtin_amdgcn_s_setprio(1);
    const int wm = wave & 1, wn = wave >> 1;
    const int xcd = blockIdx.x & 7;
    constexpr int esz = OUT_F32 ? 4 : 2;
    const int total = p.plan[PLAN_TOTAL];
    int qdone = 0;  // claim queues found drained

    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem_raw));
    const __attribute__((address_space(3))) uint8_t* lds =
        (const __attribute__((address_space(3))) uint8_t*)(smem_raw);
    __attribute__((address_space(3))) int32_t* tab =
        (__attribute__((address_space(3))) int32_t*)(smem_raw + sizeof(BwdSmem));
    const bool tab_lds = p.E <= LDS_TABLE_MAX_E;
    if (tab_lds) fill_lds_tables(tab, p.plan, p.offsets, p.E);
    if (tid0 == 0) s_tile = claim_tile(p.plan, xcd, total, qdone);
    __syncthreads();
    int tile = __builtin_amdgcn_readfirstlane(s_tile);
    if (tile < 0) return;

    auto lane_of = [&]() {
        int t = tid0;
        asm volatile("" : "+v"(t));
        return t;
    };

    auto setup = [&](int tl) -> BwdTile {
        const int lane = lane_of() & 63;
        const TileRef tr = decode_tile_any(tab_lds, tab, p.plan, p.offsets, p.E, tl, lane);
        const int e = tr.e;
        const int64_t off0 = tr.off0, off1 = tr.off1;
        const uint8_t *a, *as, *b, *bs;
        int64_t lda, ldas, ldb, ldbs, R, ldc;
        int rows_a, rows_b;
        char* c;
        const float* rs = nullptr;
        if constexpr (!WGRAD) {
            const int KT = (int)((p.K + BWD_BN - 1) / BWD_BN);
            int mt, kt;
            grouped_tile(tr.local, (int)((off1 - off0 + BWD_BM - 1) / BWD_BM), KT, mt, kt);
            const int64_t m0 = off0 + (int64_t)mt * BWD_BM, k0 = (int64_t)kt * BWD_BN;
            const int64_t cw = 128 * ((int64_t)e + (int64_t)e * p.N / 128);
            a = p.dy_codes + m0 * p.N; as = p.dy_scale + m0;
            lda = p.N; ldas = p.m_total; rows_a = (int)min((int64_t)BWD_BM, off1 - m0);
            if constexpr (BF16) {
                // bf16 rows x [M][N]
                a = p.dy_codes + m0 * p.N * 2; as = p.dy_codes;
                lda = 2 * p.N; ldas = 0;
            }
            if constexpr (W4) {
                // expert e's packed weight rows [K] of N/2 code bytes and N/16
                // E4M3 scale bytes, and their fp32 scales
                b = p.wt_codes + ((int64_t)e * p.K + k0) * (p.N / 2);
                bs = p.wt_scale + ((int64_t)e * p.K + k0) * (p.N / 16);
                ldb = p.N / 2; ldbs = p.N / 16;
                rs = p.wt_rscale + (int64_t)e * p.K + k0;
            } else if constexpr (BF16) {
                // expert e's bf16 weight rows [K][N]
                b = p.wt_codes + ((int64_t)e * p.K + k0) * p.N * 2; bs = p.wt_codes;
                ldb = 2 * p.N; ldbs = 0;
            } else if (p.b_rows) {
                b = p.wt_codes + ((int64_t)e * p.K + k0) * p.N; bs = p.wt_scale + (int64_t)e * p.K + k0;
                ldb = p.N; ldbs = (int64_t)p.E * p.K;
            } else {
                b = p.wt_codes + k0 * p.Pw + cw; bs = p.wt_scale + (cw / 32) * p.K + k0;
                ldb = p.Pw; ldbs = p.K;
            }
            rows_b = (int)min((int64_t)BWD_BN, p.K - k0);
            R = BF16 ? 2 * p.N : p.N;  // bytes of k per A row
            c = reinterpret_cast<char*>(p.out) + (m0 * p.K + k0) * esz; ldc = p.K;
        } else {
            const int KT = (int)((p.K + BWD_BN - 1) / BWD_BN);
            int nt, kt;
            grouped_tile(tr.local, (int)((p.N + BWD_BM - 1) / BWD_BM), KT, nt, kt);
            const int64_t n0 = (int64_t)nt * BWD_BM, k0 = (int64_t)kt * BWD_BN;
            const int64_t c0 = 128 * ((int64_t)e + off0 / 128);
            a = p.dyt_codes + n0 * p.P + c0; as = p.dyt_scale + (c0 / 32) * p.N + n0;
            lda = p.P; ldas = p.N; rows_a = (int)min((int64_t)BWD_BM, p.N - n0);
            b = p.xt_codes + k0 * p.P + c0; bs = p.xt_scale + (c0 / 32) * p.K + k0;
            ldb = p.P; ldbs = p.K; rows_b = (int)min((int64_t)BWD_BN, p.K - k0);
            R = 32 * ((off1 - off0 + 31) / 32);
            c = reinterpret_cast<char*>(p.out) + (((int64_t)e * p.N + n0) * p.K + k0) * esz; ldc = p.K;
        }
        BwdTile ts;
        ts.dA = make_desc(uniform_ptr(a)); ts.dAs = make_desc(uniform_ptr(as));
        ts.dB = make_desc(uniform_ptr(b)); ts.dBs = make_desc(uniform_ptr(bs));
        ts.lda = __builtin_amdgcn_readfirstlane((uint32_t)lda);
        ts.ldb = __builtin_amdgcn_readfirstlane((uint32_t)ldb);
        ts.ldas = __builtin_amdgcn_readfirstlane((uint32_t)ldas);
        ts.ldbs = __builtin_amdgcn_readfirstlane((uint32_t)ldbs);
        ts.R = __builtin_amdgcn_readfirstlane((uint32_t)R);
        ts.rows_a = __builtin_amdgcn_readfirstlane(rows_a);
        ts.rows_b = __builtin_amdgcn_readfirstlane(rows_b);
        ts.nsteps = (int)((ts.R + 63) / 64);
        ts.c = uniform_ptr(c);
        ts.rs = rs;
        ts.ldcb = __builtin_amdgcn_readfirstlane((uint32_t)(ldc * esz));
        const int drow0 = 64 * dw + (lane >> 3);
        ts.vra = (uint32_t)drow0 * ts.lda;
        ts.vrb = (uint32_t)drow0 * ts.ldb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ins = 4 * dw + i;
            const int row = 64 * (ins & 3) + lane;
            const uint32_t kb = (uint32_t)(ins >> 2);
            ts.vsa[i] = row < ts.rows_a ? kb * ts.ldas + row : OOB;
        }
        return ts;
    };

    // DMA of super-stage S into slot S % 2 by DMA wave dw (0..3), in 13
    // parts so they can sit between MFMAs: parts 0..7 move code rows (A and
    // B of instruction i; A only with packed weights); with MXFP8, parts
    // 8..11 the dgrad A scales and part 12 the packed scale blocks (block dw
    // of the super-stage, 256 rows); with packed weights, parts 8..10 the B
    // rows and scales and part 12 their fp32 scales.
    auto issue_part = [&](const BwdTile& ts, int S, auto PC) {
        constexpr int part = decltype(PC)::value;
        if constexpr (BF16 && !W4 && part >= 8) return;  // bf16 operands carry no scales
        if constexpr (W4 && part >= 11 && part != 12) return;
        const int lane = lane_of() & 63;
        const uint32_t q = (uint32_t)S & 1;
        const uint32_t kbase = (uint32_t)S * SS_BK;
        if constexpr (W4 && part >= 8) {
            // Packed weight rows: 32 code bytes and 4 E4M3 scale bytes per row
            // per super-stage (64 elements).  Parts 8 and 9: code instruction
            // c = 2 * dw + part - 8 covers rows 32c + lane / 2, 16-byte half
            // lane & 1, landing as [row][32 bytes] with the halves swapped on
            // bit 2 of the row (fewer bank conflicts in the reads).  Part 10:
            // the scale dwords of rows 64 * dw + lane.  Part 12, with the
            // tile's second super-stage only: the rows' fp32 scales into rs.
            if constexpr (part < 10) {
                const int c = 2 * dw + (part - 8);
                const int row = 32 * c + (lane >> 1);
                const uint32_t bo = (uint32_t)S * 32u + 16u * (uint32_t)((lane & 1) ^ ((row >> 2) & 1));
                const bool ok = (row < ts.rows_b) & (bo < ts.ldb);
                dma16(ts.dB, ok ? (uint32_t)row * ts.ldb + bo : OOB,
                      lds_at<offsetof(BwdSlot, b)>(lds0 + q * SLOT_BYTES + 1024u * (uint32_t)c));
            } else if constexpr (part == 10) {
                const int row = 64 * dw + lane;
                const uint32_t so = (uint32_t)S * 4u;
                const bool ok = (row < ts.rows_b) & (so < ts.ldbs);
                dma4(ts.dBs, ok ? (uint32_t)row * ts.ldbs + so : OOB,
                     lds_at<offsetof(BwdSlot, sb)>(lds0 + q * SLOT_BYTES + 256u * (uint32_t)dw));
            } else {
                if (S == 1) {
                    const int row = 64 * dw + lane;
                    dma4(make_desc(uniform_ptr(ts.rs)), row < ts.rows_b ? 4u * (uint32_t)row : OOB,
                         lds_at<offsetof(BwdSmem, rs)>(lds0 + 256u * (uint32_t)dw));
                }
            }
            return;
        }
        if constexpr (part < 8) {
            constexpr int i = part;
            const int row = 64 * dw + 8 * i + (lane >> 3);
            const uint32_t ch = (uint32_t)((lane & 7) ^ swz8(8 * (i & 1) + (lane >> 3)));
            const bool okk = kbase + 16 * ch < ts.R;
            const uint32_t ko = kbase + 16 * ch;
            const uint32_t base = lds0 + q * SLOT_BYTES + 8192u * (uint32_t)dw;
            dma16(ts.dA, (okk & (row < ts.rows_a)) ? ts.vra + (uint32_t)(8 * i) * ts.lda + ko : OOB,
                  lds_at<offsetof(BwdSlot, a) + 1024u * i>(base));
            if constexpr (!W4)
                dma16(ts.dB, (okk & (row < ts.rows_b)) ? ts.vrb + (uint32_t)(8 * i) * ts.ldb + ko : OOB,
                      lds_at<offsetof(BwdSlot, b) + 1024u * i>(base));
        } else if constexpr (part < 12) {
            if constexpr (!WGRAD) {
                constexpr int i = part - 8;
                const int ins = 4 * dw + i;
                const uint32_t blk = 4 * (uint32_t)S + (uint32_t)(ins >> 2);
                const bool oks = blk * 32 < ts.R;
                const uint32_t sblk = 4 * (uint32_t)S;
                const uint32_t base = lds0 + q * SLOT_BYTES + 1024u * (uint32_t)dw;
                dma1(ts.dAs, oks ? ts.vsa[i] + sblk * ts.ldas : OOB, lds_at<offsetof(BwdSlot, sa) + 256u * i>(base));
            }
        } else {
            const uint32_t blk = 4 * (uint32_t)S + (uint32_t)dw;
            const bool oks = blk * 32 < ts.R;
            // one dword (4 rows) per lane: the whole wave takes part, so the
            // part has no branch for the compiler to sink matrix-core work past
            const uint32_t rb = 4u * (uint32_t)lane;
            const uint32_t base = lds0 + q * SLOT_BYTES + 256u * (uint32_t)dw;
            if constexpr (WGRAD)
                dma4(ts.dAs, (oks & (rb < (uint32_t)ts.rows_a)) ? blk * ts.ldas + rb : OOB,
                     lds_at<offsetof(BwdSlot, sa)>(base));
            dma4(ts.dBs, (oks & (rb < (uint32_t)ts.rows_b)) ? blk * ts.ldbs + rb : OOB,
                 lds_at<offsetof(BwdSlot, sb)>(base));
        }
    };
    auto issue_dyn = [&](const BwdTile& ts, int S, int part) {
        switch (part) {
            case 0: issue_part(ts, S, IC<0>{}); break;
            case 1: issue_part(ts, S, IC<1>{}); break;
            case 2: issue_part(ts, S, IC<2>{}); break;
            case 3: issue_part(ts, S, IC<3>{}); break;
            case 4: issue_part(ts, S, IC<4>{}); break;
            case 5: issue_part(ts, S, IC<5>{}); break;
            case 6: issue_part(ts, S, IC<6>{}); break;
            case 7: issue_part(ts, S, IC<7>{}); break;
            case 8: issue_part(ts, S, IC<8>{}); break;
            case 9: issue_part(ts, S, IC<9>{}); break;
            case 10: issue_part(ts, S, IC<10>{}); break;
            case 11: issue_part(ts, S, IC<11>{}); break;
            case 12: issue_part(ts, S, IC<12>{}); break;
            default: break;
        }
    };
    auto issue = [&](const BwdTile& ts, int S) {
#pragma unroll
        for (int part = 0; part < 13; ++part) issue_dyn(ts, S, part);
    };

    if (dwave) {
        const BwdTile first = setup(tile);
        issue(first, 0);
        issue(first, 1);
    }

    for (;;) {
        const BwdTile cur = setup(tile);
        const int tid = lane_of();
        const int lane = tid & 63;
        const int lr = lane & 31, g = lane >> 5;
        const uint32_t fr = (uint32_t)(lr * SS_BK + 16 * (g ^ swz8(lr)));
        const uint32_t fa = offsetof(BwdSlot, a) + (uint32_t)(wm * 128 * SS_BK);
        const uint32_t fb = offsetof(BwdSlot, b) + (uint32_t)(wn * 64 * SS_BK);
        constexpr uint32_t ESA = WGRAD ? 1u : 4u;
        const uint32_t fsa = offsetof(BwdSlot, sa) + ESA * (uint32_t)(256 * g + wm * 128 + lr);
        const uint32_t fsb = offsetof(BwdSlot, sb) + (uint32_t)(256 * g + wn * 64 + lr);

        // the next tile's claim: its atomic's round trip overlaps this tile
        PendingClaim pclaim{0, -1};
        if (tid == 0) pclaim = claim_start(p.plan, xcd, qdone);

        // Fragments of k step t: row group grp (32 rows) of A (isB false) or
        // B, logical chunks 4h + g and 4h + g + 2 of the row, and the scale of
        // k block 2h + g.
        auto rd = [&](int t, auto ISB, int grp, int8v& v, int& sc) {
            constexpr bool isB = decltype(ISB)::value;
            const uint32_t q = ((uint32_t)t >> 1) & 1, h = (uint32_t)t & 1;
            if constexpr (W4 && isB) {
                // packed weight row: the code dwords of the step's two halves
                // (elements 8g.. of each 16) into v[0] and v[4], the row's
                // scale bytes of the step into sc; dequantized later
                const uint32_t row = (uint32_t)(wn * 64 + 32 * grp + lr);
                const uint32_t co = q * SLOT_BYTES + (uint32_t)offsetof(BwdSlot, b) + row * 32u +
                                    16u * (h ^ ((row >> 2) & 1u)) + 4u * (uint32_t)g;
                v[0] = *(const __attribute__((address_space(3))) int*)(lds + co);
                v[4] = *(const __attribute__((address_space(3))) int*)(lds + co + 8u);
                sc = (int)(*(const __attribute__((address_space(3))) uint32_t*)(
                               lds + q * SLOT_BYTES + (uint32_t)offsetof(BwdSlot, sb) + row * 4u) >>
                           (16u * h));
                return;
            }
            const uint32_t es = isB ? 1u : ESA;
            const uint32_t so = q * SLOT_BYTES + (isB ? fsb : fsa) + es * (h * 512u + 32u * (uint32_t)grp);
            const uint32_t o = q * SLOT_BYTES + (isB ? fb : fa) + (uint32_t)(32 * grp * SS_BK);
            const u32x4 x0 = *(const __attribute__((address_space(3))) u32x4*)(lds + o + (fr ^ (64u * h)));
            const u32x4 x1 = *(const __attribute__((address_space(3))) u32x4*)(lds + o + (fr ^ (64u * h + 32u)));
            sc = 0;
            if constexpr (!BF16)
                sc = (es == 4u) ? *(const __attribute__((address_space(3))) int*)(lds + so)
                                : (int)*(const __attribute__((address_space(3))) uint8_t*)(lds + so);
            v = int8v{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
        };

        float16v acc[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

        // One set of fragments, refilled as it frees: MFMA m of a k step is
        // (i, j) = (m % 4, m / 4), so B fragment 0 is free after MFMA 3, A
        // fragment i after MFMA 4 + i and B fragment 1 after MFMA 7; each
        // read has at least three MFMAs of lead before its first use.
        int8v A[4], B[2];
        int SA[4], SB[2];
        auto mm = [&](int m) {
            const int i = m & 3, j = m >> 2;
            acc[i][j] = mfma_step<BF16>(A[i], B[j], SA[i], SB[j], acc[i][j]);
        };
        // packed weights: B fragment j's half HF from its raw code dword
        auto dq = [&](int j, int hf) {
            if constexpr (W4) {
                if (hf)
                    w4_dequant_half<1>(B[j], (uint32_t)SB[j]);
                else
                    w4_dequant_half<0>(B[j], (uint32_t)SB[j]);
            }
        };
        auto refill = [&](int t, int m) {
            if (m == 3) rd(t + 1, IC<1>{}, 0, B[0], SB[0]);
            if (m >= 4) rd(t + 1, IC<0>{}, m - 4, A[m - 4], SA[m - 4]);
            if (m == 7) rd(t + 1, IC<1>{}, 1, B[1], SB[1]);
            // packed weights: B fragment 0 (read after MFMA 3) is dequantized
            // after MFMA 6, fragment 1 (read after MFMA 7 of the previous
            // step) after MFMAs 1 and 2, before its first use at MFMA 4
            if (m == 1) dq(1, 0);
            if (m == 2) dq(1, 1);
            if (m == 6) { dq(0, 0); dq(0, 1); }
        };
        // The k loop runs as two straight-line versions: DMA waves (DW) and
        // the others.  k step t even: DMA waves issue the rest of the
        // super-stage begun in the previous odd step (MORE; none at t = 0).
        auto kloop = [&](auto DWC) {
            constexpr bool DW = decltype(DWC)::value != 0;
            auto step_even = [&](int t, auto MOREC) {
                constexpr bool MORE = DW && decltype(MOREC)::value != 0;
                const int S = (t >> 1) + 1;
                auto body = [&](auto MC) {
                    constexpr int m = decltype(MC)::value;
                    mm(m);
                    if constexpr (MORE && P1 + 4 + m < 13) issue_part(cur, S, IC<P1 + 4 + m>{});
                    refill(t, m);
                    if constexpr (!MORE) __builtin_amdgcn_sched_barrier(0);
                };
                body(IC<0>{}); body(IC<1>{}); body(IC<2>{}); body(IC<3>{});
                body(IC<4>{}); body(IC<5>{}); body(IC<6>{}); body(IC<7>{});
                if constexpr (MORE) {
                    // the DMA wave's order: each MFMA, then its refill part, then its reads
                    auto pin = [&](auto MC) {
                        constexpr int m = decltype(MC)::value;
                        constexpr int part = P1 + 4 + m;
                        ws_sched_step<BF16 ? 2 : 1, part < 13 ? ws_part_dma<WGRAD, OPS>(part) : 0,
                                      ws_reads_after<BF16 ? 2 : 3, (BF16 && !W4) ? 2 : 3>(m)>();
                    };
                    pin(IC<0>{}); pin(IC<1>{}); pin(IC<2>{}); pin(IC<3>{});
                    pin(IC<4>{}); pin(IC<5>{}); pin(IC<6>{}); pin(IC<7>{});
                    __builtin_amdgcn_sched_barrier(0);
                }
            };
            // k step t odd: barrier X (every wave holds super-stage t / 2 in
            // registers) lets the refill of its slot with super-stage t / 2 + 2
            // begin; after four MFMAs barrier Y (super-stage t / 2 + 1 has
            // landed) opens the reads of t + 1.
            auto step_odd = [&](int t) {
                wait_lgkmcnt0();
                block_barrier();
                const int S = (t >> 1) + 2;
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    mm(m);
                    if constexpr (DW) {
                        if (m < P1) issue_dyn(cur, S, m);
                        if (m == 3) wait_vmcnt<CP * P1>();
                    }
                    if (m == 3) block_barrier();
                    if constexpr (DW)
                        if (m >= 4) issue_dyn(cur, S, P1 + m - 4);
                    refill(t, m);
                    __builtin_amdgcn_sched_barrier(0);
                }
            };
            if constexpr (DW) wait_vmcnt<SS_DMA>();  // super-stage 0 has landed; 1 may fly
            block_barrier();
#pragma unroll
            for (int i = 0; i < 4; ++i) rd(0, IC<0>{}, i, A[i], SA[i]);
            rd(0, IC<1>{}, 0, B[0], SB[0]);
            rd(0, IC<1>{}, 1, B[1], SB[1]);
            if constexpr (W4) {
                // the rolling scheme dequantizes B fragment 1 during step 0
                wait_lgkmcnt0();
                dq(0, 0);
                dq(0, 1);
            }
            int t = 0;
            if (cur.nsteps >= 2) {
                step_even(0, IC<0>{});
                step_odd(1);
                for (t = 2; t + 1 < cur.nsteps; t += 2) {
                    step_even(t, IC<1>{});
                    step_odd(t + 1);
                }
            }
            if (t < cur.nsteps) {
                wait_lgkmcnt0();
                // packed weights: B fragment 1 of the last step (the entry
                // points take k % 64 == 0 for the bf16 modes, so their step
                // count is even and this tail runs for MXFP8 operands only)
                dq(1, 0);
                dq(1, 1);
#pragma unroll
                for (int m = 0; m < 8; ++m) mm(m);
            }
        };
        if (dwave)
            kloop(IC<1>{});
        else
            kloop(IC<0>{});
        if (dwave) wait_vmcnt<0>();
        if (tid == 0) s_tile = claim_finish(p.plan, xcd, total, qdone, pclaim);
        wait_lgkmcnt0();
        block_barrier();
        tile = __builtin_amdgcn_readfirstlane(s_tile);

        const int tnext = tile >= 0 ? tile : 0;

        {
            const __amdgpu_buffer_rsrc_t rc = make_rsrc(cur.c, 0x7FFFFFFFu);
            __attribute__((address_space(3))) uint8_t* st =
                (__attribute__((address_space(3))) uint8_t*)(smem_raw) + SLOT_BYTES;
            // packed weights: the fp32 scale of column wn*64 + 32j + lr
            float rsj[2] = {1.0f, 1.0f};
            if constexpr (W4) {
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    rsj[j] = *(const __attribute__((address_space(3))) float*)(
                        lds + offsetof(BwdSmem, rs) + 4u * (uint32_t)(wn * 64 + 32 * j + lr));
            }
            if constexpr (OUT_F32) {
                // f32: four passes of 64 rows (row group `pass` of both row
                // halves); staged row r = wm * 32 + row % 32 keeps 1024 bytes,
                // and its 128-byte segments swap in pairs when bit 2 of r is
                // set, which puts the two lane halves (rows 4 apart) on
                // disjoint banks
#pragma unroll
                for (int pass = 0; pass < 4; ++pass) {
#pragma unroll
                    for (int j = 0; j < 2; ++j)
#pragma unroll
                        for (int v = 0; v < 16; ++v) {
                            const uint32_t r = (uint32_t)(wm * 32 + 4 * g + 8 * (v >> 2) + (v & 3));
                            const uint32_t cb = 4u * (uint32_t)(wn * 64 + 32 * j + lr);
                            *(__attribute__((address_space(3))) float*)(st + r * 1024u + (cb ^ (128u * (uint32_t)g))) =
                                W4 ? acc[pass][j][v] * rsj[j] : acc[pass][j][v];
                        }
                    wait_lgkmcnt0();
                    block_barrier();
#pragma unroll
                    for (int it = 0; it < 8; ++it) {
                        const int c = it * 512 + tid;
                        const int r = c >> 6, cc = c & 63;
                        const int row = (r >> 5) * 128 + 32 * pass + (r & 31);
                        const uint32_t sw = 128u * (uint32_t)((r >> 2) & 1);
                        const u32x4 x = *(const __attribute__((address_space(3))) u32x4*)(st + (uint32_t)r * 1024u + ((16u * cc) ^ sw));
                        const bool ok = (row < cur.rows_a) & (4 * cc < cur.rows_b);
                        __builtin_amdgcn_raw_buffer_store_b128(x, rc, ok ? (int)((uint32_t)row * cur.ldcb + 16u * cc) : (int)OOB, 0,
                                                               OUT_STORE_NT);
                    }
                    wait_lgkmcnt0();
                    block_barrier();
                }
            } else {
                // bf16: two passes of 128 rows (pass p: every wave's row
                // groups 2p and 2p+1).  A lane rounds each pair of vertically
                // adjacent values (v, v+1 with v even) into one dword, low half
                // the even row, so LDS holds rows in pairs: pair P (64 per
                // pass) keeps 1024 bytes, columns 8k..8k+3 of every 8-column
                // chunk k in its first 512 bytes and columns 8k+4..8k+7 in the
                // second.  The 64-byte units of each half are XOR-permuted by
                // s = half + 2 * bit 1 of P, so the four 64-byte pieces one
                // write instruction touches (two halves, pairs 2 apart) fall
                // on different banks, while a read of 16 consecutive bytes per
                // lane stays conflict-free.  Each read item (pair, chunk) then
                // leaves as two 16-byte row stores.
#pragma unroll
                for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
                    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
                        for (int j = 0; j < 2; ++j)
#pragma unroll
                            for (int v = 0; v < 16; v += 2) {
                                const int P = wm * 32 + 16 * ii + 4 * (v >> 2) + 2 * g + ((v >> 1) & 1);
                                const int col = wn * 64 + 32 * j + lr;
                                const int k = col >> 3, w = col & 7, half = w >> 2;
                                const uint32_t sx = 64u * (uint32_t)((half + 2 * ((P >> 1) & 1)) & 3);
                                const uint32_t o = (uint32_t)P * 1024u + 512u * (uint32_t)half +
                                                   ((16u * (uint32_t)k + 4u * (uint32_t)(w & 3)) ^ sx);
                                *(__attribute__((address_space(3))) uint32_t*)(st + o) =
                                    W4 ? pack_bf16x2(acc[2 * pass + ii][j][v] * rsj[j], acc[2 * pass + ii][j][v + 1] * rsj[j])
                                       : pack_bf16x2(acc[2 * pass + ii][j][v], acc[2 * pass + ii][j][v + 1]);
                            }
                    wait_lgkmcnt0();
                    block_barrier();
#pragma unroll
                    for (int it = 0; it < 4; ++it) {
                        const int item = it * 512 + tid;
                        const int P = item >> 5, k = item & 31;
                        const uint32_t sa0 = 64u * (uint32_t)(2 * ((P >> 1) & 1));
                        const uint32_t po = (uint32_t)P * 1024u;
                        const u32x4 x0 = *(const __attribute__((address_space(3))) u32x4*)(st + po + ((16u * k) ^ sa0));
                        const u32x4 x1 = *(const __attribute__((address_space(3))) u32x4*)(st + po + 512u + ((16u * k) ^ (sa0 + 64u)));
                        u32x4 ev, od;
                        ev[0] = __builtin_amdgcn_perm(x0[1], x0[0], 0x05040100u);
                        ev[1] = __builtin_amdgcn_perm(x0[3], x0[2], 0x05040100u);
                        ev[2] = __builtin_amdgcn_perm(x1[1], x1[0], 0x05040100u);
                        ev[3] = __builtin_amdgcn_perm(x1[3], x1[2], 0x05040100u);
                        od[0] = __builtin_amdgcn_perm(x0[1], x0[0], 0x07060302u);
                        od[1] = __builtin_amdgcn_perm(x0[3], x0[2], 0x07060302u);
                        od[2] = __builtin_amdgcn_perm(x1[1], x1[0], 0x07060302u);
                        od[3] = __builtin_amdgcn_perm(x1[3], x1[2], 0x07060302u);
                        const int row = (P >> 5) * 128 + 32 * (2 * pass + ((P >> 4) & 1)) + 2 * (P & 15);
                        const bool okc = 8 * k < cur.rows_b;
                        const uint32_t go = (uint32_t)row * cur.ldcb + 16u * (uint32_t)k;
                        __builtin_amdgcn_raw_buffer_store_b128(ev, rc, (okc & (row < cur.rows_a)) ? (int)go : (int)OOB, 0, OUT_STORE_NT);
                        __builtin_amdgcn_raw_buffer_store_b128(od, rc, (okc & (row + 1 < cur.rows_a)) ? (int)(go + cur.ldcb) : (int)OOB, 0, OUT_STORE_NT);
                    }
                    wait_lgkmcnt0();
                    block_barrier();
                }
            }
        }
        if (tile < 0) break;
        // The next tile's first two super-stages go out only now: issued
        // before the epilogue, their loads sat in the CU's memory queue ahead
        // of the output stores and held the epilogue up.
        if (dwave) {
            const BwdTile nx = setup(tnext);
            issue(nx, 0);
            issue(nx, 1);
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
    const int lds_max = (int)(sizeof(BwdSmem) + lds_table_bytes(LDS_TABLE_MAX_E));
    if (!attr_set) {
        const void* ks[8] = {reinterpret_cast<const void*>(&k_gemm_bwd_ws<true, true, OPS_MX>),
                             reinterpret_cast<const void*>(&k_gemm_bwd_ws<true, false, OPS_MX>),
                             reinterpret_cast<const void*>(&k_gemm_bwd_ws<false, true, OPS_MX>),
                             reinterpret_cast<const void*>(&k_gemm_bwd_ws<false, false, OPS_MX>),
                             reinterpret_cast<const void*>(&k_gemm_bwd_ws<true, false, OPS_BF16>),
                             reinterpret_cast<const void*>(&k_gemm_bwd_ws<false, false, OPS_BF16>),
                             reinterpret_cast<const void*>(&k_gemm_bwd_ws<true, false, OPS_W4>),
                             reinterpret_cast<const void*>(&k_gemm_bwd_ws<false, false, OPS_W4>)};
        for (const void* k : ks) {
            err = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, lds_max);
            if (err != hipSuccess) return err;
        }
        attr_set = true;
    }
    const size_t lds = sizeof(BwdSmem) + lds_table_bytes(args.E);
#define BSQ_GEMM_LAUNCH(F32, WG, OPS) \
    hipLaunchKernelGGL((k_gemm_bwd_ws<F32, WG, OPS>), dim3(grid), dim3(512), lds, s, args)
    if (args.bf16 || args.w4) {
        if (args.wgrad || (args.bf16 && args.w4)) return hipErrorInvalidValue;  // row-ragged tiles only
        if (args.w4) {
            if (args.out_f32)
                BSQ_GEMM_LAUNCH(true, false, OPS_W4);
            else
                BSQ_GEMM_LAUNCH(false, false, OPS_W4);
        } else if (args.out_f32) {
            BSQ_GEMM_LAUNCH(true, false, OPS_BF16);
        } else {
            BSQ_GEMM_LAUNCH(false, false, OPS_BF16);
        }
    } else if (args.out_f32) {
        if (args.wgrad)
            BSQ_GEMM_LAUNCH(true, true, OPS_MX);
        else
            BSQ_GEMM_LAUNCH(true, false, OPS_MX);
    } else {
        if (args.wgrad)
            BSQ_GEMM_LAUNCH(false, true, OPS_MX);
        else
            BSQ_GEMM_LAUNCH(false, false, OPS_MX);
    }
#undef BSQ_GEMM_LAUNCH
    return hipGetLastError();
}

}  // namespace bsq
