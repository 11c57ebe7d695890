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
// MXFP8 operands run in k_gemm_bwd_ws: 8 waves, two per SIMD, each owning
// 128 x 64 outputs (4 x 2 MFMA tiles).  The operand stream is bound by the
// latency of the CU's outstanding L2 requests, and a DMA instruction that
// finds the memory queue full stalls the wave that issues it.  Waves 4..7
// issue every DMA instruction and waves 0..3 none, so each SIMD always holds
// one wave whose MFMAs never wait behind a DMA issue, and the DMA waves place
// one MFMA between consecutive DMA instructions so that their own MFMAs run
// while they stall.  Two super-stages are in flight (see the kernel).
//
// bf16 A operands run in k_gemm_bf16a: 4 waves, 2 x 2, 128 x 128 each (4 x 4
// MFMA tiles, fp32 accumulators in AGPRs), fragments double-buffered in
// registers per 64-byte k step (the MFMAs of step t run while step t+1 is read
// from LDS), and a ring slot refilled as soon as both of its steps sit in
// registers.  Two operand modes (OPS): plain bf16 operands (the bf16
// baseline) and bf16 activations against packed NVFP4-variant weights (frozen
// expert storage): B fragments arrive as E2M1 codes plus E4M3 block scales and
// are dequantized to bf16 in registers -- every E2M1 x E4M3 product is exact
// in bf16 -- and the weight rows' fp32 scales are applied in the epilogue.
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
// one contiguous region -- the epilogue stages its output through slot 1
// while the next tile's first super-stage lands in slot 0.
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

// One 64-byte k step of fragments for output block (i, j): a single
// block-scaled fp8 MFMA (64 k), or for bf16 operands two bf16 MFMAs (16 k
// each) on the same 32 bytes per lane -- bytes [16g, +16) then [32+16g, +16),
// i.e. elements 8g.. and 16+8g.. of the 32 the step holds, the bf16 MFMA's
// k order for lane group g.
// Operand modes of the bf16-A tile loop.
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

// Tile loop over bf16 A rows (a k step is 32 elements, 64 bytes; the
// reduction length is counted in A bytes) against bf16 B rows (OPS_BF16) or
// packed NVFP4-variant B rows (OPS_W4), on row-ragged tiles.
template <bool OUT_F32, int OPS>
__global__ __launch_bounds__(256, 1) void k_gemm_bf16a(BwdArgs p) {
    static_assert(OPS == OPS_BF16 || OPS == OPS_W4, "MXFP8 operands run in k_gemm_bwd_ws");
    constexpr bool W4 = OPS == OPS_W4;
    // DMA instructions per wave per super-stage: 16 code rows (8 of A and 8
    // of B); packed weights take 8 of A, 2 code instructions (32 bytes of 256
    // rows) and one scale instruction (4 bytes of 256 rows).
    constexpr int SS_DMA = W4 ? 11 : 16;
    extern __shared__ __align__(16) uint8_t smem_raw[];
    __shared__ int s_tile;

    const int tid0 = threadIdx.x;
    // wave-uniform by construction; readfirstlane lets the compiler keep
    // everything derived from it in SGPRs
    const int wave = __builtin_amdgcn_readfirstlane(tid0 >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int xcd = blockIdx.x & 7;
    constexpr int esz = OUT_F32 ? 4 : 2;
    const int total = p.plan[PLAN_TOTAL];
    int dq = 0;

    // 32-bit LDS byte address of the ring (DMA targets go through M0)
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem_raw));
    const __attribute__((address_space(3))) uint8_t* lds =
        (const __attribute__((address_space(3))) uint8_t*)(smem_raw);

    // decode tables in LDS behind the ring (when they fit)
    __attribute__((address_space(3))) int32_t* tab =
        (__attribute__((address_space(3))) int32_t*)(smem_raw + sizeof(BwdSmem));
    const bool tab_lds = p.E <= LDS_TABLE_MAX_E;
    if (tab_lds) fill_lds_tables(tab, p.plan, p.offsets, p.E);
    if (tid0 == 0) s_tile = claim_tile(p.plan, xcd, total, dq);
    __syncthreads();
    int tile = __builtin_amdgcn_readfirstlane(s_tile);  // uniform: keeps tile state in SGPRs
    if (tile < 0) return;

    // Lane constants come from an opaque copy of the thread index, rebuilt
    // per tile: hoisted out of the tile loop they would stay live through
    // every phase and push the kernel into spills.
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
        // C[m][k] = sum_n X[m][n] W_e[k][n] over the rows m of expert e
        const int KT = (int)((p.K + BWD_BN - 1) / BWD_BN);
        int mt, kt;
        grouped_tile(tr.local, (int)((off1 - off0 + BWD_BM - 1) / BWD_BM), KT, mt, kt);
        const int64_t m0 = off0 + (int64_t)mt * BWD_BM, k0 = (int64_t)kt * BWD_BN;
        // bf16 rows x [M][N]
        const uint8_t* a = p.dy_codes + m0 * p.N * 2;
        const int64_t lda = 2 * p.N;
        const int rows_a = (int)min((int64_t)BWD_BM, off1 - m0);
        const uint8_t *b, *bs;
        int64_t ldb, ldbs;
        const float* rs = nullptr;
        if constexpr (W4) {
            // expert e's packed weight rows [K] of N/2 code bytes and N/16
            // E4M3 scale bytes, and their fp32 scales
            b = p.wt_codes + ((int64_t)e * p.K + k0) * (p.N / 2);
            bs = p.wt_scale + ((int64_t)e * p.K + k0) * (p.N / 16);
            ldb = p.N / 2; ldbs = p.N / 16;
            rs = p.wt_rscale + (int64_t)e * p.K + k0;
        } else {
            // expert e's bf16 weight rows [K][N]
            b = p.wt_codes + ((int64_t)e * p.K + k0) * p.N * 2; bs = p.wt_codes;
            ldb = 2 * p.N; ldbs = 0;
        }
        const int rows_b = (int)min((int64_t)BWD_BN, p.K - k0);
        const int64_t R = 2 * p.N;  // bytes of k per row
        char* c = reinterpret_cast<char*>(p.out) + (m0 * p.K + k0) * esz;
        const int64_t ldc = p.K;
        BwdTile ts;
        ts.dA = make_desc(uniform_ptr(a)); ts.dAs = ts.dA;
        ts.dB = make_desc(uniform_ptr(b)); ts.dBs = make_desc(uniform_ptr(bs));
        ts.lda = __builtin_amdgcn_readfirstlane((uint32_t)lda);
        ts.ldb = __builtin_amdgcn_readfirstlane((uint32_t)ldb);
        ts.ldas = 0;
        ts.ldbs = __builtin_amdgcn_readfirstlane((uint32_t)ldbs);
        ts.R = __builtin_amdgcn_readfirstlane((uint32_t)R);
        ts.rows_a = __builtin_amdgcn_readfirstlane(rows_a);
        ts.rows_b = __builtin_amdgcn_readfirstlane(rows_b);
        ts.nsteps = (int)((ts.R + 63) / 64);  // 64-byte MFMA k steps
        ts.c = uniform_ptr(c);
        ts.rs = rs;
        ts.ldcb = __builtin_amdgcn_readfirstlane((uint32_t)(ldc * esz));
        // code instruction i (0..7) of this wave covers rows 64 * wave + 8i + lane / 8
        const int drow0 = 64 * wave + (lane >> 3);
        ts.vra = (uint32_t)drow0 * ts.lda;
        ts.vrb = (uint32_t)drow0 * ts.ldb;
        return ts;
    };

    // DMA of super-stage S of tile ts into ring slot S % 2 (SS_DMA
    // instructions per wave), in 13 parts so they can sit between MFMAs:
    // parts 0..7 move code rows (A and B of instruction i; with packed
    // weights A only), parts 8..12 the packed weight rows and scales.
    // The lane fetches logical chunk (lane & 7) ^ swz8(row) into slot
    // lane & 7; swz8(row) depends on lane / 8 and the parity of i.  A 16-byte
    // chunk or a 32-element scale block past R reads as zero.
    auto issue_part = [&](const BwdTile& ts, int S, auto PC) {
        constexpr int part = decltype(PC)::value;
        if constexpr (!W4 && part >= 8) return;  // bf16 operands carry no scales
        if constexpr (W4 && part >= 11 && part != 12) return;
        const int lane = lane_of() & 63;
        const uint32_t q = (uint32_t)S & 1;
        const uint32_t kbase = (uint32_t)S * SS_BK;
        if constexpr (W4 && part >= 8) {
            // Packed weight rows: 32 code bytes and 4 E4M3 scale bytes per row
            // per super-stage (64 elements).  Parts 8 and 9: code instruction
            // c = 2 * wave + part - 8 covers rows 32c + lane / 2, 16-byte half
            // lane & 1, landing as [row][32 bytes].  Part 10: the scale dwords
            // of rows 64 * wave + lane.  Part 12, with the tile's second
            // super-stage only: the rows' fp32 scales into rs (read by the
            // epilogue, after which the next tile's second super-stage is
            // issued).
            if constexpr (part < 10) {
                // LDS half lane & 1 of a row holds code half (lane & 1) ^ bit 2
                // of the row, which halves the bank conflicts of the reads
                const int c = 2 * wave + (part - 8);
                const int row = 32 * c + (lane >> 1);
                const uint32_t bo = (uint32_t)S * 32u + 16u * (uint32_t)((lane & 1) ^ ((row >> 2) & 1));
                const bool ok = (row < ts.rows_b) & (bo < ts.ldb);
                dma16(ts.dB, ok ? (uint32_t)row * ts.ldb + bo : OOB,
                      lds_at<offsetof(BwdSlot, b)>(lds0 + q * SLOT_BYTES + 1024u * (uint32_t)c));
            } else if constexpr (part == 10) {
                const int row = 64 * wave + lane;
                const uint32_t so = (uint32_t)S * 4u;
                const bool ok = (row < ts.rows_b) & (so < ts.ldbs);
                dma4(ts.dBs, ok ? (uint32_t)row * ts.ldbs + so : OOB,
                     lds_at<offsetof(BwdSlot, sb)>(lds0 + q * SLOT_BYTES + 256u * (uint32_t)wave));
            } else {
                if (S == 1) {
                    const int row = 64 * wave + lane;
                    dma4(make_desc(uniform_ptr(ts.rs)), row < ts.rows_b ? 4u * (uint32_t)row : OOB,
                         lds_at<offsetof(BwdSmem, rs)>(lds0 + 256u * (uint32_t)wave));
                }
            }
            return;
        }
        if constexpr (part < 8) {
            constexpr int i = part;
            const int row = 64 * wave + 8 * i + (lane >> 3);
            const uint32_t ch = (uint32_t)((lane & 7) ^ swz8(8 * (i & 1) + (lane >> 3)));
            const bool okk = kbase + 16 * ch < ts.R;
            const uint32_t ko = kbase + 16 * ch;
            const uint32_t base = lds0 + q * SLOT_BYTES + 8192u * (uint32_t)wave;
            dma16(ts.dA, (okk & (row < ts.rows_a)) ? ts.vra + (uint32_t)(8 * i) * ts.lda + ko : OOB,
                  lds_at<offsetof(BwdSlot, a) + 1024u * i>(base));
            if constexpr (!W4)
                dma16(ts.dB, (okk & (row < ts.rows_b)) ? ts.vrb + (uint32_t)(8 * i) * ts.ldb + ko : OOB,
                      lds_at<offsetof(BwdSlot, b) + 1024u * i>(base));
        }
    };
    auto issue = [&](const BwdTile& ts, int S) {
        issue_part(ts, S, IC<0>{}); issue_part(ts, S, IC<1>{}); issue_part(ts, S, IC<2>{});
        issue_part(ts, S, IC<3>{}); issue_part(ts, S, IC<4>{}); issue_part(ts, S, IC<5>{});
        issue_part(ts, S, IC<6>{}); issue_part(ts, S, IC<7>{}); issue_part(ts, S, IC<8>{});
        issue_part(ts, S, IC<9>{}); issue_part(ts, S, IC<10>{}); issue_part(ts, S, IC<11>{});
        issue_part(ts, S, IC<12>{});
    };

    {
        const BwdTile first = setup(tile);
        issue(first, 0);
        issue(first, 1);
    }

    for (;;) {
        // this tile's state, rebuilt from the LDS decode tables (not carried
        // across iterations, which would force it through memory)
        const BwdTile cur = setup(tile);
        const int tid = lane_of();
        const int lane = tid & 63;
        const int lr = lane & 31, g = lane >> 5;
        // Fragment read geometry: lane (lr, g) of k step h reads chunks 4h + g
        // and 4h + g + 2 of row lr of each 32-row group; swz8(row) = swz8(lr),
        // and (4h + g + 2d) ^ swz8 = (g ^ swz8) ^ (4h + 2d).
        const uint32_t fr = (uint32_t)(lr * SS_BK + 16 * (g ^ swz8(lr)));
        const uint32_t fa = offsetof(BwdSlot, a) + (uint32_t)(wm * 128 * SS_BK);
        const uint32_t fb = offsetof(BwdSlot, b) + (uint32_t)(wn * 128 * SS_BK);

        // claim the next tile now; the atomic's latency hides behind this one
        int next_tile = 0;
        if (tid == 0) next_tile = claim_tile(p.plan, xcd, total, dq);

        // Fragments of k step t (ring slot (t / 2) % 2, half h = t % 2): lane
        // (row, g) takes logical chunks 4h + g and 4h + g + 2 of its row (the
        // bf16 MFMAs' k order).  Part 2i reads the A rows of group i, part
        // 2i+1 the B rows.
        auto read_part = [&](int t, BwdFrag& f, int part) {
            const uint32_t q = ((uint32_t)t >> 1) & 1, h = (uint32_t)t & 1;
            if constexpr (W4) {
                // parts 0..3: packed B fragments (two code dwords and the
                // row's scale dword, dequantized later), parts 4..7: A
                if (part < 4) {
                    const uint32_t row = (uint32_t)(wn * 128 + 32 * part + lr);
                    const uint32_t co = q * SLOT_BYTES + (uint32_t)offsetof(BwdSlot, b) + row * 32u +
                                        16u * (h ^ ((row >> 2) & 1u)) + 4u * (uint32_t)g;
                    f.b[part][0] = *(const __attribute__((address_space(3))) int*)(lds + co);
                    f.b[part][4] = *(const __attribute__((address_space(3))) int*)(lds + co + 8u);
                    f.sb[part] = (int)(*(const __attribute__((address_space(3))) uint32_t*)(
                                           lds + q * SLOT_BYTES + (uint32_t)offsetof(BwdSlot, sb) + row * 4u) >>
                                       (16u * h));
                    return;
                }
                part = 2 * (part - 4);
            }
            const int i = part >> 1;
            const uint32_t o = q * SLOT_BYTES + ((part & 1) ? fb : fa) + (uint32_t)(32 * i * SS_BK);
            const u32x4 x0 = *(const __attribute__((address_space(3))) u32x4*)(lds + o + (fr ^ (64u * h)));
            const u32x4 x1 = *(const __attribute__((address_space(3))) u32x4*)(lds + o + (fr ^ (64u * h + 32u)));
            const int8v v = int8v{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
            if (part & 1) f.b[i] = v; else f.a[i] = v;
        };
        auto read = [&](int t, BwdFrag& f) {
#pragma unroll
            for (int part = 0; part < 8; ++part) read_part(t, f, part);
        };
        // packed B: half-fragment hf2 (0..7) of the fragments read by read_part
        auto dequant = [&](BwdFrag& f, int hf2) {
            if constexpr (W4) {
                if (hf2 & 1)
                    w4_dequant_half<1>(f.b[hf2 >> 1], (uint32_t)f.sb[hf2 >> 1]);
                else
                    w4_dequant_half<0>(f.b[hf2 >> 1], (uint32_t)f.sb[hf2 >> 1]);
            }
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
                    acc[i][j] = mfma_step<true>(f.a[i], f.b[j], f.sa[i], f.sb[j], acc[i][j]);
        };
        // k step t (fragments in cur) with t even: both halves of its
        // super-stage are in LDS; the MFMAs of t run with the reads of t+1.
        auto step_even = [&](int t, const BwdFrag& cf, BwdFrag& nf) {
            wait_lgkmcnt0();
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const int i = k >> 2, j = k & 3;
                acc[i][j] = mfma_step<true>(cf.a[i], cf.b[j], cf.sa[i], cf.sb[j], acc[i][j]);
                if (k >= 2 && k < 10) read_part(t + 1, nf, k - 2);
                if (W4 && k >= 8) dequant(nf, k - 8);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        // k step t odd: wait until super-stage t/2 + 1 has landed (the only
        // DMA in flight) and every wave holds both halves of super-stage t/2
        // in registers, then refill its slot with super-stage t/2 + 2 while
        // the MFMAs of t run, and read t+1.
        auto step_odd = [&](int t, const BwdFrag& cf, BwdFrag& nf) {
            wait_vmcnt<0>();
            wait_lgkmcnt0();
            block_barrier();
            const int S = (t >> 1) + 2;
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const int i = k >> 2, j = k & 3;
                acc[i][j] = mfma_step<true>(cf.a[i], cf.b[j], cf.sa[i], cf.sb[j], acc[i][j]);
                switch (k) {
                    case 0: issue_part(cur, S, IC<0>{}); break;
                    case 1: issue_part(cur, S, IC<1>{}); break;
                    case 2: issue_part(cur, S, IC<2>{}); break;
                    case 3: issue_part(cur, S, IC<3>{}); break;
                    case 4: issue_part(cur, S, IC<4>{}); break;
                    case 5: issue_part(cur, S, IC<5>{}); break;
                    case 6: issue_part(cur, S, IC<6>{}); break;
                    case 7: issue_part(cur, S, IC<7>{}); break;
                    case 8: issue_part(cur, S, IC<8>{}); break;
                    case 9: issue_part(cur, S, IC<9>{}); break;
                    case 10: issue_part(cur, S, IC<10>{}); break;
                    case 11: issue_part(cur, S, IC<11>{}); break;
                    case 12: issue_part(cur, S, IC<12>{}); break;
                    default: break;
                }
                if (k >= 4 && k < 12) read_part(t + 1, nf, k - 4);
                if (W4 && k >= 8) dequant(nf, k - 8);
                __builtin_amdgcn_sched_barrier(0);
            }
        };

        // super-stages 0 and 1 are in flight (issued by the previous tile or
        // the kernel prologue); wait for 0
        wait_vmcnt<SS_DMA>();  // super-stage 1 may still fly
        block_barrier();
        BwdFrag X, Y;
        read(0, X);
        if constexpr (W4) {
            wait_lgkmcnt0();
#pragma unroll
            for (int hf2 = 0; hf2 < 8; ++hf2) dequant(X, hf2);
        }
        int t = 0;
        for (; t + 1 < cur.nsteps; t += 2) {
            step_even(t, X, Y);
            step_odd(t + 1, Y, X);
        }
        if (t < cur.nsteps) {
            wait_lgkmcnt0();
            mma(X);
        }
        // drain every DMA of this tile and publish the next tile
        wait_vmcnt<0>();
        if (tid == 0) s_tile = next_tile;
        wait_lgkmcnt0();
        block_barrier();
        tile = __builtin_amdgcn_readfirstlane(s_tile);

        // The next tile's first super-stage goes to slot 0 now, so its
        // latency hides behind the epilogue, which stages through slot 1.
        const int tnext = tile >= 0 ? tile : 0;  // a valid index for the unused case
        const BwdTile nxt = setup(tnext);
        if (tile >= 0) issue(nxt, 0);

        // Epilogue through slot 1.  Lane (lr, g) holds column wn*128 + 32j + lr
        // of rows wm*128 + 32i + 8(v/4) + 4g + v%4.  Stores outside a partial
        // tile get an out-of-range offset.
        {
            const __amdgpu_buffer_rsrc_t rc = make_rsrc(cur.c, 0x7FFFFFFFu);
            __attribute__((address_space(3))) uint8_t* st =
                (__attribute__((address_space(3))) uint8_t*)(smem_raw) + SLOT_BYTES;
            // packed weights: the fp32 scale of column wn*128 + 32j + lr
            float rsj[4] = {1.0f, 1.0f, 1.0f, 1.0f};
            if constexpr (W4) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    rsj[j] = *(const __attribute__((address_space(3))) float*)(
                        lds + offsetof(BwdSmem, rs) + 4u * (uint32_t)(wn * 128 + 32 * j + lr));
            }
            if constexpr (OUT_F32) {
                // f32: four passes of 64 rows (pass i: every wave's row group
                // i), staged row r = wm * 32 + (row % 32) keeps 1024 bytes; its
                // 128-byte segments are swapped in pairs when bit 2 of r is
                // set, which puts the two lane halves (rows 4 apart) on
                // disjoint banks.
                const uint32_t wrow = (uint32_t)(wm * 32 + 4 * g) * 1024u + (uint32_t)(wn * 512 + 4 * lr);
                const uint32_t wev = wrow + 128u * (uint32_t)g;        // column tiles j = 0, 2
                const uint32_t wod = wrow + 128u * (uint32_t)(1 - g);  // column tiles j = 1, 3
#pragma unroll
                for (int pass = 0; pass < 4; ++pass) {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
#pragma unroll
                        for (int v = 0; v < 16; ++v) {
                            const uint32_t o = ((j & 1) ? wod : wev) + 256u * (j >> 1) +
                                               (uint32_t)(8 * (v >> 2) + (v & 3)) * 1024u;
                            *(__attribute__((address_space(3))) float*)(st + o) =
                                W4 ? acc[pass][j][v] * rsj[j] : acc[pass][j][v];
                        }
                    wait_lgkmcnt0();
                    block_barrier();
#pragma unroll
                    for (int it = 0; it < 16; ++it) {
                        const int c = it * 256 + tid;          // 64 chunks of 4 columns per row
                        const int r = c >> 6, cc = c & 63;
                        const int row = (r >> 5) * 128 + 32 * pass + (r & 31);
                        const uint32_t sw = 128u * (uint32_t)((r >> 2) & 1);
                        const u32x4 x = *(const __attribute__((address_space(3))) u32x4*)(st + (uint32_t)r * 1024u + ((16u * cc) ^ sw));
                        const bool ok = (row < cur.rows_a) & (4 * cc < cur.rows_b);
                        __builtin_amdgcn_raw_buffer_store_b128(x, rc, ok ? (int)((uint32_t)row * cur.ldcb + 16u * cc) : (int)OOB, 0,
                                                               OUT_STORE_NT);
                    }
                    // every wave's reads of this pass are done before the next
                    // pass (or the next tile's second super-stage) overwrites slot 1
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
                        for (int j = 0; j < 4; ++j)
#pragma unroll
                            for (int v = 0; v < 16; v += 2) {
                                const int P = wm * 32 + 16 * ii + 4 * (v >> 2) + 2 * g + ((v >> 1) & 1);
                                const int col = wn * 128 + 32 * j + lr;
                                const int k = col >> 3, w = col & 7, half = w >> 2;
                                const uint32_t sx = 64u * (uint32_t)((half + 2 * ((P >> 1) & 1)) & 3);
                                const uint32_t o = (uint32_t)P * 1024u + 512u * (uint32_t)half +
                                                   ((16u * (uint32_t)k + 4u * (uint32_t)(w & 3)) ^ sx);
                                *(__attribute__((address_space(3))) uint32_t*)(st + o) =
                                    W4 ? pack_bf16x2(acc[2 * pass + ii][j][v] * rsj[j],
                                                     acc[2 * pass + ii][j][v + 1] * rsj[j])
                                       : pack_bf16x2(acc[2 * pass + ii][j][v], acc[2 * pass + ii][j][v + 1]);
                            }
                    wait_lgkmcnt0();
                    block_barrier();
#pragma unroll
                    for (int it = 0; it < 8; ++it) {
                        const int item = it * 256 + tid;
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
                    // every wave's reads of this pass are done before the next
                    // pass (or the next tile's second super-stage) overwrites slot 1
                    wait_lgkmcnt0();
                    block_barrier();
                }
            }
        }
        if (tile < 0) break;
        issue(nxt, 1);
    }
    // outstanding output stores complete before the wave ends
}

// MXFP8 tile loop with the operand stream split from the matrix-core issue:
// 8 waves (two per SIMD), each owning a 128 x 64 block of the 256 x 256 tile
// (4 x 2 MFMA tiles, 128 accumulators).  Waves 4..7 also issue every DMA
// instruction, exactly as the four waves of the single-issuer loop do, so a
// DMA issue that stalls on the CU's full memory queue holds up only the
// matrix-core work of its own wave; waves 0..3 never enter that queue.
// Two super-stages are in flight: the refill of a ring slot starts as soon as
// every wave holds the slot's data in registers (barrier X), and the wait for
// the next super-stage (barrier Y) comes after the first refill instructions.
// Number of DMA instructions in issue part `part` of a DMA wave, and of LDS
// reads after MFMA m of a k step (refill order: B 0 after MFMA 3, A m - 4
// after MFMA m >= 4, B 1 after MFMA 7; three reads per fragment).
template <bool WGRAD>
constexpr int ws_part_dma(int part) { return part < 8 ? 2 : (part < 12 ? (WGRAD ? 0 : 1) : (WGRAD ? 2 : 1)); }
constexpr int ws_reads_after(int m) { return m < 3 ? 0 : (m < 7 ? 3 : 6); }
// Pins one MFMA, then NV DMA instructions, then ND LDS reads, in order.
template <int NV, int ND>
__device__ __forceinline__ void ws_sched_step() {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (NV > 0) __builtin_amdgcn_sched_group_barrier(0x010, NV, 0);
    if constexpr (ND > 0) __builtin_amdgcn_sched_group_barrier(0x100, ND, 0);
}

template <bool OUT_F32, bool WGRAD>
__global__ __launch_bounds__(512, 1) void k_gemm_bwd_ws(BwdArgs p) {
    constexpr int SS_DMA = WGRAD ? 18 : 21;  // DMA instructions per DMA wave per super-stage
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
    int dq = 0;

    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem_raw));
    const __attribute__((address_space(3))) uint8_t* lds =
        (const __attribute__((address_space(3))) uint8_t*)(smem_raw);
    __attribute__((address_space(3))) int32_t* tab =
        (__attribute__((address_space(3))) int32_t*)(smem_raw + sizeof(BwdSmem));
    const bool tab_lds = p.E <= LDS_TABLE_MAX_E;
    if (tab_lds) fill_lds_tables(tab, p.plan, p.offsets, p.E);
    if (tid0 == 0) s_tile = claim_tile(p.plan, xcd, total, dq);
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
        if constexpr (!WGRAD) {
            const int KT = (int)((p.K + BWD_BN - 1) / BWD_BN);
            int mt, kt;
            grouped_tile(tr.local, (int)((off1 - off0 + BWD_BM - 1) / BWD_BM), KT, mt, kt);
            const int64_t m0 = off0 + (int64_t)mt * BWD_BM, k0 = (int64_t)kt * BWD_BN;
            const int64_t cw = 128 * ((int64_t)e + (int64_t)e * p.N / 128);
            a = p.dy_codes + m0 * p.N; as = p.dy_scale + m0;
            lda = p.N; ldas = p.m_total; rows_a = (int)min((int64_t)BWD_BM, off1 - m0);
            if (p.b_rows) {
                b = p.wt_codes + ((int64_t)e * p.K + k0) * p.N; bs = p.wt_scale + (int64_t)e * p.K + k0;
                ldb = p.N; ldbs = (int64_t)p.E * p.K;
            } else {
                b = p.wt_codes + k0 * p.Pw + cw; bs = p.wt_scale + (cw / 32) * p.K + k0;
                ldb = p.Pw; ldbs = p.K;
            }
            rows_b = (int)min((int64_t)BWD_BN, p.K - k0);
            R = p.N;
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
        ts.rs = nullptr;
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

    // DMA of super-stage S into slot S % 2 by DMA wave dw, in 13 parts (the
    // same split of the stage over four issuing waves as the single-issuer
    // loop): parts 0..7 code rows of A and B, 8..11 dgrad A scales, 12 the
    // packed scale blocks (block dw of the super-stage, 256 rows).
    auto issue_part = [&](const BwdTile& ts, int S, auto PC) {
        constexpr int part = decltype(PC)::value;
        const int lane = lane_of() & 63;
        const uint32_t q = (uint32_t)S & 1;
        const uint32_t kbase = (uint32_t)S * SS_BK;
        if constexpr (part < 8) {
            constexpr int i = part;
            const int row = 64 * dw + 8 * i + (lane >> 3);
            const uint32_t ch = (uint32_t)((lane & 7) ^ swz8(8 * (i & 1) + (lane >> 3)));
            const bool okk = kbase + 16 * ch < ts.R;
            const uint32_t ko = kbase + 16 * ch;
            const uint32_t base = lds0 + q * SLOT_BYTES + 8192u * (uint32_t)dw;
            dma16(ts.dA, (okk & (row < ts.rows_a)) ? ts.vra + (uint32_t)(8 * i) * ts.lda + ko : OOB,
                  lds_at<offsetof(BwdSlot, a) + 1024u * i>(base));
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

        int next_tile = 0;
        if (tid == 0) next_tile = claim_tile(p.plan, xcd, total, dq);

        // Fragments of k step t: row group grp (32 rows) of A (isB false) or
        // B, logical chunks 4h + g and 4h + g + 2 of the row, and the scale of
        // k block 2h + g.
        auto rd = [&](int t, auto ISB, int grp, int8v& v, int& sc) {
            constexpr bool isB = decltype(ISB)::value;
            const uint32_t q = ((uint32_t)t >> 1) & 1, h = (uint32_t)t & 1;
            const uint32_t es = isB ? 1u : ESA;
            const uint32_t so = q * SLOT_BYTES + (isB ? fsb : fsa) + es * (h * 512u + 32u * (uint32_t)grp);
            const uint32_t o = q * SLOT_BYTES + (isB ? fb : fa) + (uint32_t)(32 * grp * SS_BK);
            const u32x4 x0 = *(const __attribute__((address_space(3))) u32x4*)(lds + o + (fr ^ (64u * h)));
            const u32x4 x1 = *(const __attribute__((address_space(3))) u32x4*)(lds + o + (fr ^ (64u * h + 32u)));
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
            acc[i][j] = mfma_step<false>(A[i], B[j], SA[i], SB[j], acc[i][j]);
        };
        auto refill = [&](int t, int m) {
            if (m == 3) rd(t + 1, IC<1>{}, 0, B[0], SB[0]);
            if (m >= 4) rd(t + 1, IC<0>{}, m - 4, A[m - 4], SA[m - 4]);
            if (m == 7) rd(t + 1, IC<1>{}, 1, B[1], SB[1]);
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
                        ws_sched_step<part < 13 ? ws_part_dma<WGRAD>(part) : 0, ws_reads_after(m)>();
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
                        if (m == 3) wait_vmcnt<2 * P1>();
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
#pragma unroll
                for (int m = 0; m < 8; ++m) mm(m);
            }
        };
        if (dwave)
            kloop(IC<1>{});
        else
            kloop(IC<0>{});
        if (dwave) wait_vmcnt<0>();
        if (tid == 0) s_tile = next_tile;
        wait_lgkmcnt0();
        block_barrier();
        tile = __builtin_amdgcn_readfirstlane(s_tile);

        const int tnext = tile >= 0 ? tile : 0;
        if (dwave && tile >= 0) issue(setup(tnext), 0);

        {
            const __amdgpu_buffer_rsrc_t rc = make_rsrc(cur.c, 0x7FFFFFFFu);
            __attribute__((address_space(3))) uint8_t* st =
                (__attribute__((address_space(3))) uint8_t*)(smem_raw) + SLOT_BYTES;
            if constexpr (OUT_F32) {
                // four passes of 64 rows (row group `pass` of both row halves);
                // staged row r = wm * 32 + row % 32 keeps 1024 bytes, and its
                // 128-byte segments swap in pairs when bit 2 of r is set
#pragma unroll
                for (int pass = 0; pass < 4; ++pass) {
#pragma unroll
                    for (int j = 0; j < 2; ++j)
#pragma unroll
                        for (int v = 0; v < 16; ++v) {
                            const uint32_t r = (uint32_t)(wm * 32 + 4 * g + 8 * (v >> 2) + (v & 3));
                            const uint32_t cb = 4u * (uint32_t)(wn * 64 + 32 * j + lr);
                            *(__attribute__((address_space(3))) float*)(st + r * 1024u + (cb ^ (128u * (uint32_t)g))) =
                                acc[pass][j][v];
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
                // two passes of 128 rows in row pairs, laid out as in the
                // single-issuer loop
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
                                    pack_bf16x2(acc[2 * pass + ii][j][v], acc[2 * pass + ii][j][v + 1]);
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
        if (dwave) issue(setup(tnext), 1);
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
        const void* ks[8] = {reinterpret_cast<const void*>(&k_gemm_bwd_ws<true, true>),
                             reinterpret_cast<const void*>(&k_gemm_bwd_ws<true, false>),
                             reinterpret_cast<const void*>(&k_gemm_bwd_ws<false, true>),
                             reinterpret_cast<const void*>(&k_gemm_bwd_ws<false, false>),
                             reinterpret_cast<const void*>(&k_gemm_bf16a<true, OPS_BF16>),
                             reinterpret_cast<const void*>(&k_gemm_bf16a<false, OPS_BF16>),
                             reinterpret_cast<const void*>(&k_gemm_bf16a<true, OPS_W4>),
                             reinterpret_cast<const void*>(&k_gemm_bf16a<false, OPS_W4>)};
        for (const void* k : ks) {
            err = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, lds_max);
            if (err != hipSuccess) return err;
        }
        attr_set = true;
    }
    const size_t lds = sizeof(BwdSmem) + lds_table_bytes(args.E);
#define BSQ_MX_LAUNCH(F32, WG) hipLaunchKernelGGL((k_gemm_bwd_ws<F32, WG>), dim3(grid), dim3(512), lds, s, args)
#define BSQ_BF16A_LAUNCH(F32, OPS) hipLaunchKernelGGL((k_gemm_bf16a<F32, OPS>), dim3(grid), dim3(256), lds, s, args)
    if (args.bf16 || args.w4) {
        if (args.wgrad || (args.bf16 && args.w4)) return hipErrorInvalidValue;  // row-ragged tiles only
        if (args.w4) {
            if (args.out_f32)
                BSQ_BF16A_LAUNCH(true, OPS_W4);
            else
                BSQ_BF16A_LAUNCH(false, OPS_W4);
        } else if (args.out_f32) {
            BSQ_BF16A_LAUNCH(true, OPS_BF16);
        } else {
            BSQ_BF16A_LAUNCH(false, OPS_BF16);
        }
    } else if (args.out_f32) {
        if (args.wgrad)
            BSQ_MX_LAUNCH(true, true);
        else
            BSQ_MX_LAUNCH(true, false);
    } else {
        if (args.wgrad)
            BSQ_MX_LAUNCH(false, true);
        else
            BSQ_MX_LAUNCH(false, false);
    }
#undef BSQ_MX_LAUNCH
#undef BSQ_BF16A_LAUNCH
    return hipGetLastError();
}

}  // namespace bsq
