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
// per super-stage with 15 MFMA k steps of latency to spare.  The refill slot
// runs on across tile boundaries: two super-stages before a tile ends it
// starts fetching the next tile, so a tile begins with its first two
// super-stages in LDS and no DMA wait.
//
// k order inside a 64-element group: the MFMA takes 8 k values per lane from
// lane group g = lane / 32.  Lane g of a row takes the group's code bytes
// [16g, 16g + 16) -- k in [32g, 32g + 32) -- and feeds dword j of them to k
// step j; A and B use the same assignment, so every product pairs equal k.
// The two 16-element scale blocks a lane touches in a group are bytes 2g and
// 2g + 1 of the row's scale dword for that group.
//
// Output columns: lane l of MFMA tile j reads the B row at ring position
// 32 j + l of its wave's 128 rows, and the DMA places there output column
// 4 l + j, so a lane ends the tile with four adjacent columns of every row
// it holds.  The epilogue scales and rounds them in registers and stores
// them directly (each store instruction covers two rows of 256 contiguous
// bytes), with no LDS staging and no barrier.
//
// Schedule: each k step issues its 16 MFMAs with the dequantization of the
// next step (8 fragments, half a fragment per MFMA; half-height tiles: 8
// MFMAs, 6 fragments), the LDS reads of the next group and, once per
// super-stage, the ring refill pinned between them by sched_barrier, so
// VALU, LDS and DMA work runs in the matrix core's shadow.  The loop body has no branches: a branch splits the schedule into
// blocks, and the compiler then sinks each step's dequantization past it,
// next to the MFMAs that wait for it.
//
// Expert tails: an expert's last row tile holds its remaining 1..256 rows,
// the rest padding.  A tile of at most 128 rows runs a second copy of the
// loop (chosen once per tile, so neither copy has a branch inside) in which
// wave row wm takes row groups wm and 2 + wm: 8 MFMAs per k step instead of
// 16, and 6 fragments to dequantize instead of 8 (the B fragments are needed
// either way).  The padding MFMA work falls from 10.5% to 5.2% of the bench
// shape's.
//
// SWIGLU (the gate/up projection with the activation in its epilogue): the
// weight stack holds [gate; up] rows per expert (N = 2 I, I % 128 == 0).
// Output tile nt covers H columns [128 nt, +128); wave column wn takes H
// columns 64 wn + 0..63, and its MFMA tiles j = 0, 1 read the gate rows and
// j = 2, 3 the matching up rows of columns 64 wn + 2 l + (j & 1).  Each lane
// thus holds gate and up of two adjacent H columns; the epilogue rounds each
// scaled value to bf16 -- the values the plain GEMM would store -- and
// writes H = swiglu_pair(gate, up): the gate/up output never reaches memory.
// The "Cursor Composer 2 report deep dive", section 1, places the per-token
// scaling cost in the quantize and GEMM epilogue; here the activation joins
// it.
#include "device_common.h"
#include "gemm_common.h"
#include "gemm_pipe.h"

#include <stddef.h>

namespace bsq {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int FWD_BM = 256;
constexpr int FWD_BN = 256;
constexpr int FS_K = 256;                 // K elements per super-stage
constexpr int FS_CB = FS_K / 2;           // code bytes per row per super-stage
constexpr int FS_SB = FS_K / 16;          // scale bytes per row per super-stage
constexpr int FS_CODE_TILE = 256 * FS_CB; // one operand's codes (32 KB)
constexpr int FS_SCALE_TILE = 256 * FS_SB;

struct FwdSmem {
    uint8_t a[2][FS_CODE_TILE];
    uint8_t b[2][FS_CODE_TILE];
    uint8_t sa[2][FS_SCALE_TILE];
    uint8_t sb[2][FS_SCALE_TILE];
    // Per-token decode scales of the tile's rows and per-output-channel
    // scales of its columns, double-buffered: the next tile's land while the
    // current tile's epilogue reads its own.
    float rs_a[2][FWD_BM];
    float rs_w[2][FWD_BN];
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

template <bool OUT_F32, bool SWIGLU, bool KFULL>
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
    // dword lane & 3 of the row's 16 scale bytes.  KFULL (K a multiple of
    // 256, scale rows 16-byte aligned): one instruction per operand moves
    // row 64 * wave + lane's 16 bytes.
    const int srow0 = 64 * wave + (lane >> 2);
    const uint32_t sdw = (uint32_t)(lane & 3);
    // Fragment reads: lane (lr, g) of group gg takes logical chunk 2gg + g of
    // row lr of each 32-row group: slot (2gg + g) ^ swz8(lr).
    const uint32_t fr = (uint32_t)(lr * FS_CB + 16 * (g ^ swz8(lr)));
    const uint32_t fa = offsetof(FwdSmem, a) + (uint32_t)(wm * 128 * FS_CB);
    const uint32_t fb = offsetof(FwdSmem, b) + (uint32_t)(wn * 128 * FS_CB);
    // (lane group g's two scale bytes of a group sit at byte 2g of its dword)
    const uint32_t fsa = offsetof(FwdSmem, sa) + (uint32_t)((wm * 128 + lr) * FS_SB + 2 * g);
    const uint32_t fsb = offsetof(FwdSmem, sb) + (uint32_t)((wn * 128 + lr) * FS_SB + 2 * g);

    // decode tables in LDS behind the staging buffers (when they fit)
    __attribute__((address_space(3))) int32_t* tab =
        (__attribute__((address_space(3))) int32_t*)(smem_raw + sizeof(FwdSmem));
    const bool tab_lds = p.E <= LDS_TABLE_MAX_E;
    if (tab_lds) fill_lds_tables(tab, p.plan, p.offsets, p.E);
    if (tid == 0) s_tile = claim_tile(p.plan, xcd, total, dq);
    __syncthreads();
    int tile = __builtin_amdgcn_readfirstlane(s_tile);  // uniform: keeps tile state in SGPRs

    // State of the tile whose operands are in flight (uniform).  B rows reach
    // LDS permuted: ring position 128 wn + 32 j + l (the row that lane l of
    // wave column wn reads for MFMA tile j) holds
    //   plain:  output column 128 wn + 4 l + j,
    //   SWIGLU: gate (j < 2) or up (j >= 2) row of H column 64 wn + 2 l + (j & 1),
    // so each lane ends a tile holding four adjacent output columns of every
    // row it owns (SWIGLU: gate and up of two adjacent H columns) and the
    // epilogue stores straight from the accumulators.  For DMA wave w the
    // position's row splits into a wave term, a lane term and an instruction
    // term (see issue_part).
    int64_t m_base = 0, n_base = 0;
    int rows_a = 0, rows_b = 0, nt = 0;
    __amdgpu_buffer_rsrc_t dA = rsrc_n(nullptr, 0), dB = dA, dAs = dA, dBs = dA;
    const float* rs_w_src = nullptr;
    const int bw0 = SWIGLU ? 64 * (wave >> 1) : 128 * (wave >> 1) + 2 * (wave & 1);  // local B row, wave term
    // Per-lane DMA offsets at k = 0 (codes: row part only, the chunk comes
    // from vch0 / vch1).  Rows past the tile's valid rows fall outside the
    // descriptor's byte range and read as zero.
    const uint32_t vra = (uint32_t)drow0 * KB;
    const uint32_t vrb = (uint32_t)((SWIGLU ? 2 : 4) * (lane >> 3)) * KB;
    const uint32_t vsa = (uint32_t)srow0 * KS + 4 * sdw;
    const uint32_t vsb = (uint32_t)((SWIGLU ? 2 : 4) * (lane >> 2)) * KS + 4 * sdw;
    const uint32_t vsa16 = (uint32_t)(64 * wave + lane) * KS;
    const uint32_t vsb16 = (uint32_t)((SWIGLU ? 2 : 4) * (lane & 31) + (lane >> 5)) * KS;
    const uint32_t vch0 = 16 * dch0, vch1 = 16 * dch1;
    // with the chunk of each parity folded in (instruction i uses parity i & 1)
    const uint32_t va0 = vra + vch0, va1 = vra + vch1, vb0 = vrb + vch0, vb1 = vrb + vch1;

    uint32_t par = 0;  // ring slot of the current tile's super-stage 0
    int rb = 0;        // scale buffer of the current tile
    auto setup = [&](int t) {
        const TileRef tr = decode_tile_any(tab_lds, tab, p.plan, p.offsets, p.E, t, lane);
        const int e = tr.e;
        const int64_t off0 = tr.off0, off1 = tr.off1;
        int mt;
        grouped_tile(tr.local, (int)((off1 - off0 + FWD_BM - 1) / FWD_BM), NT, mt, nt);
        m_base = uniform_i64(off0 + (int64_t)mt * FWD_BM);
        rows_a = __builtin_amdgcn_readfirstlane((int)min((int64_t)FWD_BM, off1 - m_base));
        n_base = uniform_i64((int64_t)nt * FWD_BN);
        rows_b = SWIGLU ? FWD_BN : __builtin_amdgcn_readfirstlane((int)min((int64_t)FWD_BN, p.N - n_base));
        // first weight row of this wave's DMA rows (SWIGLU: odd waves fetch up rows)
        const int64_t wrow = SWIGLU ? uniform_i64((int64_t)e * p.N + ((wave & 1) ? p.N / 2 : 0) + 128 * (int64_t)nt + bw0)
                                    : uniform_i64((int64_t)e * p.N + n_base + bw0);
        // B rows this wave may read past wrow: plain, local rows bw0 ..
        // rows_b - 1; SWIGLU, the 64 rows of its half (all valid)
        const uint32_t nbr = SWIGLU ? 64u : (uint32_t)max(0, rows_b - bw0);
        dA = rsrc_n(uniform_ptr(p.a_codes + m_base * (int64_t)KB), (uint32_t)rows_a * KB);
        dB = rsrc_n(uniform_ptr(p.w_codes + wrow * (int64_t)KB), nbr * KB);
        dAs = rsrc_n(uniform_ptr(p.a_bscale + m_base * (int64_t)KS), (uint32_t)rows_a * KS);
        dBs = rsrc_n(uniform_ptr(p.w_bscale + wrow * (int64_t)KS), nbr * KS);
        // column scales in natural order: rs_w[c] is output column c of the
        // tile (SWIGLU: gate rows at 0..127, up rows at 128..255)
        rs_w_src = SWIGLU ? uniform_ptr(p.w_rscale + (int64_t)e * p.N + 128 * (int64_t)nt + (wave >= 2 ? p.N / 2 - 128 : 0))
                          : uniform_ptr(p.w_rscale + (int64_t)e * p.N + n_base);
    };

    // DMA of super-stage S into ring slot q in 12 parts of 2
    // instructions: parts 0..7 code rows (A and B of instruction i),
    // parts 8..11 scale rows.  Chunks past K read as zero.
    auto issue_part = [&](int S, uint32_t q, int part, bool ok) {
        // Each offset is a loop-invariant lane base plus a wave-uniform term;
        // the row pitch is laundered at each use, so the compiler forms the
        // sum at the DMA instead of keeping one live register per
        // (instruction, operand) across the loops.
        if (part < 8) {
            const int i = part;
            // B: ring position 64 w + 8 i + lane / 8 holds local row bw0 + 4 (lane / 8) + bir
            // (SWIGLU: 2 (lane / 8))
            const int bir = SWIGLU ? 16 * (i & 3) + (i >> 2) : 32 * (i & 3) + (i >> 2);
            const uint32_t kb = opaque_s(KB);
            const uint32_t ks = (uint32_t)S * FS_CB;
            // chunk inside the row (only the last super-stage of a K tail has any outside)
            const bool okk = KFULL ? ok : ok & (ks + ((i & 1) ? vch1 : vch0) < KB);
            const uint32_t ldst = q * FS_CODE_TILE + 1024u * (uint32_t)(8 * wave + i);
            const uint32_t oa = ((i & 1) ? va1 : va0) + (ks + (uint32_t)(8 * i) * kb);
            const uint32_t ob = ((i & 1) ? vb1 : vb0) + (ks + (uint32_t)bir * kb);
            dma_lds_r<16>(dA, okk ? oa : OOB, LA + ldst);
            dma_lds_r<16>(dB, okk ? ob : OOB, LB + ldst);
        } else if constexpr (KFULL) {
            // B: ring position 64 w + lane holds local row bw0 + 4 (lane % 32) + lane / 32
            // (SWIGLU: 2 (lane % 32))
            if (part == 8) {
                const uint32_t so = (uint32_t)S * FS_SB;
                const uint32_t ldst = q * FS_SCALE_TILE + 1024u * (uint32_t)wave;
                dma_lds_r<16>(dAs, ok ? vsa16 + so : OOB, LSA + ldst);
                dma_lds_r<16>(dBs, ok ? vsb16 + so : OOB, LSB + ldst);
            }
        } else {
            const int i = part - 8;
            // B: ring position 64 w + 16 i + lane / 4 holds local row bw0 + 4 (lane / 4) + sir
            // (SWIGLU: 2 (lane / 4))
            const int sir = SWIGLU ? 32 * (i & 1) + (i >> 1) : 64 * (i & 1) + (i >> 1);
            const uint32_t kq = opaque_s(KS);
            const uint32_t so = (uint32_t)S * FS_SB;
            const bool oks = ok & (so + 4 * sdw < KS);
            const uint32_t ldst = q * FS_SCALE_TILE + 256u * (uint32_t)(4 * wave + i);
            const uint32_t oa = vsa + (so + (uint32_t)(16 * i) * kq);
            const uint32_t ob = vsb + (so + (uint32_t)sir * kq);
            dma_lds_r<4>(dAs, oks ? oa : OOB, LSA + ldst);
            dma_lds_r<4>(dBs, oks ? ob : OOB, LSB + ldst);
        }
    };
    // the tile's row and column scales into buffer rb
    auto issue_rscale = [&](int rb) {
        const int r = 64 * wave + lane;
        dma4(make_desc(uniform_ptr(p.a_rscale + m_base)), r < rows_a ? 4u * (uint32_t)r : OOB,
             LRA + 1024u * (uint32_t)rb + 256u * wave);
        dma4(make_desc(rs_w_src), r < rows_b ? 4u * (uint32_t)r : OOB, LRW + 1024u * (uint32_t)rb + 256u * wave);
    };

    // LDS reads of group G (super-stage G / 4, group G % 4 of it); part f
    // (0..7) reads fragment f: A rows of group f, or B rows of group f - 4.
    // HALF (a tile of at most 128 rows): A fragment i holds row group 2i + wm
    // instead of 4wm + i, so both wave rows share the valid rows 0..127.
    auto read_part = [&](int G, FwdRaw& r, int f, auto HALFC) {
        constexpr bool HALF = decltype(HALFC)::value != 0;
        const uint32_t q = (((uint32_t)G >> 2) + par) & 1, gg = (uint32_t)G & 3;
        const int i = f & 3;
        const int rg = (f < 4 && HALF) ? 64 * i - 96 * wm : 32 * i;  // rows past the wave's base row
        const uint32_t co = ((f < 4) ? fa : fb) + q * FS_CODE_TILE + (uint32_t)(rg * FS_CB);
        const uint32_t so = ((f < 4) ? fsa : fsb) + q * FS_SCALE_TILE + (uint32_t)(rg * FS_SB) + 4 * gg;
        r.c[f] = *(const __attribute__((address_space(3))) u32x4*)(lds + co + (fr ^ (32u * gg)));
        r.s[f] = *(const __attribute__((address_space(3))) uint16_t*)(lds + so);
    };
    // this lane's two block scales of fragment f in the group, as fp16
    auto conv_scale = [&](const FwdRaw& r, int f) -> half2v {
        return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.s[f], 1.0f, false);
    };

    // Tile pipeline.  A tile's super-stage 0 lives in ring slot `par`.  The
    // refill slot of super-stage S always fills the slot S just released:
    // with super-stage S + 2 of this tile while there is one, then with
    // super-stages 0 and 1 of the next tile (whose DMA state setup() loads
    // at the start of super-stage nsup - 2, when this tile's DMA is all
    // issued), else with nothing (out-of-range reads).  The schedule thus
    // has no branches, and the next tile's operands land under this tile's
    // MFMAs.  Tiles with fewer than 3 super-stages start the next tile's DMA
    // after the main loop.
    if (tile >= 0) {
        setup(tile);
#pragma unroll
        for (int part = 0; part < 12; ++part) issue_part(0, 0, part, true);
#pragma unroll
        for (int part = 0; part < 12; ++part) issue_part(1, 1, part, true);
        issue_rscale(0);
        wait_vmcnt<0>();
    }

    for (;;) {
        if (tile < 0) break;
        // claim the next tile now; the atomic's round trip hides behind
        // this tile (its value is first read when the next tile is published)
        PendingClaim pclaim{0, -1};
        if (tid == 0) pclaim = claim_start(p.plan, xcd, dq);
        // this tile's epilogue coordinates (setup() moves on to the next tile
        // during the last super-stage)
        const int64_t em = m_base, en = n_base;
        const int ea = rows_a, eb = rows_b, ent = nt, erb = rb;
        const uint32_t qn = ((uint32_t)nsup + par) & 1;  // slot of the next tile's super-stage 0
        int ntile = -1;
        bool has_next = false;  // the DMA state holds the next tile's

        float16v acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

        // every wave waited for its own share of super-stages 0 and 1 (and
        // the scales) after its previous epilogue
        block_barrier();

        FwdRaw raw[2];
        FwdOps ops[2];
        half2v sh[8];

        // A k step's fragments: all eight, or (HALF) A row groups 0 and 1 and
        // the four B fragments.  Dequant items (fragment, half) per MFMA slot:
        // full tiles one per slot (slot k: fragment k / 2, half k % 2); HALF
        // tiles twelve over eight slots (slots 0..3 both halves of fragments
        // 0, 1, 4, 5; slots 4..7 one half of fragments 6, 7).
        auto run_tile = [&](auto HALFC) {
            constexpr bool HALF = decltype(HALFC)::value != 0;
            constexpr int NF = HALF ? 6 : 8;
            constexpr int NK = HALF ? 8 : 16;
            auto frag = [](int n) { return HALF ? (n < 2 ? n : n + 2) : n; };  // n-th fragment of a k step
#pragma unroll
            for (int n = 0; n < NF; ++n) read_part(0, raw[0], frag(n), HALFC);
            wait_lgkmcnt0();
#pragma unroll
            for (int n = 0; n < NF; ++n) {
                const int f = frag(n);
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
                            // the DMA issued one super-stage ago (super-stage
                            // S+1, or the next tile's 0) has landed, and every
                            // wave is done reading this slot
                            wait_vmcnt<0>();
                            wait_lgkmcnt0();
                            block_barrier();
                        }
                        if (j == 3) wait_lgkmcnt0();  // next group's raw data
#pragma unroll
                        for (int k = 0; k < NK; ++k) {
                            const int i = k >> 2, jj = k & 3;
                            acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(o.f[i], o.f[4 + jj], acc[i][jj], 0, 0, 0);
                            // dequantize the items of this slot for the next k step
                            auto item = [&](int f, int h, bool first) {
                                const uint32_t w = j < 3 ? cur.c[f][(j + 1) & 3] : nxt.c[f][0];
                                if (j == 3 && first) sh[f] = conv_scale(nxt, f);
                                const _Float16 sc = (j < 3 && (j + 1) >= 2) ? sh[f][1] : sh[f][0];
                                if (h)
                                    dequant_half<1>(on.f[f], w, sc);
                                else
                                    dequant_half<0>(on.f[f], w, sc);
                            };
                            if constexpr (HALF) {
                                if (k < 4) {
                                    item(frag(k), 0, true);
                                    item(frag(k), 1, false);
                                } else {
                                    item(k < 6 ? 6 : 7, k & 1, (k & 1) == 0);
                                }
                            } else {
                                item(k >> 1, k & 1, (k & 1) == 0);
                            }
                            // LDS reads of the next group
                            if (j == 0 && k < NF) read_part(G + 1, nxt, frag(k), HALFC);
                            // refill of the slot just freed with super-stage S+2
                            // (this tile's super-stage S+2, else the next tile's S+2-nsup)
                            // (6 parts in each of k steps 1 and 2: a burst of DMA
                            // instructions stalls the wave issuing them)
                            if (gg == 3 && (j == 1 || j == 2) && k < 6)
                                issue_part(S + 2 < nsup ? S + 2 : S + 2 - nsup, ((uint32_t)S + par) & 1, 6 * (j - 1) + k,
                                           (S + 2 < nsup) | has_next);
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    }
                }
            };
            for (int S = 0; S < nsup; ++S) {
                // the barrier inside super-stage nsup - 3 publishes the next
                // tile; from super-stage nsup - 2 on the DMA state is the next
                // tile's
                if (nsup >= 3) {
                    if (S == nsup - 3 && tid == 0) s_tile = claim_finish(p.plan, xcd, total, dq, pclaim);
                    if (S == nsup - 2) {
                        ntile = __builtin_amdgcn_readfirstlane(s_tile);
                        has_next = ntile >= 0;
                        if (has_next) {
                            setup(ntile);
                            issue_rscale(rb ^ 1);
                        }
                    }
                }
                superstage(S);
            }
        };
        // a tile of at most 128 rows (an expert's tail) runs half the MFMAs
        const bool half = ea <= FWD_BM / 2;
        if (half)
            run_tile(IC<1>{});
        else
            run_tile(IC<0>{});

        if (nsup < 3) {
            // every wave is done with the ring; the next tile's DMA now
            wait_lgkmcnt0();
            if (tid == 0) s_tile = claim_finish(p.plan, xcd, total, dq, pclaim);
            block_barrier();
            ntile = __builtin_amdgcn_readfirstlane(s_tile);
            if (ntile >= 0) {
                setup(ntile);
#pragma unroll
                for (int part = 0; part < 12; ++part) issue_part(0, qn, part, true);
#pragma unroll
                for (int part = 0; part < 12; ++part) issue_part(1, qn ^ 1u, part, true);
                issue_rscale(rb ^ 1);
            }
        }

        // Epilogue straight from the accumulators.  Lane (lr, g) of wave
        // (wm, wn) holds, in acc[i][j][v], tile row wm*128 + 32i + 8(v/4) +
        // 4g + v%4 (HALF: 32(2i + wm) + 8(v/4) + 4g + v%4, i < 2) and ring
        // column position 128 wn + 32 j + lr.  Each value is
        // scaled by s_a[row] and then s_w[col] and rounded once (bf16 to
        // nearest even); rows past the expert's end and columns past N are not
        // stored.  A store instruction writes two rows of 256 contiguous bytes
        // (plain bf16; 512 for fp32; SWIGLU: 128 bytes of H).
        {
            const __attribute__((address_space(3))) float* rsa =
                (const __attribute__((address_space(3))) float*)(lds + offsetof(FwdSmem, rs_a) + 1024u * (uint32_t)erb);
            const __attribute__((address_space(3))) float* rsw =
                (const __attribute__((address_space(3))) float*)(lds + offsetof(FwdSmem, rs_w) + 1024u * (uint32_t)erb);
            const __amdgpu_buffer_rsrc_t rc =
                make_rsrc(uniform_ptr(reinterpret_cast<char*>(p.y) +
                                      (SWIGLU ? (em * p.ldo + 128 * (int64_t)ent) * 2 : (em * p.N + en) * esz)),
                          0x7FFFFFFFu);
            // laundered: the row offsets and LDS addresses below are the same
            // for every tile, and hoisting them would keep 80 registers live
            // across the main loop
            const uint32_t ldcb = opaque_s(SWIGLU ? (uint32_t)p.ldo * 2u : (uint32_t)p.N * (uint32_t)esz);
            const int r0w = (int)opaque_v((uint32_t)(wm * 128 + 4 * g));
            if constexpr (SWIGLU) {
                const int c = 64 * wn + 2 * lr;  // H columns c, c + 1 of the tile
                const f32x2 swg = *(const __attribute__((address_space(3))) f32x2*)(rsw + c);
                const f32x2 swu = *(const __attribute__((address_space(3))) f32x2*)(rsw + 128 + c);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (half && i >= 2) continue;  // (HALF) row groups 2i + wm only
                    const int rgi = half ? 64 * i - 96 * wm : 32 * i;
#pragma unroll
                    for (int vq = 0; vq < 4; ++vq) {
                        const int r0 = r0w + rgi + 8 * vq;
                        const f32x4 sa4 = *(const __attribute__((address_space(3))) f32x4*)(rsa + r0);
#pragma unroll
                        for (int vv = 0; vv < 4; ++vv) {
                            const int v = 4 * vq + vv;
                            const float sa = sa4[vv];
                            const float g0 = (acc[i][0][v] * sa) * swg[0], g1 = (acc[i][1][v] * sa) * swg[1];
                            const float u0 = (acc[i][2][v] * sa) * swu[0], u1 = (acc[i][3][v] * sa) * swu[1];
                            const uint32_t hv = swiglu_pair(pack_bf16x2(g0, g1), pack_bf16x2(u0, u1));
                            const int row = r0 + vv;
                            __builtin_amdgcn_raw_buffer_store_b32(hv, rc, row < ea ? (int)((uint32_t)row * ldcb + 2u * (uint32_t)c) : (int)OOB,
                                                                  0, OUT_STORE_NT);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            } else {
                const int col = wn * 128 + 4 * lr;  // columns col .. col + 3 of the tile
                const bool okc = col < eb;
                const f32x4 sw = *(const __attribute__((address_space(3))) f32x4*)(rsw + col);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (half && i >= 2) continue;  // (HALF) row groups 2i + wm only
                    const int rgi = half ? 64 * i - 96 * wm : 32 * i;
#pragma unroll
                    for (int vq = 0; vq < 4; ++vq) {
                        const int r0 = r0w + rgi + 8 * vq;
                        const f32x4 sa4 = *(const __attribute__((address_space(3))) f32x4*)(rsa + r0);
#pragma unroll
                        for (int vv = 0; vv < 4; ++vv) {
                            const int v = 4 * vq + vv;
                            const float sa = sa4[vv];
                            const float y0 = (acc[i][0][v] * sa) * sw[0], y1 = (acc[i][1][v] * sa) * sw[1];
                            const float y2 = (acc[i][2][v] * sa) * sw[2], y3 = (acc[i][3][v] * sa) * sw[3];
                            const int row = r0 + vv;
                            const int off = (okc & (row < ea)) ? (int)((uint32_t)row * ldcb + (uint32_t)(col * esz)) : (int)OOB;
                            if constexpr (OUT_F32) {
                                u32x4 y;
                                y[0] = __float_as_uint(y0); y[1] = __float_as_uint(y1);
                                y[2] = __float_as_uint(y2); y[3] = __float_as_uint(y3);
                                __builtin_amdgcn_raw_buffer_store_b128(y, rc, off, 0, OUT_STORE_NT);
                            } else {
                                u32x2 y;
                                y[0] = pack_bf16x2(y0, y1);
                                y[1] = pack_bf16x2(y2, y3);
                                __builtin_amdgcn_raw_buffer_store_b64(y, rc, off, 0, OUT_STORE_NT);
                            }
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
        }
        // the next tile's super-stages 0 and 1 and scales (and these stores)
        wait_vmcnt<0>();
        par = qn;
        rb ^= 1;
        tile = ntile;
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
        const void* ks[6] = {reinterpret_cast<const void*>(&k_gemm_fwd_nvfp4v<true, false, false>),
                             reinterpret_cast<const void*>(&k_gemm_fwd_nvfp4v<false, false, false>),
                             reinterpret_cast<const void*>(&k_gemm_fwd_nvfp4v<false, true, false>),
                             reinterpret_cast<const void*>(&k_gemm_fwd_nvfp4v<true, false, true>),
                             reinterpret_cast<const void*>(&k_gemm_fwd_nvfp4v<false, false, true>),
                             reinterpret_cast<const void*>(&k_gemm_fwd_nvfp4v<false, true, true>)};
        for (const void* k : ks) {
            err = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                      (int)(sizeof(FwdSmem) + lds_table_bytes(LDS_TABLE_MAX_E)));
            if (err != hipSuccess) return err;
        }
        attr_set = true;
    }
    FwdArgs p{a_codes, a_bscale, a_rscale, w_codes, w_bscale, w_rscale, offsets, E, N, K, y, y_f32, plan, ldo};
    const size_t lds = sizeof(FwdSmem) + lds_table_bytes(E);
    // whole 256-element super-stages and 16-byte aligned scale rows: each
    // row's 16 scale bytes of a super-stage move as one 16-byte load
    const bool kfull = K % FS_K == 0 && (reinterpret_cast<uintptr_t>(a_bscale) & 15) == 0 &&
                       (reinterpret_cast<uintptr_t>(w_bscale) & 15) == 0;
#define BSQ_FWD_LAUNCH(F32, SW, KF) hipLaunchKernelGGL((k_gemm_fwd_nvfp4v<F32, SW, KF>), dim3(grid), dim3(256), lds, s, p)
    if (swiglu) {
        if (kfull) BSQ_FWD_LAUNCH(false, true, true); else BSQ_FWD_LAUNCH(false, true, false);
    } else if (y_f32) {
        if (kfull) BSQ_FWD_LAUNCH(true, false, true); else BSQ_FWD_LAUNCH(true, false, false);
    } else {
        if (kfull) BSQ_FWD_LAUNCH(false, false, true); else BSQ_FWD_LAUNCH(false, false, false);
    }
#undef BSQ_FWD_LAUNCH
    return hipGetLastError();
}

}  // namespace bsq
