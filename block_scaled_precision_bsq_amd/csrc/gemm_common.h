// Tile planner and persistent tile scheduler shared by the grouped GEMMs.
//
// Expert grouped GEMMs see skewed routing: per-expert token counts differ by
// 40x or more, and some experts are empty ("Composer 2 Technical Report",
// section 6.1: the expert grouped GEMM gets more efficient with more tokens
// per rank; the 384-expert, top-8 MoE class of "Scaling and Optimizing
// Frontier Model Training").  The counts live on the device (`offsets`), so
// the host cannot size the launch; instead:
//  1. k_plan (one workgroup) reads offsets, validates them, orders the experts
//     (by index, or longest-reduction-first when a tile's cost grows with the
//     expert's token count) and writes per-expert tile prefix sums into the
//     workspace, zeroing the claim counters;
//  2. the GEMM runs a persistent grid (one workgroup per CU).  The tile list is
//     cut into chunks of XCD_CHUNK consecutive tiles (one per CU of an XCD);
//     chunk j belongs to XCD j % 8.  Within an expert, tiles are ordered in
//     groups of GROUP_M row-tiles x all column-tiles, so one chunk covers a
//     4 x 8 block of output tiles: 4 A panels and 8 B panels instead of 32 + 1,
//     which is what one XCD's 4 MB L2 can keep resident per k stage.  Tiles
//     are claimed through one atomic counter per XCD; a workgroup drains its
//     own XCD's queue first and then steals from the others.
// Each output tile is computed by exactly one workgroup in a fixed k order:
// results do not depend on which workgroup runs it (deterministic, batch
// invariant; no split-K, no float atomics).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsq {

constexpr int PLAN_HDR = 16;      // int32 words before the per-expert arrays
constexpr int PLAN_CTR = 0;       // [0, 8): per-XCD claim counters
constexpr int PLAN_TOTAL = 8;     // total tiles
constexpr int PLAN_ERR = 9;       // 1 = invalid offsets (no work done)
constexpr int MAX_EXPERTS = 4096;

enum PlanMode { PLAN_RAGGED_ROWS = 0, PLAN_RAGGED_REDUCTION = 1 };

// int32 words of one plan: header + tile_start[E+1] + order[E].
__host__ __device__ inline int64_t plan_words(int E) { return PLAN_HDR + 2 * (int64_t)E + 1; }

__device__ __forceinline__ const int32_t* plan_start(const int32_t* plan) { return plan + PLAN_HDR; }
__device__ __forceinline__ const int32_t* plan_order(const int32_t* plan, int E) { return plan + PLAN_HDR + E + 1; }

constexpr int XCD_CHUNK = 32;  // tiles per chunk = CUs per XCD on MI355X
constexpr int GROUP_M = 4;     // row-tiles per group in the tile order

// Claim the next tile for this workgroup (thread 0 only).  Returns -1 when
// every queue is drained.  `d` is the number of queues already found empty.
__device__ __forceinline__ int claim_tile(int32_t* plan, int xcd, int total, int& d) {
    while (d < 8) {
        const int q = (xcd + d) & 7;
        const int c = atomicAdd(&plan[PLAN_CTR + q], 1);
        const int t = (q + 8 * (c / XCD_CHUNK)) * XCD_CHUNK + (c % XCD_CHUNK);
        if (t < total) return t;
        ++d;
    }
    return -1;
}

// The same claim in two halves, so that the atomic's round trip overlaps a
// tile's work: claim_start issues the first attempt (the counter value
// comes back in the background; nothing waits for it until it is used) and
// claim_finish decodes it, falling back to claim_tile when that queue was
// already drained.  Thread 0 only.
struct PendingClaim {
    int c;  // counter value returned by the atomic
    int q;  // queue it came from; -1 when every queue was already empty
};
__device__ __forceinline__ PendingClaim claim_start(int32_t* plan, int xcd, int d) {
    PendingClaim r{0, -1};
    if (d < 8) {
        r.q = (xcd + d) & 7;
        r.c = atomicAdd(&plan[PLAN_CTR + r.q], 1);
    }
    return r;
}
__device__ __forceinline__ int claim_finish(int32_t* plan, int xcd, int total, int& d, PendingClaim pc) {
    if (pc.q < 0) return -1;
    const int t = (pc.q + 8 * (pc.c / XCD_CHUNK)) * XCD_CHUNK + (pc.c % XCD_CHUNK);
    if (t < total) return t;
    ++d;
    return claim_tile(plan, xcd, total, d);
}

// Grouped order inside one expert: local index -> (row-tile, column-tile).
// GROUP_M row-tiles are swept together across all `nt` column-tiles.
__device__ __forceinline__ void grouped_tile(int local, int mt_count, int nt, int& mt, int& ct) {
    const int per_group = GROUP_M * nt;
    const int g = local / per_group;
    const int first = g * GROUP_M;
    const int rows = min(GROUP_M, mt_count - first);
    const int r = local - g * per_group;
    mt = first + r % rows;
    ct = r / rows;
}

// Position of tile t in the expert order: last i with tile_start[i] <= t
// (empty experts have tile_start[i] == tile_start[i+1] and are skipped).
__device__ __forceinline__ int find_position(const int32_t* start, int E, int t) {
    int lo = 0, hi = E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (start[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Tile decode.  A tile index maps to (expert, tile within the expert) through
// the planner's per-expert tile prefix and expert order, and the expert's
// token range comes from `offsets`.  When the expert count is small enough,
// the GEMM kernels copy the three arrays into LDS behind their staging
// buffers at kernel start, so a decode costs a few LDS reads instead of a
// chain of dependent global loads; otherwise they read the global arrays.
constexpr int LDS_TABLE_MAX_E = 800;
__host__ __device__ inline size_t lds_table_bytes(int E) {
    return E <= LDS_TABLE_MAX_E ? (size_t)4 * (3 * (size_t)E + 2) : 0;
}

struct TileRef {
    int e, local;
    int64_t off0, off1;
};

template <class P>
__device__ __forceinline__ TileRef decode_tile(P start, P order, P offs, int E, int t) {
    int lo = 0, hi = E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (start[mid] <= t) lo = mid; else hi = mid - 1;
    }
    TileRef r;
    r.e = __builtin_amdgcn_readfirstlane(order[lo]);
    r.local = __builtin_amdgcn_readfirstlane(t - start[lo]);
    r.off0 = __builtin_amdgcn_readfirstlane(offs[r.e]);
    r.off1 = __builtin_amdgcn_readfirstlane(offs[r.e + 1]);
    return r;
}

typedef const __attribute__((address_space(3))) int32_t* lds_i32p;

// LDS copy of the decode arrays (start[E+1], order[E], offsets[E+1]) at `tab`;
// every thread of the workgroup takes part; the caller synchronizes.
__device__ __forceinline__ void fill_lds_tables(__attribute__((address_space(3))) int32_t* tab, const int32_t* plan,
                                                const int32_t* offsets, int E) {
    const int32_t* start = plan_start(plan);
    const int32_t* order = plan_order(plan, E);
    for (int i = threadIdx.x; i <= E; i += blockDim.x) {
        tab[i] = start[i];
        tab[2 * E + 1 + i] = offsets[i];
        if (i < E) tab[E + 1 + i] = order[i];
    }
}

// Wave-parallel decode from the LDS tables: each round reads 64 consecutive
// tile starts (one per lane) and counts those <= t; the starts never
// decrease, so the counted entries are a prefix and the last of them is the
// expert position (one round for up to 64 experts).
__device__ __forceinline__ TileRef decode_tile_lds(lds_i32p start, lds_i32p order, lds_i32p offs, int E, int t,
                                                   int lane) {
    int pos = 0, s_pos = 0;
    for (int base = 0; base < E; base += 64) {
        const int i = base + lane;
        const int st = i < E ? start[i] : 0x7FFFFFFF;
        const int c = __builtin_popcountll(__ballot(st <= t));
        if (c > 0) {
            pos = base + c - 1;
            s_pos = __builtin_amdgcn_readlane(st, c - 1);
        }
        if (c < 64) break;
    }
    TileRef r;
    r.e = __builtin_amdgcn_readfirstlane(order[pos]);
    r.local = __builtin_amdgcn_readfirstlane(t - s_pos);
    r.off0 = __builtin_amdgcn_readfirstlane(offs[r.e]);
    r.off1 = __builtin_amdgcn_readfirstlane(offs[r.e + 1]);
    return r;
}

__device__ __forceinline__ TileRef decode_tile_any(bool in_lds, const __attribute__((address_space(3))) int32_t* tab,
                                                   const int32_t* plan, const int32_t* offsets, int E, int t,
                                                   int lane) {
    if (in_lds) return decode_tile_lds(tab, tab + E + 1, tab + 2 * E + 1, E, t, lane);
    return decode_tile<const int32_t*>(plan_start(plan), plan_order(plan, E), offsets, E, t);
}

// Cache policy of the GEMM output stores: non-temporal.  An output tile is
// written once and never read back by the kernel, so it should not displace
// operand panels from L2.
constexpr int OUT_STORE_NT = 2;

// Arguments of the MXFP8 backward GEMM kernel (one launch computes either the
// dgrad or the wgrad tiles).
struct BwdArgs {
    const uint8_t* dy_codes; const uint8_t* dy_scale;    // dgrad A: ROWWISE dY [M][N]
    const uint8_t* wt_codes; const uint8_t* wt_scale;    // dgrad B: COLWISE_T W -> [K][Pw]
    const uint8_t* dyt_codes; const uint8_t* dyt_scale;  // wgrad A: COLWISE_T dY -> [N][P]
    const uint8_t* xt_codes; const uint8_t* xt_scale;    // wgrad B: COLWISE_T X -> [K][P]
    const int32_t* offsets; int E; int64_t m_total; int64_t N; int64_t K;
    int64_t P;   // padded token columns of the COLWISE_T activations
    int64_t Pw;  // padded columns of the COLWISE_T weights
    void* out; int out_f32;
    int wgrad;   // 0: dgrad tiles, 1: wgrad tiles
    int32_t* plan;
    // dgrad tiles only: 0 = B is the COLWISE_T weight transpose Wt [K][Pw]
    // (expert e at column 128*(e + e*N/128)); 1 = B is a ROWWISE MXFP8 weight stack
    // W [E*K][N] with block-major scales [N/32][E*K] (the forward MXFP8 GEMM,
    // whose reduction is N here and whose output width is K).
    int b_rows;
    // 1: plain bf16 operands (the bf16 baseline), dgrad-style tiles with B as
    // a row-major weight stack (b_rows layout, 2 bytes per element, no scales)
    int bf16;
    // 1: bf16 A rows against a packed NVFP4-variant weight stack (frozen
    // experts): wt_codes [E*K][N/2], wt_scale [E*K][N/16] E4M3, wt_rscale
    // [E*K] fp32; dgrad-style tiles, reduction N, output width K
    int w4;
    const float* wt_rscale;
};

hipError_t launch_plan(const int32_t* offsets, int E, int64_t m_total, int mode, int bm, int nt, int kt,
                       int32_t* plan, hipStream_t s);
hipError_t launch_gemm_bwd_mxfp8(const BwdArgs& args, int grid, hipStream_t s);
hipError_t launch_gemm_fwd_nvfp4v(const uint8_t* a_codes, const uint8_t* a_bscale, const float* a_rscale,
                                  const uint8_t* w_codes, const uint8_t* w_bscale, const float* w_rscale,
                                  const int32_t* offsets, int E, int64_t m_total, int64_t N, int64_t K, void* y,
                                  int y_f32, int swiglu, int64_t ldo, int32_t* plan, int grid, hipStream_t s);

}  // namespace bsq
