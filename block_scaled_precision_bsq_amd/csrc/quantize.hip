// Quantizer kernels for gfx950: NVFP4 variant (row-wise, fused per-token
// absmax) and MXFP8 (row-wise and column-transposing per expert segment).
//
// "Composer 2 Technical Report" (papercache.org summary), section 6.1:
//  - MoE forward: BF16 -> FP4 E2M1 with an FP8 E4M3 scale per 16-element block
//    and an FP32 scale per token, replacing the per-tensor FP32 scale, which is
//    batch-variant and leaks information from later tokens into earlier ones;
//  - NVFP4 quantization needs IEEE-compliant division (a fast approximate
//    divide made RL training diverge);
//  - MoE backward: MXFP8, E4M3 values with an E8M0 scale per 32 elements.
// The per-token scale costs a row reduction ("Cursor Composer 2 report deep
// dive", section 1): here it is fused -- one wave keeps its whole row in VGPRs,
// reduces block maxima with cross-lane shuffles and encodes from registers,
// so HBM sees one read of the row and one write of the codes.
//
// This file is compiled with -ffp-contract=off: every float operation below
// is a single IEEE operation in round-to-nearest-even with denormals kept.
#include "device_common.h"
#include "gemm_pipe.h"

namespace bsq {

// ---------------------------------------------------------------- NVFP4v
//
// One wave64 per row; lane l owns 16-element blocks l, l+64, l+128, ...
// (BPL of them at most), loaded as two 16-byte vectors each: a wave reads
// 2 KB of consecutive bytes per step.
//
// RN32(x / d_b) is computed as RN32(x * RN64(1 / d_b)): both routes give the
// same binary32 result.  Sketch: the binary64 product differs from x/d_b by
// at most ~2^-52 relative, while a quotient of two binary32 numbers is never
// a binary32 rounding midpoint and lies at least 2^-49 (relative) away from
// every midpoint, so both round to the same binary32 number.  The reciprocal
// costs one binary64 division per 16 elements instead of 16 fp32 divisions.
//
// SWIGLU: x holds rows [gate | up] of 2 * cols bf16 and the row quantized is
// H = swiglu_pair(gate, up) (device_common.h; the activation between the two
// forward GEMMs, not on the pages).  H is also written to h (when non-null),
// so the backward pass can quantize the same values; the quantization of H
// is the one above, byte for byte.

// FASTDIV (ablation only, not the method): every division of the row
// quantizer -- A / 2688, 448 a_b / A and x / d_b -- is replaced by the
// hardware reciprocal approximation times the numerator (v_rcp_f32, then
// v_mul_f32), the kind of fast divide the report warns against for NVFP4.
// Used to count the codes such a divide changes.
__device__ __forceinline__ float rcp_approx(float b) {
    asm volatile("" : "+v"(b));  // keep the reciprocal a run-time instruction
    return __builtin_amdgcn_rcpf(b);
}

// Encode one row whose 16-element blocks lane + 64 i (i < BPL, block < nb)
// this lane holds in v (16 bf16 each); bmax are the blocks' |x| maxima
// (bf16 bit patterns) and rmax this lane's maximum over them.  Writes the
// row's codes cr[cols/2], block scales br[nb] and row scale *rs.
// Scale byte of a 16-element block with |x| maximum amax_b (bf16 bits) in a
// row with |x| maximum A > 0: S_b = E4M3_RNE(RN32(448 * a_b / A)).  The
// numerator and denominator are exact; for a_b > 2^119, where 448*a_b could
// overflow, both are scaled by 2^-9 (0.875*a_b and A*2^-9: exact, finite,
// same quotient).  The quotient is RN32(num * RN64(1 / den)), as for x / d_b
// below; invA = RN64(1 / A) is computed once per row, and RN64(1 / (A 2^-9))
// = invA * 2^9 exactly.
template <bool FASTDIV>
__device__ __forceinline__ uint32_t nvfp4v_block_scale(uint32_t amax_b, float A, double invA) {
    const float ab = __uint_as_float(amax_b << 16);
    const bool big = ab > 0x1p119f;
    const float num = big ? 0.875f * ab : 448.0f * ab;
    float t;
    if constexpr (FASTDIV)
        t = num * rcp_approx(big ? A * 0x1p-9f : A);
    else
        t = (float)((double)num * (big ? invA * 0x1p9 : invA));  // in [0, 448]
    return __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(t, 448.0f, -448.0f), 0.0f, 0, false) & 0xFFu;
}

// E2M1 codes (8 bytes) of one 16-element block with scale byte S in a row
// with decode scale s_row: d_b = RN32(S_b * s_row), code = E2M1(RN32(x / d_b))
// (all zero when d_b == 0).
template <bool FASTDIV>
__device__ __forceinline__ uint2 nvfp4v_block_codes(const uint4 (&v)[2], uint32_t S, float s_row) {
    const float d = __builtin_amdgcn_cvt_f32_fp8((int)S, 0) * s_row;  // exact E4M3 value
    uint2 out = make_uint2(0, 0);
    if (d != 0.0f) {
        float q[16];
        const uint32_t w[8] = {v[0].x, v[0].y, v[0].z, v[0].w, v[1].x, v[1].y, v[1].z, v[1].w};
        if constexpr (FASTDIV) {
            const float r = rcp_approx(d);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                q[2 * j] = bf16_lo(w[j]) * r;
                q[2 * j + 1] = bf16_hi(w[j]) * r;
            }
        } else {
            const double inv = 1.0 / (double)d;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                q[2 * j] = (float)((double)bf16_lo(w[j]) * inv);
                q[2 * j + 1] = (float)((double)bf16_hi(w[j]) * inv);
            }
        }
        uint32_t c0 = e2m1x2<0>(0u, q[0], q[1]);
        c0 = e2m1x2<1>(c0, q[2], q[3]);
        c0 = e2m1x2<2>(c0, q[4], q[5]);
        c0 = e2m1x2<3>(c0, q[6], q[7]);
        uint32_t c1 = e2m1x2<0>(0u, q[8], q[9]);
        c1 = e2m1x2<1>(c1, q[10], q[11]);
        c1 = e2m1x2<2>(c1, q[12], q[13]);
        c1 = e2m1x2<3>(c1, q[14], q[15]);
        out = make_uint2(c0, c1);
    }
    return out;
}

// The row's decode scale from the wave-wide |x| maximum rmax (bf16 bits):
// s_row = RN32(A / 2688) (0 for an all-zero row, whose outputs are all zero).
template <bool FASTDIV>
__device__ __forceinline__ float nvfp4v_row_scale(uint32_t rmax) {
    const float A = __uint_as_float(rmax << 16);
    return rmax == 0 ? 0.0f : (FASTDIV ? A * rcp_approx(2688.0f) : A / 2688.0f);  // IEEE binary32 division
}

// Encode one row whose 16-element blocks lane + 64 i (i < BPL, block < nb)
// this lane holds in v (16 bf16 each); bmax are the blocks' |x| maxima
// (bf16 bit patterns) and rmax this lane's maximum over them.  Writes the
// row's codes cr[cols/2], block scales br[nb] and row scale *rs.
template <int BPL, bool FASTDIV>
__device__ __forceinline__ void nvfp4v_encode_row(const uint4 (&v)[BPL][2], const uint32_t (&bmax)[BPL], uint32_t rmax,
                                                  int nb, int lane, uint8_t* __restrict__ cr,
                                                  uint8_t* __restrict__ br, float* __restrict__ rs) {
    rmax = wave_max_u32(rmax);
    const float s_row = nvfp4v_row_scale<FASTDIV>(rmax);
    if (lane == 0) *rs = s_row;
    const float A = __uint_as_float(rmax << 16);
    const double invA = FASTDIV || !rmax ? 0.0 : 1.0 / (double)A;
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
        const int b = lane + 64 * i;
        if (b >= nb) continue;
        const uint32_t S = rmax ? nvfp4v_block_scale<FASTDIV>(bmax[i], A, invA) : 0u;
        br[b] = (uint8_t)S;
        st_stream8(cr + 8 * b, rmax ? nvfp4v_block_codes<FASTDIV>(v[i], S, s_row) : make_uint2(0, 0));
    }
}


template <int BPL, bool SWIGLU, bool FASTDIV = false>
__global__ __launch_bounds__(256) void k_quantize_nvfp4v(const uint16_t* __restrict__ x, int64_t rows,
                                                         int cols, int64_t ldx, uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ bscale,
                                                         float* __restrict__ rscale, uint16_t* __restrict__ h,
                                                         int64_t ldh) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int nb = cols >> 4;
    const uint16_t* xr = x + row * ldx;

    uint4 v[BPL][2];
    uint32_t bmax[BPL];
    uint32_t rmax = 0;
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
        const int b = lane + 64 * i;
        if (b < nb) {
            const uint4* p = reinterpret_cast<const uint4*>(xr + 16 * b);
            v[i][0] = ld_stream16(p);
            v[i][1] = ld_stream16(p + 1);
            if constexpr (SWIGLU) {
                const uint4* pu = reinterpret_cast<const uint4*>(xr + cols + 16 * b);
                const uint4 u0 = ld_stream16(pu), u1 = ld_stream16(pu + 1);
                v[i][0] = make_uint4(swiglu_pair(v[i][0].x, u0.x), swiglu_pair(v[i][0].y, u0.y),
                                     swiglu_pair(v[i][0].z, u0.z), swiglu_pair(v[i][0].w, u0.w));
                v[i][1] = make_uint4(swiglu_pair(v[i][1].x, u1.x), swiglu_pair(v[i][1].y, u1.y),
                                     swiglu_pair(v[i][1].z, u1.z), swiglu_pair(v[i][1].w, u1.w));
                if (h) {
                    uint4* ph = reinterpret_cast<uint4*>(h + row * ldh + 16 * b);
                    st_stream16(ph, v[i][0]);
                    st_stream16(ph + 1, v[i][1]);
                }
            }
        } else {
            v[i][0] = make_uint4(0, 0, 0, 0);
            v[i][1] = make_uint4(0, 0, 0, 0);
        }
        uint32_t m = 0;
        m = absmax2_bf16(m, v[i][0].x); m = absmax2_bf16(m, v[i][0].y);
        m = absmax2_bf16(m, v[i][0].z); m = absmax2_bf16(m, v[i][0].w);
        m = absmax2_bf16(m, v[i][1].x); m = absmax2_bf16(m, v[i][1].y);
        m = absmax2_bf16(m, v[i][1].z); m = absmax2_bf16(m, v[i][1].w);
        bmax[i] = fold_max16(m);
        rmax = max(rmax, bmax[i]);
    }
    uint8_t* cr = codes + row * (int64_t)(cols >> 1);
    uint8_t* br = bscale + row * (int64_t)nb;
    nvfp4v_encode_row<BPL, FASTDIV>(v, bmax, rmax, nb, lane, cr, br, rscale + row);
}

// ---------------------------------------------------------------- MXFP8

struct MxBlock {
    uint4 c0, c1;   // 32 E4M3 codes
    uint32_t sbyte; // E8M0
};

// Encode one block of 32 values given as 16 bf16 pairs.  Each pair goes
// through v_cvt_scalef32_pk_fp8_bf16, which divides by a power-of-two scale
// and rounds to E4M3 (nearest even) -- exact, since the scale is a power of
// two -- but turns results past 448 into NaN instead of saturating, so the
// bf16 magnitudes are first clamped to 448 * 2^sh on their bit patterns
// (one unsigned and one signed packed 16-bit min: bf16 is sign-magnitude).
// The instruction's behaviour (byte order, word select, every bf16 pattern
// at scales 2^-127 .. 2^127) was checked against the definition on the GPU.
__device__ __forceinline__ MxBlock mx_encode(const uint32_t (&w)[16]) {
    typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
    typedef int16_t i16x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef short s16x2 __attribute__((ext_vector_type(2)));
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) m = absmax2_bf16(m, w[j]);
    m = fold_max16(m);
    MxBlock r;
    if (m == 0) {
        r.c0 = make_uint4(0, 0, 0, 0);
        r.c1 = make_uint4(0, 0, 0, 0);
        r.sbyte = 0;
        return r;
    }
    // floor(log2 A) from the bf16 exponent field; any subnormal A gives a
    // shared exponent below -127, which clamps to -127.
    const int biased = (int)(m >> 7);  // sign bit is clear
    const int e = biased ? biased - 127 : -127;
    const int sh = min(max(e - 8, -127), 127);
    r.sbyte = (uint32_t)(sh + 127);
    // 448 * 2^sh as bf16 bits (finite inputs give sh <= 119), and 2^sh as the
    // fp32 scale (2^-127 is subnormal)
    const uint32_t T = ((uint32_t)(sh + 135) << 7) | 0x60u;
    const u16x2 tu = {(uint16_t)(T | 0x8000u), (uint16_t)(T | 0x8000u)};
    const i16x2 ti = {(int16_t)T, (int16_t)T};
    const float scale = __uint_as_float(sh > -127 ? (uint32_t)(sh + 127) << 23 : 0x00400000u);
    auto clamp2 = [&](uint32_t x) -> bf16x2 {
        // negative values keep their sign bit through the unsigned min and are
        // below T as signed; positive ones pass the unsigned min unchanged
        const u16x2 a = __builtin_elementwise_min(__builtin_bit_cast(u16x2, x), tu);
        return __builtin_bit_cast(bf16x2, __builtin_elementwise_min(__builtin_bit_cast(i16x2, a), ti));
    };
    uint32_t out[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        s16x2 o = {0, 0};
        o = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(o, clamp2(w[2 * j]), scale, false);
        o = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(o, clamp2(w[2 * j + 1]), scale, true);
        out[j] = __builtin_bit_cast(uint32_t, o);
    }
    r.c0 = make_uint4(out[0], out[1], out[2], out[3]);
    r.c1 = make_uint4(out[4], out[5], out[6], out[7]);
    return r;
}

// Row-wise MXFP8.  A workgroup owns 32 rows x 32 blocks (1024 columns) --
// small enough that the grid (3584 workgroups for 16384 x 7168) spreads
// evenly over the compute units;
// neighbouring threads take neighbouring blocks of a row (64-byte loads and
// 32-byte code stores, contiguous across a wave).  Scales are block-major, so
// a thread's scale byte is `rows` bytes away from its neighbour's: the bytes
// are gathered in LDS as [block][row] and leave as one 32-byte run per block
// (16-byte stores when every run is 16-byte aligned, bytes otherwise).
constexpr int MXR_ROWS = 32;
constexpr int MXR_BLK = 32;
constexpr int MXR_PITCH = MXR_ROWS + 8;  // bytes per block row in LDS (bank spread)

// GATHER: output row r quantizes source row row_index[r] of x (src_rows
// rows): the token permutation of an expert dispatch fused into the
// quantizer; an index outside [0, src_rows) reads as a zero row.
template <bool ALIGNED16, bool GATHER>
__global__ __launch_bounds__(256) void k_quantize_mxfp8_rowwise(const uint16_t* __restrict__ x, int64_t rows,
                                                                int cols, int64_t ldx,
                                                                uint8_t* __restrict__ codes,
                                                                uint8_t* __restrict__ scale,
                                                                const int32_t* __restrict__ row_index,
                                                                int64_t src_rows) {
    __shared__ __align__(16) uint8_t sb[MXR_BLK * MXR_PITCH];
    const int nb = cols >> 5;
    const int nbt = (nb + MXR_BLK - 1) / MXR_BLK;
    const int64_t r0 = (int64_t)(blockIdx.x / nbt) * MXR_ROWS;
    const int b0 = (int)(blockIdx.x % nbt) * MXR_BLK;
    const int t = threadIdx.x;
    const int bl = t & 31;       // block within the tile
    const int b = b0 + bl;
    // Row offsets are relative to the tile's first row: 128 * ldx * 2 bytes
    // stay below 2^31 (host check).  Rows past the end and blocks past the
    // row read as zero and are not stored.
    // (GATHER: offsets from x itself, src_rows * ldx * 2 < 2^31 by a host check)
    const __amdgpu_buffer_rsrc_t rx = GATHER ? make_rsrc(x, (uint32_t)(src_rows * ldx * 2))
                                             : make_rsrc(uniform_ptr(x + r0 * ldx), 0x7FFFFFFFu);
    const bool okb = b < nb;
#pragma unroll 1
    for (int it = 0; it < MXR_ROWS / 8; it += 4) {
        // four rows of this thread's block in flight at once
        uint32_t w[4][16];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int rl = 8 * (it + u) + (t >> 5);
            bool ok = okb & (r0 + rl < rows);
            uint32_t off;
            if constexpr (GATHER) {
                const int64_t src = ok ? (int64_t)row_index[r0 + rl] : -1;
                ok &= (src >= 0) & (src < src_rows);
                off = (uint32_t)((src * ldx + 32 * b) * 2);
            } else {
                off = (uint32_t)(((int64_t)rl * ldx + 32 * b) * 2);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint4 v = buf_load16(rx, ok ? off + 16u * q : OOB);
                w[u][4 * q] = v.x; w[u][4 * q + 1] = v.y; w[u][4 * q + 2] = v.z; w[u][4 * q + 3] = v.w;
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int rl = 8 * (it + u) + (t >> 5);
            const int64_t row = r0 + rl;
            const MxBlock r = mx_encode(w[u]);
            if (okb & (row < rows)) {
                uint4* o = reinterpret_cast<uint4*>(codes + row * (int64_t)cols + 32 * b);
                st_stream16(o, r.c0);
                st_stream16(o + 1, r.c1);
                sb[bl * MXR_PITCH + rl] = (uint8_t)r.sbyte;
            }
        }
    }
    __syncthreads();
    // block bl2 = t / CPB leaves as bytes [16 * (t % CPB), +16) of its run of
    // MXR_ROWS rows
    constexpr int CPB = MXR_ROWS / 16;
    if (t >= MXR_BLK * CPB) return;
    const int bl2 = t / CPB, q = t % CPB;
    const int bb = b0 + bl2;
    const int64_t rr = r0 + 16 * q;
    if (bb >= nb || rr >= rows) return;
    uint8_t* dst = scale + (int64_t)bb * rows + rr;
    const uint8_t* src = &sb[bl2 * MXR_PITCH + 16 * q];
    if (ALIGNED16 && rr + 16 <= rows) {
        const uint2 lo = *reinterpret_cast<const uint2*>(src);
        const uint2 hi = *reinterpret_cast<const uint2*>(src + 8);
        *reinterpret_cast<uint4*>(dst) = make_uint4(lo.x, lo.y, hi.x, hi.y);
    } else {
        const int n = (int)min((int64_t)16, rows - rr);
        for (int k = 0; k < n; ++k) dst[k] = src[k];
    }
}

// Column-transposing MXFP8 per group.  A workgroup owns 128 padded output
// columns (four 32-blocks of tokens) x 128 channels.  Block b of the tile is
// padded column range [p0 + 32b, +32) = tokens [m0_b, m0_b + n_b) of one
// group (n_b < 32 at a group's end, 0 in padding; groups start on multiples
// of 128 columns, so all four blocks belong to the same group).  The bf16 tile
// [128 token slots][128 channels] (256-byte rows, 32 KB) arrives through
// buffer-to-LDS DMA, slots past n_b as zeros.  Thread (pair p, block b) then
// encodes channels 2p and 2p+1 of block b from 32 dword reads (one token row
// per read, a wave covering one row: conflict-free) and writes each channel's
// 32 codes as two 16-byte stores; the 4 blocks of a channel form one
// contiguous 128-byte run of codes[channel][p0 .. p0+128).  Workgroups that
// are neighbours in launch order take neighbouring channel tiles of the same
// token rows.
constexpr int COLT_TOK = 128;
constexpr int COLT_CH = 128;

// Group of padded column pc: the last g with start(g) = 128 * (g + off[g]/128)
// <= pc (starts strictly increase).  Wave-wide 64-ary search: one round of
// loads for up to 64 groups.  Returns the group; lane l's (start, off) of
// group base + l come back through `base`, `st`, `of0`, `of1` for the caller.
__device__ __forceinline__ int colt_find_base(const int32_t* __restrict__ offsets, int ngroups, int64_t pc, int lane) {
    int lo = 0, n = ngroups;
    while (n > 64) {
        const int step = (n + 63) / 64;
        const int g = lo + lane * step;
        const bool le = (g < lo + n) && (128 * ((int64_t)g + offsets[g] / 128) <= pc);
        const int cnt = __builtin_popcountll(__ballot(le));
        const int nlo = lo + max(cnt - 1, 0) * step;
        n = min(step, lo + n - nlo);
        lo = nlo;
    }
    const int g = lo + lane;
    const bool le = (g < lo + n) && (128 * ((int64_t)g + offsets[g] / 128) <= pc);
    return lo + max(__builtin_popcountll(__ballot(le)) - 1, 0);
}

// DUAL: the same pass also writes the ROWWISE quantization (blocks of 32
// channels along each token row, codes rcodes [rows][cols], block-major
// scales rscale [cols/32][rows]) of the tile's tokens from the LDS tile, so
// a tensor that needs both layouts is read once.
//
// The tile holds token rows of 128 channels (256 bytes); 16-byte chunk k of
// tile row r sits at chunk position k ^ (r & 15), so both the column reads
// (one channel pair across rows) and the row reads (16 consecutive rows at
// one chunk) spread over all banks.
template <bool DUAL>
__global__ __launch_bounds__(256) void k_quantize_mxfp8_colwise_t(
    const uint16_t* __restrict__ x, int64_t rows, int cols, int64_t ldx, const int32_t* __restrict__ offsets,
    int ngroups, int64_t P, uint8_t* __restrict__ codes, uint8_t* __restrict__ scale,
    uint8_t* __restrict__ rcodes, uint8_t* __restrict__ rscale) {
    // exactly 32 KB of LDS, so five workgroups fit a CU
    __shared__ __align__(16) uint8_t tile[COLT_TOK * COLT_CH * 2];
    int64_t blk_m0[4];
    int blk_n[4];
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    // launch order: channel tile fastest, so concurrently running workgroups
    // read neighbouring parts of the same token rows
    const int nct = (cols + COLT_CH - 1) / COLT_CH;
    const int64_t p0 = (int64_t)(blockIdx.x / nct) * COLT_TOK;
    const int c_base = (int)(blockIdx.x % nct) * COLT_CH;

    {
        // every wave finds the segments of the tile's 4 blocks itself (wave-
        // uniform results): group starts are multiples of 128, so the 4 blocks
        // of a tile lie in one group's span, found from p0; with at most 61
        // groups the window starting at group 0 holds them all and one round
        // of loads does
        const int g0 = ngroups <= 61 ? 0 : __builtin_amdgcn_readfirstlane(colt_find_base(offsets, ngroups, p0, lane));
        const int g = g0 + lane;
        const bool have = g < ngroups;
        const int32_t of0 = have ? offsets[g] : 0;
        const int32_t of1 = have ? offsets[g + 1] : 0;
        const int64_t st = 128 * ((int64_t)g + of0 / 128);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int64_t pc = p0 + 32 * b;
            const int k = max(__builtin_popcountll(__ballot(have && st <= pc)) - 1, 0);
            const int64_t stk = 128 * ((int64_t)(g0 + k) + __builtin_amdgcn_readlane(of0, k) / 128);
            const int64_t mb = __builtin_amdgcn_readlane(of0, k) + (pc - stk);
            // segment bounds clamped to the input's rows, so offsets that break
            // the precondition still never read or write outside the tensors
            const int64_t end = min((int64_t)__builtin_amdgcn_readlane(of1, k), rows);
            const bool ok = pc < P && mb >= 0 && mb < end;
            blk_m0[b] = uniform_i64(ok ? mb : 0);
            blk_n[b] = __builtin_amdgcn_readfirstlane(ok ? (int)min((int64_t)32, end - mb) : 0);
        }
    }

    // DMA: instruction i of this wave covers tile rows 4 * (8 * wave + i) + lane / 16,
    // 16 bytes (8 channels) per lane.  Offsets are taken from the first token
    // of the tile, so they stay below 2^31 (host check: 258 * ldx < 2^31).
    {
        // first token of the tile: blocks run in token order, so the first
        // block holding tokens has the smallest m0
        int64_t mlo = 0;
#pragma unroll
        for (int b = 3; b >= 0; --b) mlo = blk_n[b] > 0 ? blk_m0[b] : mlo;
        mlo = uniform_i64(mlo);
        const i32x4 d = make_desc(uniform_ptr(x + mlo * ldx));
        const uint32_t L = __builtin_amdgcn_readfirstlane(lds_addr(tile));
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int ins = 8 * wave + i;
            // tile row 4 * ins + lane / 16 = 32 * wave + ii: block `wave`;
            // the lane's LDS slot lane & 15 receives chunk (lane & 15) ^ (ii & 15)
            const int ii = 4 * i + (lane >> 4);
            const int ch = c_base + 8 * ((lane & 15) ^ (ii & 15));
            int64_t m0w = blk_m0[0];
            int nw = blk_n[0];
#pragma unroll
            for (int q = 1; q < 4; ++q) {
                if (wave == q) { m0w = blk_m0[q]; nw = blk_n[q]; }
            }
            const bool ok = (ii < nw) & (ch < cols);
            const uint32_t off = (uint32_t)(((m0w - mlo + ii) * ldx + ch) * 2);
            dma16(d, ok ? off : OOB, L + 1024u * (uint32_t)ins);
        }
        wait_vmcnt<0>();
        __syncthreads();
    }

    const int pr = t & 63, b = t >> 6;  // channel pair, block (one block per wave)
    const int64_t pc = p0 + 32 * b;
    const int c = c_base + 2 * pr;
    const bool active = pc < P && c < cols;
    MxBlock e0, e1;
    if (active) {
        uint32_t w0[16], w1[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            // pair pr is dword pr & 3 of logical chunk pr >> 2; rows 2j and 2j+1 of the block
            const uint32_t o0 = (uint32_t)(((pr >> 2) ^ ((2 * j) & 15)) * 16 + (pr & 3) * 4);
            const uint32_t o1 = (uint32_t)(((pr >> 2) ^ ((2 * j + 1) & 15)) * 16 + (pr & 3) * 4);
            const uint32_t r0 = *reinterpret_cast<const uint32_t*>(&tile[(32 * b + 2 * j) * 256 + o0]);
            const uint32_t r1 = *reinterpret_cast<const uint32_t*>(&tile[(32 * b + 2 * j + 1) * 256 + o1]);
            w0[j] = __builtin_amdgcn_perm(r1, r0, 0x05040100u);  // low halves: channel 2p, tokens 2j, 2j+1
            w1[j] = __builtin_amdgcn_perm(r1, r0, 0x07060302u);  // high halves: channel 2p+1
        }
        e0 = mx_encode(w0);
        e1 = mx_encode(w1);
        uint8_t* sp = scale + (pc >> 5) * cols + c;  // block-major: coalesced across channels
        sp[0] = (uint8_t)e0.sbyte;
        sp[1] = (uint8_t)e1.sbyte;
    }
    if constexpr (DUAL) {
        // row blocks: lane l of wave w takes tile row r = 32 w + (l & 31)
        // (token blk_m0[w] + (l & 31) when the block holds one) and the
        // 32-channel blocks h, h + 2 with h = l / 32: the two half-waves
        // write neighbouring 32-byte pieces of a row, and 16 lanes that read
        // LDS together take 16 rows, so the chunk swizzle keeps them apart
        const int ii = lane & 31, h = lane >> 5, r = 32 * wave + ii;
        int64_t m0w = blk_m0[0];
        int nw = blk_n[0];
#pragma unroll
        for (int q = 1; q < 4; ++q) {
            if (wave == q) { m0w = blk_m0[q]; nw = blk_n[q]; }
        }
        if (ii < nw) {
            const int64_t m = m0w + ii;
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
                const int cb = h + 2 * jb;
                const int cc = c_base + 32 * cb;
                if (cc >= cols) continue;
                uint32_t wv[16];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint4 u = *reinterpret_cast<const uint4*>(&tile[r * 256 + (((4 * cb + q) ^ (r & 15)) * 16)]);
                    wv[4 * q] = u.x; wv[4 * q + 1] = u.y; wv[4 * q + 2] = u.z; wv[4 * q + 3] = u.w;
                }
                const MxBlock eb = mx_encode(wv);
                uint4* o = reinterpret_cast<uint4*>(rcodes + m * (int64_t)cols + cc);
                o[0] = eb.c0;
                o[1] = eb.c1;
                rscale[(int64_t)(cc >> 5) * rows + m] = (uint8_t)eb.sbyte;
            }
        }
    }
    // The codes leave through LDS as whole 128-byte rows (one channel, the
    // tile's 128 tokens): output row r keeps its eight 16-byte chunks at
    // chunk ^ ((r >> 1) & 7), which spreads the eight rows a group of lanes
    // writes (rows 2p, p = 8k .. 8k+7) over all banks.
    __syncthreads();  // every wave is done reading the input tile
    uint8_t* otile = tile;
    if (active) {
        const int r0 = 2 * pr;
        const int sw = pr & 7;  // (r >> 1) & 7 for rows 2p and 2p+1
        *reinterpret_cast<uint4*>(&otile[r0 * 128 + (((2 * b) ^ sw) * 16)]) = e0.c0;
        *reinterpret_cast<uint4*>(&otile[r0 * 128 + (((2 * b + 1) ^ sw) * 16)]) = e0.c1;
        *reinterpret_cast<uint4*>(&otile[(r0 + 1) * 128 + (((2 * b) ^ sw) * 16)]) = e1.c0;
        *reinterpret_cast<uint4*>(&otile[(r0 + 1) * 128 + (((2 * b + 1) ^ sw) * 16)]) = e1.c1;
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int id = it * 256 + t;         // 128 rows x 8 chunks
        const int r = id >> 3, part = id & 7;
        const int64_t pp = p0 + 16 * part;   // first token of the chunk
        if (pp < P && c_base + r < cols) {
            const uint4 v = *reinterpret_cast<const uint4*>(&otile[r * 128 + ((part ^ ((r >> 1) & 7)) * 16)]);
            *reinterpret_cast<uint4*>(codes + (int64_t)(c_base + r) * P + pp) = v;
        }
    }
}

// ------------------------------------------------------- debug encoders

__global__ void k_debug_e2m1(const float* __restrict__ in, uint8_t* __restrict__ out, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) out[i] = (uint8_t)(e2m1x2<0>(0u, in[i], 0.0f) & 15u);
}

__global__ void k_debug_e4m3(const float* __restrict__ in, uint8_t* __restrict__ out, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) out[i] = (uint8_t)(e4m3x4(in[i], 0.0f, 0.0f, 0.0f) & 0xFFu);
}

// ---------------------------------------------------------------- launchers

// A dispatch counts its work-items in 32 bits: at most 2^24 - 1 workgroups of
// 256 threads.
constexpr int64_t kMaxWorkgroups = ((int64_t)1 << 24) - 1;

template <bool SWIGLU, bool FASTDIV = false>
static hipError_t launch_nvfp4v(const uint16_t* x, int64_t rows, int cols, int64_t ldx, uint8_t* codes,
                                uint8_t* bscale, float* rscale, uint16_t* h, int64_t ldh, hipStream_t s) {
    const int nb = cols / 16;
    if ((rows + 3) / 4 > kMaxWorkgroups) return hipErrorInvalidValue;  // beyond the host-checked sizes
    const dim3 grid((unsigned)((rows + 3) / 4));
#define BSQ_NVFP4V_LAUNCH(BPL)                                                                       \
    hipLaunchKernelGGL((k_quantize_nvfp4v<BPL, SWIGLU, FASTDIV>), grid, dim3(256), 0, s, x, rows, cols, \
                       ldx, codes, bscale, rscale, h, ldh)
    if (nb <= 64)
        BSQ_NVFP4V_LAUNCH(1);
    else if (nb <= 128)
        BSQ_NVFP4V_LAUNCH(2);
    else if (nb <= 256)
        BSQ_NVFP4V_LAUNCH(4);
    else if (nb <= 512)
        BSQ_NVFP4V_LAUNCH(8);
    else if (nb <= 1024)
        BSQ_NVFP4V_LAUNCH(16);
    else
        return hipErrorInvalidValue;  // rejected by the host checks (cols > 16384)
#undef BSQ_NVFP4V_LAUNCH
    return hipGetLastError();
}

hipError_t launch_quantize_nvfp4v(const uint16_t* x, int64_t rows, int cols, int64_t ldx, uint8_t* codes,
                                  uint8_t* bscale, float* rscale, hipStream_t s) {
    return launch_nvfp4v<false>(x, rows, cols, ldx, codes, bscale, rscale, nullptr, 0, s);
}

hipError_t launch_quantize_nvfp4v_fastdiv(const uint16_t* x, int64_t rows, int cols, int64_t ldx, uint8_t* codes,
                                          uint8_t* bscale, float* rscale, hipStream_t s) {
    return launch_nvfp4v<false, true>(x, rows, cols, ldx, codes, bscale, rscale, nullptr, 0, s);
}

hipError_t launch_swiglu_quantize_nvfp4v(const uint16_t* gu, int64_t rows, int inter, int64_t ldgu, uint16_t* h,
                                         int64_t ldh, uint8_t* codes, uint8_t* bscale, float* rscale,
                                         hipStream_t s) {
    return launch_nvfp4v<true>(gu, rows, inter, ldgu, codes, bscale, rscale, h, ldh, s);
}

template <bool GATHER>
static hipError_t launch_mxfp8_rowwise(const uint16_t* x, int64_t rows, int cols, int64_t ldx, uint8_t* codes,
                                       uint8_t* scale, const int32_t* row_index, int64_t src_rows, hipStream_t s) {
    const int nbt = (cols / 32 + MXR_BLK - 1) / MXR_BLK;
    const int64_t nwg = ((rows + MXR_ROWS - 1) / MXR_ROWS) * nbt;
    if (nwg >= kMaxWorkgroups) return hipErrorInvalidValue;
    const bool a16 = (rows % 16 == 0) && ((reinterpret_cast<uintptr_t>(scale) & 15) == 0);
    if (a16)
        hipLaunchKernelGGL((k_quantize_mxfp8_rowwise<true, GATHER>), dim3((unsigned)nwg), dim3(256), 0, s, x, rows,
                           cols, ldx, codes, scale, row_index, src_rows);
    else
        hipLaunchKernelGGL((k_quantize_mxfp8_rowwise<false, GATHER>), dim3((unsigned)nwg), dim3(256), 0, s, x, rows,
                           cols, ldx, codes, scale, row_index, src_rows);
    return hipGetLastError();
}

hipError_t launch_quantize_mxfp8_rowwise(const uint16_t* x, int64_t rows, int cols, int64_t ldx, uint8_t* codes,
                                         uint8_t* scale, hipStream_t s) {
    return launch_mxfp8_rowwise<false>(x, rows, cols, ldx, codes, scale, nullptr, 0, s);
}

hipError_t launch_quantize_mxfp8_gather(const uint16_t* x, int64_t src_rows, int cols, int64_t ldx,
                                        const int32_t* row_index, int64_t rows, uint8_t* codes, uint8_t* scale,
                                        hipStream_t s) {
    return launch_mxfp8_rowwise<true>(x, rows, cols, ldx, codes, scale, row_index, src_rows, s);
}

hipError_t launch_quantize_mxfp8_colwise_t(const uint16_t* x, int64_t rows, int cols, int64_t ldx,
                                           const int32_t* offsets, int ngroups, int64_t P, uint8_t* codes,
                                           uint8_t* scale, hipStream_t s) {
    const int64_t nwg = (int64_t)((cols + COLT_CH - 1) / COLT_CH) * ((P + COLT_TOK - 1) / COLT_TOK);
    if (nwg >= kMaxWorkgroups) return hipErrorInvalidValue;  // beyond the host-checked sizes
    const dim3 grid((unsigned)nwg);
    hipLaunchKernelGGL(k_quantize_mxfp8_colwise_t<false>, grid, dim3(256), 0, s, x, rows, cols, ldx, offsets,
                       ngroups, P, codes, scale, nullptr, nullptr);
    return hipGetLastError();
}

hipError_t launch_quantize_mxfp8_dual(const uint16_t* x, int64_t rows, int cols, int64_t ldx, const int32_t* offsets,
                                      int ngroups, int64_t P, uint8_t* t_codes, uint8_t* t_scale, uint8_t* r_codes,
                                      uint8_t* r_scale, hipStream_t s) {
    const int64_t nwg = (int64_t)((cols + COLT_CH - 1) / COLT_CH) * ((P + COLT_TOK - 1) / COLT_TOK);
    if (nwg >= kMaxWorkgroups) return hipErrorInvalidValue;
    const dim3 grid((unsigned)nwg);
    hipLaunchKernelGGL(k_quantize_mxfp8_colwise_t<true>, grid, dim3(256), 0, s, x, rows, cols, ldx, offsets,
                       ngroups, P, t_codes, t_scale, r_codes, r_scale);
    return hipGetLastError();
}

hipError_t launch_debug_encode(int which, const float* in, uint8_t* out, int64_t n, hipStream_t s) {
    if ((n + 255) / 256 > kMaxWorkgroups) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((n + 255) / 256));
    if (which == 0)
        hipLaunchKernelGGL(k_debug_e2m1, grid, dim3(256), 0, s, in, out, n);
    else
        hipLaunchKernelGGL(k_debug_e4m3, grid, dim3(256), 0, s, in, out, n);
    return hipGetLastError();
}

}  // namespace bsq
