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
template <int BPL>
__global__ __launch_bounds__(256) void k_quantize_nvfp4v(const uint16_t* __restrict__ x, int64_t rows,
                                                         int cols, int64_t ldx, uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ bscale,
                                                         float* __restrict__ rscale) {
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
        } else {
            v[i][0] = make_uint4(0, 0, 0, 0);
            v[i][1] = make_uint4(0, 0, 0, 0);
        }
        uint32_t m = 0;
        m = absmax_bf16x2(m, v[i][0].x); m = absmax_bf16x2(m, v[i][0].y);
        m = absmax_bf16x2(m, v[i][0].z); m = absmax_bf16x2(m, v[i][0].w);
        m = absmax_bf16x2(m, v[i][1].x); m = absmax_bf16x2(m, v[i][1].y);
        m = absmax_bf16x2(m, v[i][1].z); m = absmax_bf16x2(m, v[i][1].w);
        bmax[i] = m;
        rmax = max(rmax, m);
    }
    rmax = wave_max_u32(rmax);

    uint8_t* cr = codes + row * (int64_t)(cols >> 1);
    uint8_t* br = bscale + row * (int64_t)nb;
    if (rmax == 0) {  // all-zero row: zero scale, zero codes
#pragma unroll
        for (int i = 0; i < BPL; ++i) {
            const int b = lane + 64 * i;
            if (b < nb) {
                *reinterpret_cast<uint2*>(cr + 8 * b) = make_uint2(0, 0);
                br[b] = 0;
            }
        }
        if (lane == 0) rscale[row] = 0.0f;
        return;
    }
    const float A = __uint_as_float(rmax << 16);
    const float s_row = A / 2688.0f;  // IEEE binary32 division
    if (lane == 0) rscale[row] = s_row;

#pragma unroll
    for (int i = 0; i < BPL; ++i) {
        const int b = lane + 64 * i;
        if (b >= nb) continue;
        // t_b = RN32(448 * a_b / A): numerator and denominator exact; for
        // a_b > 2^119 both are scaled by 2^-8 to keep 448*a_b finite.
        const float ab = __uint_as_float(bmax[i] << 16);
        float num, den;
        if (ab <= 0x1p119f) { num = 448.0f * ab; den = A; }
        else                { num = 1.75f * ab;  den = A * 0x1p-8f; }
        const float t = num / den;  // in [0, 448]
        const uint32_t S = e4m3x4(t, 0.0f, 0.0f, 0.0f) & 0xFFu;
        br[b] = (uint8_t)S;
        const float d = e4m3_value(S) * s_row;
        uint2 out = make_uint2(0, 0);
        if (d != 0.0f) {
            const double inv = 1.0 / (double)d;
            float q[16];
            const uint32_t w[8] = {v[i][0].x, v[i][0].y, v[i][0].z, v[i][0].w,
                                   v[i][1].x, v[i][1].y, v[i][1].z, v[i][1].w};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                q[2 * j] = (float)((double)bf16_lo(w[j]) * inv);
                q[2 * j + 1] = (float)((double)bf16_hi(w[j]) * inv);
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
        *reinterpret_cast<uint2*>(cr + 8 * b) = out;
    }
}

// ---------------------------------------------------------------- MXFP8

struct MxBlock {
    uint4 c0, c1;   // 32 E4M3 codes
    uint32_t sbyte; // E8M0
};

// Encode one block of 32 floats given as 16 bf16 pairs.
__device__ __forceinline__ MxBlock mx_encode(const uint32_t (&w)[16]) {
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) m = absmax_bf16x2(m, w[j]);
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
    uint32_t out[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        // x * 2^-sh is exact except for results far below E4M3's smallest
        // subnormal, which encode to (signed) zero either way.
        out[j] = e4m3x4(__builtin_ldexpf(bf16_lo(w[2 * j]), -sh), __builtin_ldexpf(bf16_hi(w[2 * j]), -sh),
                        __builtin_ldexpf(bf16_lo(w[2 * j + 1]), -sh),
                        __builtin_ldexpf(bf16_hi(w[2 * j + 1]), -sh));
    }
    r.c0 = make_uint4(out[0], out[1], out[2], out[3]);
    r.c1 = make_uint4(out[4], out[5], out[6], out[7]);
    return r;
}

// Row-wise MXFP8: one thread per 32-element block; neighbouring threads take
// neighbouring blocks of a row (64-byte loads, 32-byte stores, contiguous).
__global__ __launch_bounds__(256) void k_quantize_mxfp8_rowwise(const uint16_t* __restrict__ x, int64_t rows,
                                                                int cols, int64_t ldx,
                                                                uint8_t* __restrict__ codes,
                                                                uint8_t* __restrict__ scale) {
    const int nb = cols >> 5;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gid >= rows * nb) return;
    const int64_t row = gid / nb;
    const int b = (int)(gid - row * nb);
    const uint4* p = reinterpret_cast<const uint4*>(x + row * ldx + 32 * b);
    uint32_t w[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint4 t = ld_stream16(p + q);
        w[4 * q] = t.x; w[4 * q + 1] = t.y; w[4 * q + 2] = t.z; w[4 * q + 3] = t.w;
    }
    const MxBlock r = mx_encode(w);
    uint4* o = reinterpret_cast<uint4*>(codes + row * (int64_t)cols + 32 * b);
    o[0] = r.c0;
    o[1] = r.c1;
    scale[(int64_t)b * rows + row] = (uint8_t)r.sbyte;  // block-major scales
}

// Column-transposing MXFP8 per group: a workgroup owns 128 padded output
// columns (four 32-blocks of tokens) x 256 channels.  It stages the bf16
// [128 tokens x 256 channels] tile in LDS with coalesced 16-byte loads, then
// thread t walks channel t down the tile and writes its 4 blocks as one
// contiguous 128-byte run of codes[channel][p0 .. p0+128); the block-major
// scale bytes of neighbouring channels are neighbours in memory.
constexpr int COLT_TOK = 128;
constexpr int COLT_CH = 256;
constexpr int COLT_PITCH = COLT_CH + 8;  // bf16 elements; keeps 16-byte rows aligned

__global__ __launch_bounds__(256) void k_quantize_mxfp8_colwise_t(
    const uint16_t* __restrict__ x, int64_t rows, int cols, int64_t ldx, const int32_t* __restrict__ offsets,
    int ngroups, int64_t P, uint8_t* __restrict__ codes, uint8_t* __restrict__ scale) {
    __shared__ __align__(16) uint16_t tile[COLT_TOK * COLT_PITCH];
    __shared__ int64_t blk_m0[4];
    __shared__ int blk_n[4];
    const int t = threadIdx.x;
    const int64_t p0 = (int64_t)blockIdx.x * COLT_TOK;
    const int c_base = blockIdx.y * COLT_CH;

    if (t < 4) {
        // Group g starts at padded column 32*(g + offsets[g]/32), strictly
        // increasing in g: find the last group starting at or before pc.
        const int64_t pc = p0 + 32 * t;
        int64_t m0 = 0;
        int n = 0;
        if (pc < P) {
            int lo = 0, hi = ngroups - 1, g = -1;
            while (lo <= hi) {
                const int mid = (lo + hi) >> 1;
                const int64_t st = 32 * ((int64_t)mid + offsets[mid] / 32);
                if (st <= pc) { g = mid; lo = mid + 1; } else { hi = mid - 1; }
            }
            if (g >= 0) {
                const int64_t st = 32 * ((int64_t)g + offsets[g] / 32);
                const int64_t mb = offsets[g] + (pc - st);
                const int64_t end = offsets[g + 1];
                if (mb < end) {
                    m0 = mb;
                    n = (int)min((int64_t)32, end - mb);
                }
            }
        }
        blk_m0[t] = m0;
        blk_n[t] = n;
    }
    __syncthreads();

    // Stage: 128 token slots x 256 channels, 16 bytes per thread per step.
    const int q = t & 31;
    const int ch = c_base + 8 * q;
#pragma unroll 4
    for (int i = 0; i < COLT_TOK / 8; ++i) {
        const int s = (t >> 5) + 8 * i;
        const int b = s >> 5, ii = s & 31;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (ii < blk_n[b] && ch < cols)
            val = ld_stream16(x + (blk_m0[b] + ii) * ldx + ch);
        *reinterpret_cast<uint4*>(&tile[s * COLT_PITCH + 8 * q]) = val;
    }
    __syncthreads();

    const int c = c_base + t;
    if (c >= cols) return;
    uint8_t* crow = codes + (int64_t)c * P;
#pragma unroll 1
    for (int b = 0; b < 4; ++b) {
        const int64_t pc = p0 + 32 * b;
        if (pc >= P) break;
        uint32_t w[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const uint32_t lo = tile[(32 * b + 2 * j) * COLT_PITCH + t];
            const uint32_t hi = tile[(32 * b + 2 * j + 1) * COLT_PITCH + t];
            w[j] = lo | (hi << 16);
        }
        const MxBlock r = mx_encode(w);
        uint4* o = reinterpret_cast<uint4*>(crow + pc);
        o[0] = r.c0;
        o[1] = r.c1;
        scale[(pc >> 5) * cols + c] = (uint8_t)r.sbyte;  // block-major: coalesced across channels
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

hipError_t launch_quantize_nvfp4v(const uint16_t* x, int64_t rows, int cols, int64_t ldx, uint8_t* codes,
                                  uint8_t* bscale, float* rscale, hipStream_t s) {
    const int nb = cols / 16;
    const dim3 grid((unsigned)((rows + 3) / 4));
    if (nb <= 64)
        hipLaunchKernelGGL(k_quantize_nvfp4v<1>, grid, dim3(256), 0, s, x, rows, cols, ldx, codes, bscale, rscale);
    else if (nb <= 128)
        hipLaunchKernelGGL(k_quantize_nvfp4v<2>, grid, dim3(256), 0, s, x, rows, cols, ldx, codes, bscale, rscale);
    else if (nb <= 256)
        hipLaunchKernelGGL(k_quantize_nvfp4v<4>, grid, dim3(256), 0, s, x, rows, cols, ldx, codes, bscale, rscale);
    else if (nb <= 512)
        hipLaunchKernelGGL(k_quantize_nvfp4v<8>, grid, dim3(256), 0, s, x, rows, cols, ldx, codes, bscale, rscale);
    else if (nb <= 1024)
        hipLaunchKernelGGL(k_quantize_nvfp4v<16>, grid, dim3(256), 0, s, x, rows, cols, ldx, codes, bscale, rscale);
    else
        return hipErrorInvalidValue;  // rejected by the host checks (cols > 16384)
    return hipGetLastError();
}

hipError_t launch_quantize_mxfp8_rowwise(const uint16_t* x, int64_t rows, int cols, int64_t ldx, uint8_t* codes,
                                         uint8_t* scale, hipStream_t s) {
    const int64_t nblk = rows * (cols / 32);
    hipLaunchKernelGGL(k_quantize_mxfp8_rowwise, dim3((unsigned)((nblk + 255) / 256)), dim3(256), 0, s, x, rows,
                       cols, ldx, codes, scale);
    return hipGetLastError();
}

hipError_t launch_quantize_mxfp8_colwise_t(const uint16_t* x, int64_t rows, int cols, int64_t ldx,
                                           const int32_t* offsets, int ngroups, int64_t P, uint8_t* codes,
                                           uint8_t* scale, hipStream_t s) {
    const dim3 grid((unsigned)((P + COLT_TOK - 1) / COLT_TOK), (unsigned)((cols + COLT_CH - 1) / COLT_CH));
    hipLaunchKernelGGL(k_quantize_mxfp8_colwise_t, grid, dim3(256), 0, s, x, rows, cols, ldx, offsets, ngroups, P,
                       codes, scale);
    return hipGetLastError();
}

hipError_t launch_debug_encode(int which, const float* in, uint8_t* out, int64_t n, hipStream_t s) {
    const dim3 grid((unsigned)((n + 255) / 256));
    if (which == 0)
        hipLaunchKernelGGL(k_debug_e2m1, grid, dim3(256), 0, s, in, out, n);
    else
        hipLaunchKernelGGL(k_debug_e4m3, grid, dim3(256), 0, s, in, out, n);
    return hipGetLastError();
}

}  // namespace bsq
