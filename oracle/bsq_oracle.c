/*
 * bsq_oracle.c -- plain, slow CPU oracle for the block-scaled MoE expert GEMM
 * path.  TEST INFRASTRUCTURE ONLY: it is linked by the tests, the smoke check
 * and the bench's CPU-baseline leg, never by the product path, and it shares
 * no code, header, table or constant generator with the HIP library.
 *
 * Built with gcc -O2 -ffp-contract=off -fno-fast-math on x86-64 (SSE2 scalar
 * float, IEEE denormals), so every `float` operation below is one correctly
 * rounded IEEE-754 binary32 operation in round-to-nearest-even.
 *
 * Sources (pages as printed; the pages name the formats but print no formulas):
 *  - "Composer 2 Technical Report" (papercache.org summary), section 6.1
 *    "Training infrastructure": the MoE forward uses an NVFP4 variant -- BF16
 *    values quantized to FP4 E2M1 with one FP8 E4M3 scale per 16-element block
 *    and one FP32 scale per token, replacing the per-tensor FP32 scale; the
 *    backward uses standard MXFP8 (E4M3 values, E8M0 scale per 32 elements);
 *    NVFP4 quantization needs IEEE-compliant division, MXFP8 does not.
 *  - "Cursor Composer 2 report deep dive" (machinelearningatscale), section 1
 *    "The kernel section": same recipe; per-tensor scales are batch-variant and
 *    leak future-token information, per-token scaling costs latency in the
 *    quantize and GEMM epilogue.
 *
 * Readings where the pages are silent (each one is listed in the design notes):
 *  E2M1     sign + 2-bit exponent (bias 1) + 1-bit mantissa; magnitudes
 *           {0, .5, 1, 1.5, 2, 3, 4, 6}; no Inf/NaN.
 *  E4M3     OCP E4M3FN: bias 7, subnormals m*2^-9, max 448 (0x7E); 0x7F/0xFF
 *           are NaN and never produced.
 *  E8M0     value 2^(byte-127); 0xFF (NaN) never produced.
 *  Rounding round-to-nearest-even everywhere; E2M1 saturates at 6, E4M3 at
 *           448; the sign bit of the input is kept on every code.
 *  NVFP4v   per row x[0..K): A = max|x|.  A == 0 -> all outputs zero.
 *           Otherwise s_row = RN32(A / 2688) (the stored per-token decode scale;
 *           2688 = 6 * 448); per 16-block b: a_b = max|x| in the block,
 *           t_b = RN32(448 * a_b / A), S_b = E4M3(t_b);
 *           d_b = RN32(S_b * s_row); if d_b == 0 the block's codes are 0,
 *           else code = sign(x) | E2M1(RN32(x / d_b)).
 *           Nibble order: element 2j in the low nibble of byte j.
 *  MXFP8    per 32-block: A = max|x|; A == 0 -> scale byte 0, codes 0.
 *           Else sh = clamp(floor(log2 A) - 8, -127, 127) (8 = E4M3 emax),
 *           scale byte = sh + 127, code = sign(x) | E4M3(x * 2^-sh).
 *           Scales are stored block-major: the byte of (row r, block b) of an
 *           R-row matrix is at b * R + r.
 *  COLWISE_T  the MXFP8 blocks run down the rows (tokens) of each segment
 *           [off[g], off[g+1]) and restart at each segment; the output is
 *           transposed, codes [cols][P] with P = 128*(G + ceil(rows/128)),
 *           scales [P/32][cols] (block-major); segment g starts at column
 *           c0[g] = 128*(g + floor(off[g]/128)), a whole 128-byte line of
 *           every code row; every other byte (padding, gaps) is 0.  This
 *           padded layout is the library's storage convention; the pages fix
 *           only the element format and the 32-element blocks.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <string.h>

#define ORC_API __attribute__((visibility("default")))

/* ------------------------------------------------------------ threading */

/* Thread count of the parallel loops below (timing only: every loop writes
 * disjoint outputs, so results do not depend on it). */
ORC_API void orc_set_num_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
ORC_API int orc_max_threads(void) { return omp_get_max_threads(); }

/* ---------------------------------------------------------------- decoding */

static const double kE2M1Mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

ORC_API double orc_e2m1_value(uint8_t code) {
    double v = kE2M1Mag[code & 7];
    return (code & 8) ? -v : v;
}

ORC_API double orc_e4m3_value(uint8_t b) {
    int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
    if (e == 15 && m == 7) return NAN;
    double v = (e == 0) ? ldexp((double)m, -9)        /* subnormal: m * 2^-9  */
                        : ldexp((double)(8 + m), e - 10); /* 2^(e-7) * (1+m/8) */
    return s ? -v : v;
}

ORC_API double orc_e8m0_value(uint8_t b) {
    if (b == 0xFF) return NAN;
    return ldexp(1.0, (int)b - 127);
}

static float bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* ---------------------------------------------------------------- encoding */

/* E2M1 magnitude code (0..7) of a non-negative, non-NaN value: round to the
 * nearest representable magnitude, ties to the even code, saturate at 6. */
static uint8_t e2m1_mag_code(double av) {
    if (!(av < 6.0)) return 7;
    if (av == 0.0) return 0;
    int ex;
    frexp(av, &ex);
    int E = ex - 1;            /* floor(log2 av) */
    if (E < 0) E = 0;          /* [0,2) shares the 0.5 quantum (subnormal 0.5) */
    double q = ldexp(1.0, E - 1);
    double r = nearbyint(av / q); /* av/q is exact; nearbyint is RNE */
    double val = r * q;           /* one of 0, .5, 1, 1.5, 2, 3, 4, 6 */
    for (uint8_t c = 0; c < 8; ++c)
        if (kE2M1Mag[c] == val) return c;
    return 7; /* unreachable */
}

/* E4M3 magnitude byte (0..0x7E) of a non-negative, non-NaN value: RNE with
 * saturation at 448. */
static uint8_t e4m3_mag_code(double av) {
    if (!(av < 448.0)) return 0x7E;
    if (av == 0.0) return 0;
    int ex;
    frexp(av, &ex);
    int E = ex - 1;
    if (E < -6) E = -6;                 /* subnormal range shares 2^-9 quantum */
    double r = nearbyint(av / ldexp(1.0, E - 3));
    if (r == 16.0) { r = 8.0; E += 1; } /* rounded up into the next binade */
    if (r < 8.0) return (uint8_t)r;     /* subnormal (E == -6) */
    return (uint8_t)(((E + 7) << 3) | ((int)r - 8));
}

ORC_API uint8_t orc_e2m1_encode(float v) {
    return (uint8_t)((signbit(v) ? 8 : 0) | e2m1_mag_code(fabs((double)v)));
}

ORC_API uint8_t orc_e4m3_encode(float v) {
    return (uint8_t)((signbit(v) ? 0x80 : 0) | e4m3_mag_code(fabs((double)v)));
}

ORC_API void orc_e2m1_encode_array(const float* v, uint8_t* out, int64_t n) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e2m1_encode(v[i]);
}

ORC_API void orc_e4m3_encode_array(const float* v, uint8_t* out, int64_t n) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode(v[i]);
}

/* --------------------------------------------------------- NVFP4 variant */

/* RN32(448 * a / A) for 0 <= a <= A, A > 0: one division of two exact
 * operands.  448*a has at most 11 significant bits.  For a > 2^119 it could
 * overflow, so numerator and denominator are both scaled by 2^-9 (exact: both
 * stay above 2^110, far from the subnormal range, and 448 * 2^-9 * a < a
 * stays finite), which leaves the exact quotient unchanged. */
static float block_ratio(float a, float A) {
    float num, den;
    if (a <= 0x1p119f) { num = 448.0f * a;  den = A; }
    else               { num = 0.875f * a;  den = A * 0x1p-9f; }
    return num / den;
}

ORC_API void orc_quantize_nvfp4v(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                 uint8_t* codes, uint8_t* bscale, float* rscale) {
    const int64_t nb = cols / 16;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t* xr = x + r * ldx;
        uint8_t* cr = codes + r * (cols / 2);
        uint8_t* br = bscale + r * nb;
        float A = 0.0f;
        for (int64_t k = 0; k < cols; ++k) A = fmaxf(A, fabsf(bf16_to_f32(xr[k])));
        if (A == 0.0f) {
            rscale[r] = 0.0f;
            memset(cr, 0, (size_t)(cols / 2));
            memset(br, 0, (size_t)nb);
            continue;
        }
        const float s_row = A / 2688.0f;
        rscale[r] = s_row;
        for (int64_t b = 0; b < nb; ++b) {
            float a_b = 0.0f;
            for (int k = 0; k < 16; ++k) a_b = fmaxf(a_b, fabsf(bf16_to_f32(xr[16 * b + k])));
            const float t_b = block_ratio(a_b, A);
            const uint8_t S = e4m3_mag_code((double)t_b);
            br[b] = S;
            const float d_b = (float)orc_e4m3_value(S) * s_row;
            for (int k = 0; k < 16; k += 2) {
                uint8_t c[2];
                for (int h = 0; h < 2; ++h) {
                    const float xv = bf16_to_f32(xr[16 * b + k + h]);
                    if (d_b == 0.0f) { c[h] = 0; continue; }
                    const float v = xv / d_b;        /* IEEE binary32 division */
                    c[h] = (uint8_t)((signbit(xv) ? 8 : 0) | e2m1_mag_code(fabs((double)v)));
                }
                cr[(16 * b + k) / 2] = (uint8_t)(c[0] | (c[1] << 4));
            }
        }
    }
}

ORC_API void orc_dequant_nvfp4v(const uint8_t* codes, const uint8_t* bscale, const float* rscale,
                                int64_t rows, int64_t cols, double* out) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t k = 0; k < cols; ++k) {
            const uint8_t byte = codes[r * (cols / 2) + k / 2];
            const uint8_t c = (k & 1) ? (byte >> 4) : (byte & 15);
            out[r * cols + k] = orc_e2m1_value(c) * orc_e4m3_value(bscale[r * (cols / 16) + k / 16]) *
                                (double)rscale[r];
        }
    }
}

/* ---------------------------------------------------------------- MXFP8 */

/* Shared exponent of one block with max magnitude A > 0 (exact, frexp also
 * handles subnormals). */
static int mx_shift(float A) {
    int ex;
    frexp((double)A, &ex);
    int sh = (ex - 1) - 8;
    if (sh < -127) sh = -127;
    if (sh > 127) sh = 127;
    return sh;
}

static void mx_block(const float* v, int n, uint8_t* code_out, int64_t code_stride, uint8_t* scale_out) {
    /* one block of n <= 32 values: codes at code_out[i * code_stride], E8M0 at *scale_out */
    float A = 0.0f;
    for (int i = 0; i < n; ++i) A = fmaxf(A, fabsf(v[i]));
    if (A == 0.0f) {
        *scale_out = 0;
        for (int i = 0; i < n; ++i) code_out[i * code_stride] = 0;
        return;
    }
    const int sh = mx_shift(A);
    *scale_out = (uint8_t)(sh + 127);
    for (int i = 0; i < n; ++i) {
        const double scaled = ldexp(fabs((double)v[i]), -sh); /* exact */
        code_out[i * code_stride] = (uint8_t)((signbit(v[i]) ? 0x80 : 0) | e4m3_mag_code(scaled));
    }
}

ORC_API void orc_quantize_mxfp8_rowwise(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                        uint8_t* codes, uint8_t* scale) {
    const int64_t nb = cols / 32;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < rows; ++r) {
        float v[32];
        for (int64_t b = 0; b < nb; ++b) {
            for (int i = 0; i < 32; ++i) v[i] = bf16_to_f32(x[r * ldx + 32 * b + i]);
            mx_block(v, 32, codes + r * cols + 32 * b, 1, scale + b * rows + r);
        }
    }
}

ORC_API int64_t orc_colwise_padded_cols(int32_t ngroups, int64_t rows) {
    return 128 * ((int64_t)ngroups + (rows + 127) / 128);
}

ORC_API void orc_quantize_mxfp8_colwise_t(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                          const int32_t* offsets, int32_t ngroups,
                                          uint8_t* codes, uint8_t* scale) {
    const int64_t P = orc_colwise_padded_cols(ngroups, rows);
    memset(codes, 0, (size_t)(cols * P));
    memset(scale, 0, (size_t)(cols * (P / 32)));
#pragma omp parallel for schedule(dynamic, 8)
    for (int64_t c = 0; c < cols; ++c) {
        float v[32];
        for (int32_t g = 0; g < ngroups; ++g) {
            const int64_t m0 = offsets[g], m1 = offsets[g + 1];
            const int64_t c0 = 128 * ((int64_t)g + m0 / 128);
            for (int64_t j = 0; m0 + 32 * j < m1; ++j) {
                const int64_t mb = m0 + 32 * j;
                const int n = (int)((m1 - mb) < 32 ? (m1 - mb) : 32);
                for (int i = 0; i < n; ++i) v[i] = bf16_to_f32(x[(mb + i) * ldx + c]);
                mx_block(v, n, codes + c * P + c0 + 32 * j, 1, scale + (c0 / 32 + j) * cols + c);
            }
        }
    }
}

/* Dequantize an MXFP8 matrix whose blocks run along its rows: element (r, c) =
 * E4M3(codes[r*ld_codes + c]) * E8M0(scale[r*s_row + (c/32)*s_blk]). */
ORC_API void orc_dequant_mxfp8(const uint8_t* codes, const uint8_t* scale, int64_t rows, int64_t cols,
                               int64_t ld_codes, int64_t s_row, int64_t s_blk, double* out) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            out[r * cols + c] = orc_e4m3_value(codes[r * ld_codes + c]) *
                                orc_e8m0_value(scale[r * s_row + (c / 32) * s_blk]);
}
