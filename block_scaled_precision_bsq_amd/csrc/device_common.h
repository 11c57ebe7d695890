// Device helpers shared by the gfx950 kernels of libbsq.
//
// Number formats (named in "Composer 2 Technical Report", section 6.1):
//  E2M1  sign + 2-bit exponent (bias 1) + 1-bit mantissa, magnitudes
//        0, .5, 1, 1.5, 2, 3, 4, 6.
//  E4M3  OCP E4M3FN, bias 7, subnormals m * 2^-9, max 448.
//  E8M0  2^(byte - 127).
// All encoders round to nearest even and saturate (E2M1 at 6, E4M3 at 448).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef int int8v __attribute__((ext_vector_type(8)));

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 16-byte streaming load (data read once: nontemporal hint).
__device__ __forceinline__ uint4 ld_stream16(const void* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Streaming stores of outputs written once (non-temporal hint); used where a
// wave's stores cover whole 128-byte lines (partial-line and byte stores stay
// ordinary stores, which the L2 merges).
__device__ __forceinline__ void st_stream16(void* p, uint4 v) {
    __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void st_stream4(void* p, uint32_t v) { __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(p)); }
__device__ __forceinline__ void st_stream8(void* p, uint2 v) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    __builtin_nontemporal_store(u32x2{v.x, v.y}, reinterpret_cast<u32x2*>(p));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Per-half |bf16| maxima of m (two 16-bit magnitudes) and w: one mask and
// one packed 16-bit max (magnitudes of non-NaN bf16 order like their bits).
__device__ __forceinline__ uint32_t absmax2_bf16(uint32_t m, uint32_t w) {
    typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, m),
                                                                  __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu)));
}
// The larger of the two 16-bit halves of m.
__device__ __forceinline__ uint32_t fold_max16(uint32_t m) { return max(m & 0xFFFFu, m >> 16); }

// Two floats -> packed bf16 pair, a in the low half, rounded to nearest even
// by the hardware conversion (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// SwiGLU activation between the two forward GEMMs (not on the pages; the
// plainest DeepSeek-V3-class reading): H = silu(g) * u with silu(g) =
// g * sigmoid(g), evaluated in binary32 from t = e^-|g| in (0, 1], which never
// overflows: g / (1 + t) for g >= 0 and (g * t) / (1 + t) for g < 0, so a very
// negative gate gives the tiny value it should.  t = 2^y with y = -|g| log2(e)
// comes from the hardware exponential; for y < -126 (t below the binary32
// normal range) the argument is raised by 64 and the result scaled by 2^-64,
// so t keeps its subnormal value instead of flushing to zero.  1 / (1 + t),
// with 1 + t in [1, 2], comes from the hardware reciprocal.  Each step is
// within a few binary32 ulps (the rounding of y costs |y| 2^-24 relative in
// t), far below the bf16 rounding of the result: H lies within one bf16 ulp
// of the exactly rounded value, equal to it except next to a rounding
// boundary.
__device__ __forceinline__ float silu_mul(float g, float u) {
    const float y = -fabsf(g) * 1.44269504f;
    const bool tiny = y < -126.0f;
    float t = __builtin_amdgcn_exp2f(tiny ? y + 64.0f : y);
    t = tiny ? t * 0x1p-64f : t;
    const float num = g >= 0.0f ? g : g * t;
    return (num * __builtin_amdgcn_rcpf(1.0f + t)) * u;
}

// H of two packed bf16 gate values and the matching up values, packed bf16
// (round to nearest even), low halves first.
__device__ __forceinline__ uint32_t swiglu_pair(uint32_t gw, uint32_t uw) {
    return pack_bf16x2(silu_mul(bf16_lo(gw), bf16_lo(uw)), silu_mul(bf16_hi(gw), bf16_hi(uw)));
}

// E2M1 codes of two floats into nibbles of byte `sel` of `old`: low nibble
// from a, high nibble from b.  The hardware conversion rounds to nearest
// even, saturates to +-6 and keeps the sign of zero; a unit scale leaves the
// values unchanged (checked exhaustively against the CPU oracle).
template <int SEL>
__device__ __forceinline__ uint32_t e2m1x2(uint32_t old, float a, float b) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

// E4M3 bytes of four floats (any non-NaN values), a in the lowest byte:
// clamp to +-448 first, the hardware conversion then rounds to nearest even
// (checked exhaustively against the CPU oracle).
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
    a = __builtin_amdgcn_fmed3f(a, 448.0f, -448.0f);
    b = __builtin_amdgcn_fmed3f(b, 448.0f, -448.0f);
    c = __builtin_amdgcn_fmed3f(c, 448.0f, -448.0f);
    d = __builtin_amdgcn_fmed3f(d, 448.0f, -448.0f);
    uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// Wave-wide maximum (wave64) of a non-negative value's bit pattern.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
    return v;
}

}  // namespace bsq

namespace bsq {

// Raw buffer resource over [base, base + bytes): loads through it take a
// 32-bit byte offset and return zero when the access lies beyond `bytes`
// (used for row and k masking).  bytes must stay below 2^31.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

constexpr uint32_t OOB = 0x80000000u;  // offset that always reads zero

// Mark a wave-uniform value as such (keeps it, and what is derived from it,
// in SGPRs; buffer resources built from divergent-looking values otherwise
// force a readfirstlane loop around every load).
template <class T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ int64_t uniform_i64(int64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}

__device__ __forceinline__ uint32_t buf_load1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return (uint32_t)__builtin_bit_cast(uint8_t, __builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, 0));
}

}  // namespace bsq
