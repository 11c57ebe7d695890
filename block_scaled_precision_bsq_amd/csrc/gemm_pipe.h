// LDS staging helpers shared by the grouped GEMM and quantize kernels (gfx950).
//
// Operand tiles travel global -> LDS through the buffer-load-to-LDS path
// ("buffer_load_dwordx4 ... lds"): each wave instruction writes 64 lanes x 16
// bytes to 1 KB of consecutive LDS starting at M0, with no VGPR staging.
// Rows are stored unpadded; the 16-byte chunks of a row are permuted by an
// XOR swizzle (swz8 below) so that fragment reads, which take one chunk from
// each of 16 or 32 consecutive rows, spread over all banks.  Each kernel
// describes its own ring of stages.
//
// The loads go through the compiler's LDS-DMA builtin.  The kernels wait for
// them explicitly: s_waitcnt vmcnt(N) for their own DMA groups (the counter
// retires vector-memory operations in issue order on this target), then
// s_barrier so every wave's part of a stage is in LDS before anyone reads
// it, and s_waitcnt lgkmcnt(0) before the barrier that precedes overwriting a
// ring slot, so all reads of that slot are done.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace bsq {

typedef int i32x4 __attribute__((ext_vector_type(4)));

// compile-time index for generic lambdas (schedule slots, ring parts)
template <int V>
using IC = std::integral_constant<int, V>;

constexpr int PIPE_ROWS = 256;  // rows per operand tile

// 128-byte rows hold 8 chunks of 16 bytes; chunk c of row r lives in slot
// c ^ swz8(r).  A 16-lane quarter of a fragment read covers 16 consecutive
// rows at one chunk: rows of equal parity share 8-chunk halves of the 64 LDS
// banks and swz8 = (r >> 1) & 7 spreads them over all 8 slots.
__device__ __forceinline__ int swz8(int r) { return (r >> 1) & 7; }

// Raw buffer descriptor (base, stride 0, num_records, gfx9 data format).
__device__ __forceinline__ i32x4 make_desc(const void* base) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r.x = (int)(uint32_t)a;
    r.y = (int)((a >> 32) & 0xFFFFu);
    r.z = 0x7FFFFFFF;
    r.w = 0x00020000;
    return r;
}

// Values laundered through an empty asm: the compiler can no longer see them
// as loop invariants, so sums built from them are formed at their use.
__device__ __forceinline__ uint32_t opaque_v(uint32_t x) {
    asm volatile("" : "+v"(x));
    return x;
}
__device__ __forceinline__ uint32_t opaque_s(uint32_t x) {
    asm volatile("" : "+s"(x));
    return x;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Buffer-to-LDS DMA through the compiler's builtin, which owns M0: each lane
// moves SIZE bytes from desc+voff to LDS, lane i's data at lds_base + 16 i
// for SIZE 16 and at lds_base + 4 i for SIZE 4 and 1 (a byte lands
// zero-extended in its dword).  lds_base is wave-uniform; an offset past the
// descriptor's range reads as zero.
template <int SIZE>
__device__ __forceinline__ void dma_lds(i32x4 desc, uint32_t voff, uint32_t lds_base) {
    lds_base = __builtin_amdgcn_readfirstlane(lds_base);
    const uint64_t base = (uint64_t)(uint32_t)desc.x | ((uint64_t)((uint32_t)desc.y & 0xFFFFu) << 32);
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, desc.z, desc.w);
    __attribute__((address_space(3))) void* dst = (__attribute__((address_space(3))) void*)(uintptr_t)lds_base;
    if constexpr (SIZE == 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, voff, 0, 0, 0);
    else if constexpr (SIZE == 4)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 4, voff, 0, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 1, voff, 0, 0, 0);
}
__device__ __forceinline__ void dma16(i32x4 desc, uint32_t voff, uint32_t lds_base) { dma_lds<16>(desc, voff, lds_base); }

// The same DMA from a ready-made buffer resource (a tile's operand kept as a
// resource is not rebuilt from its descriptor words at every instruction).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_n(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
template <int SIZE>  // 16 or 4
__device__ __forceinline__ void dma_lds_r(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t lds_base) {
    lds_base = __builtin_amdgcn_readfirstlane(lds_base);
    __attribute__((address_space(3))) void* dst = (__attribute__((address_space(3))) void*)(uintptr_t)lds_base;
    if constexpr (SIZE == 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, voff, 0, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 4, voff, 0, 0, 0);
}
__device__ __forceinline__ void dma4(i32x4 desc, uint32_t voff, uint32_t lds_base) { dma_lds<4>(desc, voff, lds_base); }
__device__ __forceinline__ void dma1(i32x4 desc, uint32_t voff, uint32_t lds_base) { dma_lds<1>(desc, voff, lds_base); }

// LDS target base + OFF with the base laundered through an empty asm: the
// compiler then adds OFF right at the DMA instead of hoisting one live SGPR
// per (instruction, ring slot) out of the loops.
template <uint32_t OFF>
__device__ __forceinline__ uint32_t lds_at(uint32_t base) {
    asm volatile("" : "+s"(base));
    return base + OFF;
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ void wait_lgkmcnt0() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ void block_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

}  // namespace bsq
