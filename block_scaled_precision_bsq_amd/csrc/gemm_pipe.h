// LDS staging helpers shared by the grouped GEMM and quantize kernels (gfx950).
//
// Operand tiles travel global -> LDS through the buffer-load-to-LDS path
// ("buffer_load_dwordx4 ... lds"): each wave instruction writes 64 lanes x 16
// bytes to 1 KB of consecutive LDS starting at M0, with no VGPR staging.  A
// stage holds 256 rows x 64 bytes per operand; 16 rows fill one instruction,
// so rows are stored unpadded and the 16-byte chunks of row r are permuted by
// an XOR swizzle, chunk c living at slot c ^ swz(r).  swz(r) =
// ((r >> 1) ^ (r >> 2)) & 3 makes the fragment reads -- 16 consecutive rows,
// one chunk each -- hit 16 distinct 4-bank groups (and 8 rows, 8 groups).
//
// Four stages form a ring.  The loads are issued from inline assembly, so the
// compiler does not see LDS writes in flight and inserts no waits for them;
// the kernel waits explicitly: s_waitcnt vmcnt(N) for its own DMA groups (the
// counter retires in order), then s_barrier so every wave's part of a stage is
// in LDS before anyone reads it, and s_waitcnt lgkmcnt(0) before the barrier
// that precedes overwriting a ring slot, so all reads of that slot are done.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace bsq {

typedef int i32x4 __attribute__((ext_vector_type(4)));

// compile-time index for generic lambdas (schedule slots, ring parts)
template <int V>
using IC = std::integral_constant<int, V>;

constexpr int PIPE_ROWS = 256;                  // rows per operand tile
constexpr int PIPE_BK = 64;                     // bytes per row per stage
constexpr int PIPE_STAGE_BYTES = PIPE_ROWS * PIPE_BK;
constexpr int PIPE_NST = 4;                     // ring depth

__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

// 128-byte rows hold 8 chunks of 16 bytes; chunk c of row r lives in slot
// c ^ swz8(r).  A 16-lane quarter of a fragment read covers 16 consecutive
// rows at one chunk: rows of equal parity share 8-chunk halves of the 64 LDS
// banks and swz8 = (r >> 1) & 7 spreads them over all 8 slots.
__device__ __forceinline__ int swz8(int r) { return (r >> 1) & 7; }

// Byte offset of logical 16-byte chunk c of row r inside a stage buffer.
__device__ __forceinline__ int swz_off(int r, int c) { return r * PIPE_BK + 16 * (c ^ swz(r)); }

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

// Descriptor whose byte range ends at `bytes`: offsets at or past it read as
// zero (the row limit of a partial tile).
__device__ __forceinline__ i32x4 make_desc_n(const void* base, uint32_t bytes) {
    i32x4 r = make_desc(base);
    r.z = (int)bytes;
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
