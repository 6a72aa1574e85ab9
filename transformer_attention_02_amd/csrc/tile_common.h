// Device helpers shared by the matrix-core kernels (gfx950): vector types, the LDS tile
// swizzle, buffer descriptors and direct global->LDS loads, and the wait+barrier.
#pragma once

#include <hip/hip_runtime.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

// XOR applied to the 16-byte chunk index of row `row` of a row-major [rows, HD] bf16 LDS tile:
// 16 lanes reading one chunk of 16 consecutive rows, or 8-byte pieces of 4 consecutive rows
// at 4 column offsets (the transpose reads), hit distinct banks.
template <int HD>
__device__ __forceinline__ int swz(int row) {
    if (HD == 128) return ((row & 7) << 1) | ((row >> 3) & 1);
    return (((row >> 1) & 3) << 1) | ((row >> 3) & 1);
}

// Raw buffer descriptor: byte range [base, base + num_records) is readable, the rest reads as 0.
__device__ __forceinline__ i32x4 make_rsrc(const void *base, unsigned num_records) {
    const unsigned long long p = (unsigned long long)base;
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(unsigned)p);
    r[1] = __builtin_amdgcn_readfirstlane((int)((p >> 32) & 0xffff));
    r[2] = __builtin_amdgcn_readfirstlane((int)num_records);
    r[3] = 0x00020000;
    return r;
}

// 16 bytes per lane from (descriptor, voffset) straight into LDS at lds + 16 * lane.
// Inline asm so that the compiler does not serialise later LDS reads behind these loads:
// the kernels order them themselves with wait_barrier().
__device__ __forceinline__ void dma16(i32x4 rsrc, unsigned voff, unsigned lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(lds)
                 : "memory");
}

// 4 bytes per lane from (descriptor, voffset) straight into LDS at lds + 4 * lane.
__device__ __forceinline__ void dma4(i32x4 rsrc, unsigned voff, unsigned lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(lds)
                 : "memory");
}

// Wait until at most N of this wave's tile loads are outstanding, then a workgroup barrier.
template <int N>
__device__ __forceinline__ void wait_barrier() {
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" : : "n"(N) : "memory");
}

}  // namespace attn
