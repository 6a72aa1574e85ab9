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
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

// XOR applied to the 16-byte chunk index of row `row` of a row-major [rows, HD] bf16 LDS tile:
// 16 lanes reading one chunk of 16 consecutive rows, or 8-byte pieces of 4 consecutive rows
// at 4 column offsets (the transpose reads), hit distinct banks.
template <int HD>
__device__ __forceinline__ int swz(int row) {
    // rows of 256 bytes or more: the low four chunk bits span the 64 banks once.  16 consecutive
    // rows take 16 distinct values, and 4 consecutive rows from a multiple of 4 differ in the
    // upper two bits, so a transposed read's 32 lanes (4 rows x 32 columns) cover 16 chunks
    if (HD >= 128) return ((row & 3) << 2) | ((row >> 2) & 3);
    // 128-byte rows (two per bank span): 8 rows of one parity take 8 distinct values, and the two
    // rows of one parity in an aligned 4-row group differ in the upper bit
    return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
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

// dma16 with the streaming (non-temporal) cache policy: for data read once, so that it does not
// push reused tiles out of the L2.
__device__ __forceinline__ void dma16_nt(i32x4 rsrc, unsigned voff, unsigned lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds"
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

// Wait until at most N of this wave's tile loads are outstanding and every LDS read of this
// wave has returned, then a workgroup barrier.  After the barrier other waves refill ring slots
// that this wave has just read: a read still in flight (its consuming matrix op moved below the
// barrier by the compiler) would race with that refill, so lgkmcnt(0) is part of the wait.
template <int N>
__device__ __forceinline__ void wait_barrier() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
}

// A workgroup barrier after this wave's LDS accesses have completed, leaving its tile loads in
// flight: for exchanges through LDS in the middle of a tile.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Writes one wave's 32 output rows of HD bf16 values held in the 32x32 matrix-core C layout
// (lane l owns row l % 32; element 4g + j of block mb is column 32 mb + 8 g + 4 (l / 32) + j),
// each value times the lane's `sc`.  The rows are staged in `stage` (32 * HD * 2 bytes of LDS
// that no other wave touches; 16-byte chunk index XORed by the row, so that neither the 8-byte
// writes nor the 16-byte reads conflict) and leave as whole rows: 16-byte stores, HD / 8
// consecutive lanes per row.  Row r goes to out + 2 * (first + r * stride) bytes and is written
// only when rfirst <= r < nrows.  Row starts must be 16-byte aligned.
template <int HD>
__device__ __forceinline__ void store_rows_bf16(const f32x16 *acc, float sc, unsigned char LDS_AS *stage,
                                                unsigned char *out, int64_t first, int64_t stride, int nrows,
                                                int rfirst = 0) {
    constexpr int CPR = HD / 8;  // 16-byte chunks per row
    const int lane = threadIdx.x & 63, l32 = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int mb = 0; mb < HD / 32; ++mb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int pc = (4 * mb + g) ^ (l32 & (CPR - 1));
            *(bf16x4 LDS_AS *)(stage + l32 * HD * 2 + pc * 16 + hh * 8) =
                bf16x4{(__bf16)(acc[mb][4 * g] * sc), (__bf16)(acc[mb][4 * g + 1] * sc),
                       (__bf16)(acc[mb][4 * g + 2] * sc), (__bf16)(acc[mb][4 * g + 3] * sc)};
        }
#pragma unroll
    for (int i = 0; i < 32 * CPR / 64; ++i) {
        const int idx = i * 64 + lane, r = idx / CPR, ch = idx % CPR;
        const u32x4 val = *(const u32x4 LDS_AS *)(stage + r * HD * 2 + ((ch ^ (r & (CPR - 1))) << 4));
        if (r >= rfirst && r < nrows) *(u32x4 *)(out + (first + (int64_t)r * stride + ch * 8) * 2) = val;
    }
}

}  // namespace attn
