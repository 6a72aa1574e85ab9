// Exact LSE-weighted merge of attention results over disjoint key chunks
// (MSLK kernel reference, "Attention - Core fMHA": merge_attentions; "MSLK
// Kernel Library -- Complete Reference", Quick start, "Exact softmax merge").
//
// For every output row (b, m, head): M* = max_c lse_c, L = M* + ln sum_c
// exp(lse_c - M*), out = sum_c exp(lse_c - L) out_c.  A chunk at -inf weighs 0;
// all chunks at -inf give out = 0 and lse = -inf.
//
// One workgroup per row.  The value dimension is read by 8 chunk groups of 32
// lanes, each lane taking 4 consecutive elements of every 8th chunk, with all of
// a lane's loads issued first (before the LSEs are even reduced).  Threads c < S
// read the S LSEs and reduce them to L (wave 0 alone when S <= 64, one barrier);
// the weights go to LDS, and the 8 weighted partial sums are added through LDS.
// The kernel is instantiated for 1, 2, 4, 8 or 16 chunks per lane, so a merge of few
// chunks holds few registers and keeps more rows in flight.  Memory-bound: every chunk
// element is read once and every output element written once.
#include "kernels.h"

namespace attn {
namespace {

constexpr int NT = 256;
constexpr int GROUPS = 8;           // chunk groups per row
constexpr int SPAN = 128;           // elements of the value dim per pass (32 lanes x 4)
constexpr int MAXPER = kMaxChunks / GROUPS;

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float block_reduce(float x, float *red, bool is_max) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const float y = __shfl_xor(x, o, 64);
        x = is_max ? fmaxf(x, y) : x + y;
    }
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
    __syncthreads();
    return is_max ? fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])) : (red[0] + red[1]) + (red[2] + red[3]);
}

// 4 consecutive elements starting at element d of a chunk row; elements >= n read as 0.
__device__ __forceinline__ f32x4 load4(const void *base, int64_t off, int d, int n, bool f32) {
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    if (d + 3 < n && ((off + d) & 3) == 0) {
        if (f32) return *(const f32x4 *)((const float *)base + off + d);
        const uint2 w = *(const uint2 *)((const __bf16 *)base + off + d);
        x[0] = __uint_as_float(w.x << 16);
        x[1] = __uint_as_float(w.x & 0xffff0000u);
        x[2] = __uint_as_float(w.y << 16);
        x[3] = __uint_as_float(w.y & 0xffff0000u);
        return x;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (d + i < n) x[i] = f32 ? ((const float *)base)[off + d + i] : (float)((const __bf16 *)base)[off + d + i];
    return x;
}

// MAXP: chunks per lane and pass (ceil(S / GROUPS), rounded up to a power of two), so that small
// merges hold few registers and keep more rows in flight
template <int MAXP>
__global__ __launch_bounds__(NT) void merge_kernel(MergeArgs a) {
    __shared__ float red[4];
    __shared__ float w_s[kMaxChunks];
    __shared__ f32x4 part[GROUPS][SPAN / 4];

    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    const int hf = (int)(row % a.Htot);
    const int m = (int)((row / a.Htot) % a.M);
    const int b = (int)(row / ((int64_t)a.Htot * a.M));
    const int64_t loff = ((int64_t)b * a.Htot + hf) * a.M + m;
    const int64_t coff = (int64_t)b * a.sc.b + (int64_t)m * a.sc.m + head_offset(a.sc, hf, a.Hin);
    const int64_t ooff = (int64_t)b * a.so.b + (int64_t)m * a.so.m + head_offset(a.so, hf, a.Hin);

    // the first pass's chunk values do not depend on the weights: issue their loads before
    // the LSE reduction, so that a row costs one memory round trip when Kv <= SPAN
    const int g = tid / (SPAN / 4), j = tid % (SPAN / 4);
    const bool f32 = a.chunk_f32;
    f32x4 x[MAXP];
    auto load_pass = [&](int d0) __attribute__((always_inline)) {
        const int d = d0 + 4 * j;
#pragma unroll
        for (int i = 0; i < MAXP; ++i) {
            const int c = g + GROUPS * i;
            x[i] = c < a.S ? load4(a.chunk[c], coff, d, a.Kv, f32) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    };
    load_pass(0);

    float L;
    if (a.S <= 64) {
        // every LSE sits in wave 0: it forms the weights alone, and one barrier publishes them
        if (tid < 64) {
            const float lv = tid < a.S ? a.lse[tid][loff] : -INFINITY;
            float mx = lv;
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
            float Lw = -INFINITY;
            if (mx != -INFINITY) {
                float e = tid < a.S ? expf(lv - mx) : 0.f;
#pragma unroll
                for (int o = 32; o >= 1; o >>= 1) e += __shfl_xor(e, o, 64);
                Lw = mx + logf(e);
                if (tid < a.S) w_s[tid] = expf(lv - Lw);
            }
            if (tid == 0) red[0] = Lw;
        }
        __syncthreads();
        L = red[0];
    } else {
        const float lv = tid < a.S ? a.lse[tid][loff] : -INFINITY;
        const float mx = block_reduce(lv, red, true);
        L = -INFINITY;
        if (mx != -INFINITY) {
            const float sum = block_reduce(tid < a.S ? expf(lv - mx) : 0.f, red, false);
            L = mx + logf(sum);
            if (tid < a.S) w_s[tid] = expf(lv - L);
            __syncthreads();
        }
    }
    if (L == -INFINITY) {  // every chunk empty (uniform)
        for (int d = tid; d < a.Kv; d += NT) {
            if (a.out_f32) ((float *)a.o)[ooff + d] = 0.f;
            else ((__bf16 *)a.o)[ooff + d] = (__bf16)0.f;
        }
        if (a.lse_out && tid == 0) a.lse_out[loff] = -INFINITY;
        return;
    }
    if (a.lse_out && tid == 0) a.lse_out[loff] = L;

    for (int d0 = 0; d0 < a.Kv; d0 += SPAN) {
        if (d0 > 0) load_pass(d0);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < MAXP; ++i) {
            const int c = g + GROUPS * i;
            if (c < a.S) acc += w_s[c] * x[i];
        }
        part[g][j] = acc;
        __syncthreads();
        if (tid < SPAN) {
            float s = 0.f;
#pragma unroll
            for (int gg = 0; gg < GROUPS; ++gg) s += part[gg][tid >> 2][tid & 3];
            const int dd = d0 + tid;
            if (dd < a.Kv) {
                if (a.out_f32) ((float *)a.o)[ooff + dd] = s;
                else ((__bf16 *)a.o)[ooff + dd] = (__bf16)s;
            }
        }
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_merge(const MergeArgs &a, hipStream_t stream) {
    const int64_t rows = (int64_t)a.B * a.M * a.Htot;
    if (rows <= 0) return hipSuccess;
    if (rows > 0x7fffffff) return hipErrorInvalidConfiguration;
    const int per = (a.S + GROUPS - 1) / GROUPS;
    if (per <= 1) hipLaunchKernelGGL(merge_kernel<1>, dim3((unsigned)rows), dim3(NT), 0, stream, a);
    else if (per <= 2) hipLaunchKernelGGL(merge_kernel<2>, dim3((unsigned)rows), dim3(NT), 0, stream, a);
    else if (per <= 4) hipLaunchKernelGGL(merge_kernel<4>, dim3((unsigned)rows), dim3(NT), 0, stream, a);
    else if (per <= 8) hipLaunchKernelGGL(merge_kernel<8>, dim3((unsigned)rows), dim3(NT), 0, stream, a);
    else hipLaunchKernelGGL(merge_kernel<MAXPER>, dim3((unsigned)rows), dim3(NT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace attn
