// Exact LSE-weighted merge of attention results over disjoint key chunks
// (MSLK kernel reference, "Attention - Core fMHA": merge_attentions; "MSLK
// Kernel Library -- Complete Reference", Quick start, "Exact softmax merge").
//
// For every output row (b, m, head): M* = max_c lse_c, L = M* + ln sum_c
// exp(lse_c - M*), out = sum_c exp(lse_c - L) out_c.  A chunk at -inf weighs 0;
// all chunks at -inf give out = 0 and lse = -inf.
//
// One wave per row.  The per-row LSE values are wave-uniform (scalar loads); the
// lanes split the value dimension, so each chunk row is one coalesced read.
// Memory-bound: every chunk element is read once, every output written once.
#include "kernels.h"

namespace attn {
namespace {

constexpr int WAVES = 4;

__global__ __launch_bounds__(WAVES * 64) void merge_kernel(MergeArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * WAVES + (threadIdx.x >> 6);
    const int64_t rows = (int64_t)a.B * a.M * a.Htot;
    if (row >= rows) return;
    const int hf = (int)(row % a.Htot);
    const int m = (int)((row / a.Htot) % a.M);
    const int b = (int)(row / ((int64_t)a.Htot * a.M));
    const int64_t loff = ((int64_t)b * a.Htot + hf) * a.M + m;
    const int64_t coff = (int64_t)b * a.sc.b + (int64_t)m * a.sc.m + head_offset(a.sc, hf, a.Hin);
    const int64_t ooff = (int64_t)b * a.so.b + (int64_t)m * a.so.m + head_offset(a.so, hf, a.Hin);

    float mx = -INFINITY;
    for (int c = 0; c < a.S; ++c) mx = fmaxf(mx, a.lse[c][loff]);

    if (mx == -INFINITY) {
        for (int d = lane; d < a.Kv; d += 64) {
            if (a.out_f32) ((float *)a.o)[ooff + d] = 0.f;
            else ((__bf16 *)a.o)[ooff + d] = (__bf16)0.f;
        }
        if (a.lse_out && lane == 0) a.lse_out[loff] = -INFINITY;
        return;
    }
    float sum = 0.f;
    for (int c = 0; c < a.S; ++c) sum += expf(a.lse[c][loff] - mx);
    const float L = mx + logf(sum);

    for (int d0 = 0; d0 < a.Kv; d0 += 64) {
        const int d = d0 + lane;
        float acc = 0.f;
        if (d < a.Kv) {
            for (int c = 0; c < a.S; ++c) {
                const float w = expf(a.lse[c][loff] - L);
                const float x = a.chunk_f32 ? ((const float *)a.chunk[c])[coff + d]
                                            : (float)((const __bf16 *)a.chunk[c])[coff + d];
                acc = fmaf(w, x, acc);
            }
            if (a.out_f32) ((float *)a.o)[ooff + d] = acc;
            else ((__bf16 *)a.o)[ooff + d] = (__bf16)acc;
        }
    }
    if (a.lse_out && lane == 0) a.lse_out[loff] = L;
}

}  // namespace

hipError_t launch_merge(const MergeArgs &a, hipStream_t stream) {
    const int64_t rows = (int64_t)a.B * a.M * a.Htot;
    if (rows <= 0) return hipSuccess;
    const int64_t grid = (rows + WAVES - 1) / WAVES;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(merge_kernel, dim3((unsigned)grid), dim3(WAVES * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace attn
