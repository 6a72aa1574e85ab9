// Split-KV decode: per-chunk partial attention for one query row per (batch, head)
// ("MSLK Kernel Library -- Complete Reference", Glossary, split-K / split-KV:
// parallelise the reduction over the KV sequence, then combine partials; the
// chunk results are exactly those of memory_efficient_attention_partial on
// each key chunk, and the merge kernel combines them).
//
// The work is a stream over the K/V cache, about one flop per byte, so the
// kernel is built for HBM bandwidth, not for the matrix cores:
//   * one workgroup (4 waves) per (chunk, batch, head); consecutive workgroups
//     are consecutive heads of the same chunk, so neighbouring workgroups read
//     neighbouring bytes of the [B, Mkv, H, D] cache;
//   * a key row (D elements) is read by D/8 lanes (bf16) with 16-byte loads,
//     eight rows per lane in flight before any arithmetic;
//   * phase 1 streams K: q.k per row, reduced across the row's lanes, scores
//     kept in LDS; phase 2 takes the exact max and the exponentials over the
//     chunk (no per-key rescaling); phase 3 streams V and accumulates p v.
//   * chunks longer than the LDS score buffer are cut into sub-chunks combined
//     with the running-max rescale;
//   * KV-cache layouts ("Attention - Biases & masks": BlockDiagonalPaddedKeysMask,
//     PagedBlockDiagonalPaddedKeysMask): per-sequence key counts on the device,
//     and for a paged cache the physical row of every key of a sub-chunk is
//     resolved once into LDS from the block table.
// Output: the chunk's normalised fp32 output and its natural-log LSE; an empty
// chunk gives 0 and -inf.
#include <type_traits>

#include "kernels.h"

namespace attn {
namespace {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr int NT = 256;
constexpr int SUB = 2048;  // scores per sub-chunk held in LDS
constexpr int UNROLL = 8;  // key rows per lane in flight

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <bool F32>
__device__ __forceinline__ void unpack(const u32x4 &w, float *x) {
    if (F32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(w[i]);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(w[i] << 16);
            x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
}

__device__ __forceinline__ float block_max(float x, float *red) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__device__ __forceinline__ float block_sum(float x, float *red) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
}

// MODE 0: k/v [B, Mkv, ...], every sequence has Mkv keys.  MODE 1: padded lanes [B, cap, ...] with
// seqlens[b] valid keys.  MODE 2: paged cache [1, num_pages * page_size, ...]; key j of sequence b is
// row block_tables[b][j / page_size] * page_size + j % page_size (page numbers clamped to the cache).
template <int HD, bool F32, int MODE>
__global__ __launch_bounds__(NT) void decode_kernel(DecodeArgs a) {
    constexpr int EPL = F32 ? 4 : 8;   // elements per 16-byte load
    constexpr int LPK = HD / EPL;      // lanes per key row
    constexpr int KPP = NT / LPK;      // key rows per pass of the workgroup
    using T = typename std::conditional<F32, float, __bf16>::type;

    __shared__ float sc[SUB];
    __shared__ float acc_s[KPP][HD];
    __shared__ float red[4];
    __shared__ int rows_s[MODE == 2 ? SUB : 1];  // physical cache row of each key of the sub-chunk

    int id = blockIdx.x;
    const int hf = id % a.Htot;
    id /= a.Htot;
    const int b = id % a.B;
    const int s = id / a.B;
    const int Lb = MODE == 0 ? a.Mkv : min(max(a.seqlens[b], 0), a.cap);
    const int j0 = min(Lb, s * a.chunk);
    const int j1 = min(Lb, j0 + a.chunk);
    const int64_t kb = MODE == 2 ? 0 : (int64_t)b * a.sk.b, vb = MODE == 2 ? 0 : (int64_t)b * a.sv.b;

    const int tid = threadIdx.x, g = tid / LPK, cl = tid % LPK;
    const T *qp = (const T *)a.q + (int64_t)b * a.sq.b + head_offset(a.sq, hf, a.Hin);
    const T *kp = (const T *)a.k + kb + head_offset(a.sk, hf, a.Hin) + cl * EPL;
    const T *vp = (const T *)a.v + vb + head_offset(a.sv, hf, a.Hin) + cl * EPL;

    float qv[EPL];
    unpack<F32>(*(const u32x4 *)(qp + cl * EPL), qv);
#pragma unroll
    for (int e = 0; e < EPL; ++e) qv[e] *= a.scale_log2;

    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    for (int sub0 = j0; sub0 < j1; sub0 += SUB) {
        const int n = min(SUB, j1 - sub0);
        if (MODE == 2) {
            const int32_t *bt = a.block_tables + (int64_t)b * a.bt_stride;
            for (int i = tid; i < n; i += NT) {
                const int j = sub0 + i;
                const int pg = min(max(bt[j / a.page_size], 0), a.num_pages - 1);
                rows_s[i] = pg * a.page_size + j % a.page_size;
            }
            __syncthreads();
        }
        // phase 1: scores
        for (int p = 0; p < n; p += KPP * UNROLL) {
            u32x4 w[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const int r = p + u * KPP + g;
                const int64_t row = MODE == 2 ? (r < n ? rows_s[r] : 0) : sub0 + r;
                w[u] = r < n ? *(const u32x4 *)(kp + row * a.sk.m) : u32x4{0, 0, 0, 0};
            }
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                float x[EPL];
                unpack<F32>(w[u], x);
                float dot = 0.f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) dot = fmaf(qv[e], x[e], dot);
#pragma unroll
                for (int o = LPK / 2; o >= 1; o >>= 1) dot += __shfl_xor(dot, o, 64);
                const int r = p + u * KPP + g;
                if (cl == 0 && r < n) sc[r] = dot;
            }
        }
        __syncthreads();
        // phase 2: exact max and exponentials over the sub-chunk
        float mt = -INFINITY;
        for (int i = tid; i < n; i += NT) mt = fmaxf(mt, sc[i]);
        mt = block_max(mt, red);
        const float m_new = fmaxf(m_run, mt);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        float ls = 0.f;
        for (int i = tid; i < n; i += NT) {
            const float e = __builtin_amdgcn_exp2f(sc[i] - m_new);
            sc[i] = e;
            ls += e;
        }
        ls = block_sum(ls, red);  // its barriers also publish the exponentials
        l_run = l_run * alpha + ls;
        m_run = m_new;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] *= alpha;
        // phase 3: p-weighted sum of value rows
        for (int p = 0; p < n; p += KPP * UNROLL) {
            u32x4 w[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const int r = p + u * KPP + g;
                const int64_t row = MODE == 2 ? (r < n ? rows_s[r] : 0) : sub0 + r;
                w[u] = r < n ? *(const u32x4 *)(vp + row * a.sv.m) : u32x4{0, 0, 0, 0};
            }
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const int r = p + u * KPP + g;
                const float pr = r < n ? sc[r] : 0.f;
                float x[EPL];
                unpack<F32>(w[u], x);
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[e] = fmaf(pr, x[e], acc[e]);
            }
        }
        __syncthreads();  // sc is rewritten by the next sub-chunk
    }

    // combine the KPP row groups
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc_s[g][cl * EPL + e] = acc[e];
    __syncthreads();
    const int64_t obase = ((int64_t)s * a.B + b) * a.Htot + hf;
    for (int d = tid; d < HD; d += NT) {
        float tot = 0.f;
#pragma unroll
        for (int r = 0; r < KPP; ++r) tot += acc_s[r][d];
        a.ws_o[obase * HD + d] = l_run > 0.f ? tot / l_run : 0.f;
    }
    if (tid == 0) a.ws_lse[obase] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
}

template <int HD, bool F32, int MODE>
hipError_t launch(const DecodeArgs &a, hipStream_t stream) {
    const int64_t grid = (int64_t)a.S * a.B * a.Htot;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((decode_kernel<HD, F32, MODE>), dim3((unsigned)grid), dim3(NT), 0, stream, a);
    return hipGetLastError();
}

template <int HD, bool F32>
hipError_t launch_mode(const DecodeArgs &a, hipStream_t stream) {
    if (a.block_tables) return launch<HD, F32, 2>(a, stream);
    if (a.seqlens) return launch<HD, F32, 1>(a, stream);
    return launch<HD, F32, 0>(a, stream);
}

}  // namespace

hipError_t launch_decode_partials(const DecodeArgs &a, bool f32, hipStream_t stream) {
    if (a.D == 128) return f32 ? launch_mode<128, true>(a, stream) : launch_mode<128, false>(a, stream);
    if (a.D == 64) return f32 ? launch_mode<64, true>(a, stream) : launch_mode<64, false>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace attn
