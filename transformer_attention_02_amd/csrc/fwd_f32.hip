// Fused attention forward for fp32 inputs (vector ALU, fp32 throughout).
//
// Same operation as the bf16 kernel (MSLK kernel reference, "Attention - Core
// fMHA": memory_efficient_attention_forward_requires_grad / _partial, with the
// masks of "Attention - Biases & masks"), for head dims up to 128.  Nothing is
// rounded below fp32, so the result tracks the exact softmax to ~1e-6.
//
// One wave per workgroup, one query row per lane (64 rows per workgroup).
// Keys stream through LDS in tiles of 32; every lane reads the same key row at
// the same time (an LDS broadcast).  Per tile: 32 scores, one max, one rescale
// of the running output, 32 exponentials.
#include "kernels.h"

namespace attn {
namespace {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr int TB = 32;  // keys per tile
constexpr int BM = 64;  // query rows per workgroup

template <int KD, int KVD>
__global__ __launch_bounds__(64) void fwd_f32_kernel(FwdArgs a) {
    __shared__ __attribute__((aligned(16))) float ks_[TB][KD];
    __shared__ __attribute__((aligned(16))) float vs_[TB][KVD];

    const int tid = threadIdx.x;
    const int BH = a.B * a.Htot;
    const int tiles = (a.max_seqlen_q + BM - 1) / BM;
    int id = blockIdx.x;
    const int bh = id % BH;
    id /= BH;
    const int seq = id % a.nseq;
    const int tile = tiles - 1 - id / a.nseq;
    const int b = bh / a.Htot, hf = bh % a.Htot;

    int qs = 0, qe = a.Mq, kst = 0, ke = a.Mkv;
    if (a.mask >= kMaskBlockDiag) {
        const int32_t *skp = a.seqstart_k ? a.seqstart_k : a.seqstart_q;
        qs = min(max(a.seqstart_q[seq], 0), a.Mq);
        qe = min(max(a.seqstart_q[seq + 1], qs), a.Mq);
        kst = min(max(skp[seq], 0), a.Mkv);
        ke = min(max(skp[seq + 1], kst), a.Mkv);
    }
    const int Lq = qe - qs, Lk = ke - kst;
    const int row0 = tile * BM;
    if (tile < 0 || row0 >= Lq) return;
    const bool causal = (a.mask == kMaskCausal || a.mask == kMaskBlockDiagCausal);
    const int nkeys = causal ? min(Lk, row0 + BM) : Lk;

    const float *qp = (const float *)a.q + (int64_t)b * a.sq.b + head_offset(a.sq, hf, a.Hin) + (int64_t)qs * a.sq.m;
    const float *kp = (const float *)a.k + (int64_t)b * a.sk.b + head_offset(a.sk, hf, a.Hin) + (int64_t)kst * a.sk.m;
    const float *vp = (const float *)a.v + (int64_t)b * a.sv.b + head_offset(a.sv, hf, a.Hin) + (int64_t)kst * a.sv.m;

    const int qrow = row0 + tid;
    float q[KD];
#pragma unroll
    for (int d = 0; d < KD; ++d) q[d] = (qrow < Lq && d < a.K) ? qp[(int64_t)qrow * a.sq.m + d] : 0.f;

    float o[KVD];
#pragma unroll
    for (int d = 0; d < KVD; ++d) o[d] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    const float c = a.scale_log2;

    for (int kt0 = 0; kt0 < nkeys; kt0 += TB) {
        __syncthreads();
        for (int idx = tid; idx < TB * KD; idx += 64) {
            const int r = idx / KD, d = idx % KD, j = kt0 + r;
            ks_[r][d] = (j < Lk && d < a.K) ? kp[(int64_t)j * a.sk.m + d] : 0.f;
        }
        for (int idx = tid; idx < TB * KVD; idx += 64) {
            const int r = idx / KVD, d = idx % KVD, j = kt0 + r;
            vs_[r][d] = (j < Lk && d < a.Kv) ? vp[(int64_t)j * a.sv.m + d] : 0.f;
        }
        __syncthreads();

        float s[TB];
        float mt = -INFINITY;
#pragma unroll
        for (int j = 0; j < TB; ++j) {
            float dot = 0.f;
#pragma unroll
            for (int d = 0; d < KD; d += 4) {
                const float4 kk = *(const float4 *)&ks_[j][d];
                dot = fmaf(q[d], kk.x, dot);
                dot = fmaf(q[d + 1], kk.y, dot);
                dot = fmaf(q[d + 2], kk.z, dot);
                dot = fmaf(q[d + 3], kk.w, dot);
            }
            const int key = kt0 + j;
            float x = dot * c;
            if (key >= nkeys || (causal && key > qrow)) x = -INFINITY;
            s[j] = x;
            mt = fmaxf(mt, x);
        }
        const float m_new = fmaxf(m_run, mt);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = exp2f(m_run - m_use);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int d = 0; d < KVD; ++d) o[d] *= alpha;
#pragma unroll
        for (int j = 0; j < TB; ++j) {
            const float p = exp2f(s[j] - m_use);
            l_run += p;
#pragma unroll
            for (int d = 0; d < KVD; d += 4) {
                const float4 vv = *(const float4 *)&vs_[j][d];
                o[d] = fmaf(p, vv.x, o[d]);
                o[d + 1] = fmaf(p, vv.y, o[d + 1]);
                o[d + 2] = fmaf(p, vv.z, o[d + 2]);
                o[d + 3] = fmaf(p, vv.w, o[d + 3]);
            }
        }
    }

    if (qrow < Lq) {
        const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
        float *op = (float *)a.o + (int64_t)b * a.so.b + head_offset(a.so, hf, a.Hin) + (int64_t)(qs + qrow) * a.so.m;
#pragma unroll
        for (int d = 0; d < KVD; ++d)
            if (d < a.Kv) op[d] = o[d] * inv;
        if (a.lse)
            a.lse[((int64_t)b * a.Htot + hf) * a.Mq + qs + qrow] =
                l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
    }
}

template <int KD, int KVD>
hipError_t launch(const FwdArgs &a, hipStream_t stream) {
    const int64_t tiles = (a.max_seqlen_q + BM - 1) / BM;
    const int64_t grid = tiles * a.nseq * (int64_t)a.B * a.Htot;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((fwd_f32_kernel<KD, KVD>), dim3((unsigned)grid), dim3(64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs &a, hipStream_t stream) {
    const bool k64 = a.K <= 64, v64 = a.Kv <= 64;
    if (k64 && v64) return launch<64, 64>(a, stream);
    if (k64) return launch<64, 128>(a, stream);
    if (v64) return launch<128, 64>(a, stream);
    return launch<128, 128>(a, stream);
}

}  // namespace attn
