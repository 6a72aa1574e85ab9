// Fused attention forward for fp32 inputs (vector ALU, fp32 throughout).
//
// Same operation as the bf16 kernel (MSLK kernel reference, "Attention - Core
// fMHA": memory_efficient_attention_forward_requires_grad / _partial, with the
// masks of "Attention - Biases & masks"), for head dims up to 128.  Nothing is
// rounded below fp32, so the result tracks the exact softmax to ~1e-6.
//
// Four lanes share a query row, each holding every fourth 16-byte chunk of q and of the
// output row, so a wave covers 16 rows; a row's dot product is the four lanes' partial sums
// combined by two quad permutations (every lane ends with the same, bitwise identical sum).
// One workgroup = 8 waves (4 when a head dim exceeds 64, for LDS) over the same 16 rows;
// the keys are dealt out in 16-key tiles round-robin over the waves, so the waves run
// independent online softmaxes over disjoint key subsets.  Each wave stages its own tiles
// in LDS; the 16 rows of a wave then read the same key row (an LDS broadcast) and the four
// lanes of a row read neighbouring chunks.  At the end the waves' (m, l, o) states are
// combined exactly, as in the merge of key chunks ("Exact softmax merge" in the site's
// Quick start): pairwise rounds through LDS.
#include "kernels.h"

namespace attn {
namespace {

constexpr float kLn2 = 0.69314718055994530942f;
// waves per workgroup, each with its own key subset: 8, or 4 when a head dim exceeds 64 (the
// per-wave K and V tiles then take twice the LDS)
template <int KD, int KVD>
constexpr int nwaves() { return KD + KVD <= 128 ? 8 : 4; }
constexpr int TB = 16;   // keys per tile
constexpr int RPW = 16;  // query rows per wave and workgroup (four lanes per row)

// Rows [0, TB) x columns [0, N) of a row-major tile at `src` (row stride `stride` floats) into
// LDS, rows >= nrows and columns >= ncols as zeros.  Every load of the tile is issued before
// the first LDS store (16-byte loads where the four columns are valid, single floats at the
// column tail), so a tile costs one memory round trip.
template <int N>
__device__ __forceinline__ void stage_tile(const float *src, int64_t stride, int nrows, int ncols, float *dst, int lane) {
    constexpr int C4 = N / 4, CNT = TB * C4 / 64;
    static_assert(CNT * 64 == TB * C4, "tile split");
    float4 r[CNT];
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
        const int idx = lane + 64 * i, row = idx / C4, c = 4 * (idx % C4);
        const float *p = src + (int64_t)row * stride + c;
        if (row < nrows && c + 4 <= ncols) {
            r[i] = *(const float4 *)p;
        } else {
            r[i].x = (row < nrows && c < ncols) ? p[0] : 0.f;
            r[i].y = (row < nrows && c + 1 < ncols) ? p[1] : 0.f;
            r[i].z = (row < nrows && c + 2 < ncols) ? p[2] : 0.f;
            r[i].w = (row < nrows && c + 3 < ncols) ? p[3] : 0.f;
        }
    }
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
        const int idx = lane + 64 * i;
        *(float4 *)&dst[(idx / C4) * N + 4 * (idx % C4)] = r[i];
    }
}

// Sum over the four lanes of a quad (DPP quad permutations [1,0,3,2] then [2,3,0,1]); the
// additions pair the same operands in every lane, so all four get the same bits.
__device__ __forceinline__ float quad_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
    return x;
}

// 4 floats of row `p` at column d (d a multiple of 4), zeros past n columns
__device__ __forceinline__ float4 load4(const float *p, int d, int n) {
    if (d + 4 <= n) return *(const float4 *)(p + d);
    float4 r;
    r.x = d < n ? p[d] : 0.f;
    r.y = d + 1 < n ? p[d + 1] : 0.f;
    r.z = d + 2 < n ? p[d + 2] : 0.f;
    r.w = d + 3 < n ? p[d + 3] : 0.f;
    return r;
}

template <int KD, int KVD>
__global__ __launch_bounds__((nwaves<KD, KVD>() * 64)) void fwd_f32_kernel(FwdArgs a) {
    constexpr int NWV = nwaves<KD, KVD>();
    constexpr int TILE_FLOATS = TB * (KD + KVD);
    constexpr int KC = KD / 16, VC = KVD / 16;  // 16-byte chunks per lane of q and of o
    constexpr int REC = KVD + 4;                // combine record per row: o[KVD], m, l (+2 pad)
    // per-wave K and V tiles; reused at the end for the cross-wave combine
    __shared__ __attribute__((aligned(16))) float smem[NWV * TILE_FLOATS > NWV / 2 * RPW * REC
                                                         ? NWV * TILE_FLOATS
                                                         : NWV / 2 * RPW * REC];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane >> 2, qd = lane & 3;  // row of the wave, chunk phase of the lane
    const int BH = a.B * a.Htot;
    const int tiles = (a.max_seqlen_q + RPW - 1) / RPW;
    int id = blockIdx.x;
    const int bh = id % BH;
    id /= BH;
    const int seq = id % a.nseq;
    const int tile = tiles - 1 - id / a.nseq;
    const int b = bh / a.Htot, hf = bh % a.Htot;

    int qs = 0, qe = a.Mq, kst = 0, ke = a.Mkv;
    if (a.packed) {
        const int32_t *skp = a.seqstart_k ? a.seqstart_k : a.seqstart_q;
        qs = min(max(a.seqstart_q[seq], 0), a.Mq);
        qe = min(max(a.seqstart_q[seq + 1], qs), a.Mq);
        kst = min(max(skp[seq], 0), a.Mkv);
        ke = min(max(skp[seq + 1], kst), a.Mkv);
    }
    const int Lq = qe - qs, Lk = ke - kst;
    const int row0 = tile * RPW;
    if (tile < 0 || row0 >= Lq) return;
    // visible keys of local row i: [i + shift - wl, i + shift + wr] within [0, Lk)
    const int64_t shift = a.bottom_right ? (int64_t)Lk - Lq : 0;
    auto clampk = [&](int64_t x, int64_t lo_, int64_t hi_) { return (int)(x < lo_ ? lo_ : (x > hi_ ? hi_ : x)); };
    const int row_last = min(row0 + RPW, Lq) - 1;
    const int kbeg = clampk((int64_t)row0 + shift - a.wl, 0, Lk);
    const int kend = max(kbeg, clampk((int64_t)row_last + shift + a.wr + 1, 0, Lk));

    const float *qp = (const float *)a.q + (int64_t)b * a.sq.b + head_offset(a.sq, hf, a.Hin) + (int64_t)qs * a.sq.m;
    const float *kp = (const float *)a.k + (int64_t)b * a.sk.b + head_offset(a.sk, hf, a.Hin) + (int64_t)kst * a.sk.m;
    const float *vp = (const float *)a.v + (int64_t)b * a.sv.b + head_offset(a.sv, hf, a.Hin) + (int64_t)kst * a.sv.m;

    const int qrow = row0 + r;
    const int klo = clampk((int64_t)qrow + shift - a.wl, 0, Lk);
    const int khi = clampk((int64_t)qrow + shift + a.wr, -1, Lk - 1);
    // chunk i of this lane covers columns 16 i + 4 qd .. + 3
    float4 q[KC];
#pragma unroll
    for (int i = 0; i < KC; ++i)
        q[i] = qrow < Lq ? load4(qp + (int64_t)qrow * a.sq.m, 16 * i + 4 * qd, a.K) : float4{0.f, 0.f, 0.f, 0.f};

    float4 o[VC];
#pragma unroll
    for (int i = 0; i < VC; ++i) o[i] = float4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    const float c = a.scale_log2;
    float *ks_ = smem + wave * TILE_FLOATS;  // [TB][KD]
    float *vs_ = ks_ + TB * KD;              // [TB][KVD]

    const int rounds = (kend - kbeg + NWV * TB - 1) / (NWV * TB);
    for (int it = 0; it < rounds; ++it) {
        const int kt0 = kbeg + (it * NWV + wave) * TB;  // this wave's tile
        __syncthreads();                          // previous tile fully read
        const int nrows = min(TB, kend - kt0);    // <= 0: this wave has no tile this round
        stage_tile<KD>(kp + (int64_t)kt0 * a.sk.m, a.sk.m, nrows, a.K, ks_, lane);
        stage_tile<KVD>(vp + (int64_t)kt0 * a.sv.m, a.sv.m, nrows, a.Kv, vs_, lane);
        __syncthreads();
        if (kt0 >= kend) continue;

        float s[TB];
#pragma unroll
        for (int j = 0; j < TB; ++j) {
            float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < KC; ++i) {
                const float4 kk = *(const float4 *)&ks_[j * KD + 16 * i + 4 * qd];
                acc[0] = fmaf(q[i].x, kk.x, acc[0]);
                acc[1] = fmaf(q[i].y, kk.y, acc[1]);
                acc[2] = fmaf(q[i].z, kk.z, acc[2]);
                acc[3] = fmaf(q[i].w, kk.w, acc[3]);
            }
            s[j] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
        }
        float mt = -INFINITY;
#pragma unroll
        for (int j = 0; j < TB; ++j) {
            const int key = kt0 + j;
            float x = quad_sum(s[j]) * c;
            if (key < klo || key > khi) x = -INFINITY;
            s[j] = x;
            mt = fmaxf(mt, x);
        }
        const float m_new = fmaxf(m_run, mt);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = exp2f(m_run - m_use);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < VC; ++i) {
            o[i].x *= alpha;
            o[i].y *= alpha;
            o[i].z *= alpha;
            o[i].w *= alpha;
        }
#pragma unroll
        for (int j = 0; j < TB; ++j) {
            const float p = exp2f(s[j] - m_use);
            l_run += p;
#pragma unroll
            for (int i = 0; i < VC; ++i) {
                const float4 vv = *(const float4 *)&vs_[j * KVD + 16 * i + 4 * qd];
                o[i].x = fmaf(p, vv.x, o[i].x);
                o[i].y = fmaf(p, vv.y, o[i].y);
                o[i].z = fmaf(p, vv.z, o[i].z);
                o[i].w = fmaf(p, vv.w, o[i].w);
            }
        }
    }

    // exact combine of the waves' states, pairwise: waves [step, 2 step) -> [0, step)
#pragma unroll
    for (int step = NWV / 2; step >= 1; step >>= 1) {
        __syncthreads();
        if (wave >= step && wave < 2 * step) {
            float *rec = smem + ((wave - step) * RPW + r) * REC;
#pragma unroll
            for (int i = 0; i < VC; ++i) *(float4 *)&rec[16 * i + 4 * qd] = o[i];
            if (qd == 0) {
                rec[KVD] = m_run;
                rec[KVD + 1] = l_run;
            }
        }
        __syncthreads();
        if (wave < step) {
            const float *rec = smem + (wave * RPW + r) * REC;
            const float m2 = rec[KVD], l2 = rec[KVD + 1];
            const float mm = fmaxf(m_run, m2);
            const float mu = (mm == -INFINITY) ? 0.f : mm;
            const float a1 = exp2f(m_run - mu), a2 = exp2f(m2 - mu);
#pragma unroll
            for (int i = 0; i < VC; ++i) {
                const float4 x = *(const float4 *)&rec[16 * i + 4 * qd];
                o[i].x = o[i].x * a1 + x.x * a2;
                o[i].y = o[i].y * a1 + x.y * a2;
                o[i].z = o[i].z * a1 + x.z * a2;
                o[i].w = o[i].w * a1 + x.w * a2;
            }
            l_run = l_run * a1 + l2 * a2;
            m_run = mm;
        }
    }

    if (wave == 0 && qrow < Lq) {
        const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
        float *op = (float *)a.o + (int64_t)b * a.so.b + head_offset(a.so, hf, a.Hin) + (int64_t)(qs + qrow) * a.so.m;
#pragma unroll
        for (int i = 0; i < VC; ++i) {
            const int d = 16 * i + 4 * qd;
            const float4 x = float4{o[i].x * inv, o[i].y * inv, o[i].z * inv, o[i].w * inv};
            if (d + 4 <= a.Kv) {
                *(float4 *)(op + d) = x;
            } else {
                if (d < a.Kv) op[d] = x.x;
                if (d + 1 < a.Kv) op[d + 1] = x.y;
                if (d + 2 < a.Kv) op[d + 2] = x.z;
            }
        }
        if (a.lse && qd == 0)
            a.lse[((int64_t)b * a.Htot + hf) * a.Mq + qs + qrow] =
                l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
    }
}

template <int KD, int KVD>
hipError_t launch(const FwdArgs &a, hipStream_t stream) {
    const int64_t tiles = (a.max_seqlen_q + RPW - 1) / RPW;
    const int64_t grid = tiles * a.nseq * (int64_t)a.B * a.Htot;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((fwd_f32_kernel<KD, KVD>), dim3((unsigned)grid), dim3(nwaves<KD, KVD>() * 64), 0, stream, a);
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
