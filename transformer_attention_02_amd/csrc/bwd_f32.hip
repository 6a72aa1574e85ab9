// Fused attention backward for fp32 inputs (vector ALU, fp32 throughout).
//
// Same operation as the bf16 backward (MSLK kernel reference, "Attention - Core fMHA":
// memory_efficient_attention_backward; masks from "Attention - Biases & masks"), for head
// dims up to 128, with nothing rounded below fp32:
//   P_ij = exp(scale q_i.k_j - lse_i) on the visible keys, D_i = dout_i.out_i,
//   dv_j = sum_i P_ij dout_i,  dS_ij = P_ij (dout_i.v_j - D_i),
//   dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i.
//
// Two launches, both with four lanes per stationary row (each lane holds a quarter of the
// row's head dims, so the row's dot products are a lane sum plus two shuffles):
//   1. bwd_f32_dq_kernel: 64 query rows per workgroup; 16-key tiles of K and V staged in
//      LDS (every lane of a quarter then reads the same key row: an LDS broadcast).  Each
//      row first forms D_i and the base-2 LSE (+inf for a row with no visible key) and
//      stores them for the second launch.
//   2. bwd_f32_dkdv_kernel: 64 keys per workgroup; 16-row tiles of Q, dout, L and D staged
//      in LDS.
#include "kernels.h"

namespace attn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int RL = 4;           // lanes per stationary row
constexpr int NT = 256;         // threads per workgroup
constexpr int ROWS = NT / RL;   // stationary rows per workgroup
constexpr int TT = 16;          // streamed rows per LDS tile

__device__ __forceinline__ int clampk(int64_t x, int64_t lo, int64_t hi) {
    return (int)(x < lo ? lo : (x > hi ? hi : x));
}

__device__ __forceinline__ void seq_bounds(const BwdArgs &a, int seq, int &qs, int &qe, int &ks, int &ke) {
    qs = 0, qe = a.Mq, ks = 0, ke = a.Mkv;
    if (a.packed) {
        const int32_t *skp = a.seqstart_k ? a.seqstart_k : a.seqstart_q;
        qs = min(max(a.seqstart_q[seq], 0), a.Mq);
        qe = min(max(a.seqstart_q[seq + 1], qs), a.Mq);
        ks = min(max(skp[seq], 0), a.Mkv);
        ke = min(max(skp[seq + 1], ks), a.Mkv);
    }
}

// Sum over the RL lanes of a row.
__device__ __forceinline__ float row_sum(float x) {
    x += __shfl_xor(x, 1, 64);
    x += __shfl_xor(x, 2, 64);
    return x;
}

// ------------------------------------------------------------------ 1. dq (and D, L per row)

template <int KD, int KVD>
__global__ __launch_bounds__(NT) void bwd_f32_dq_kernel(BwdArgs a) {
    constexpr int QK = KD / RL, QV = KVD / RL;  // head-dim elements per lane
    __shared__ __attribute__((aligned(16))) float ks_[TT][KD];
    __shared__ __attribute__((aligned(16))) float vs_[TT][KVD];

    const int tid = threadIdx.x, r = tid / RL, part = tid % RL;
    const int BH = a.B * a.Htot;
    const int tiles = (a.max_seqlen_q + ROWS - 1) / ROWS;
    int id = blockIdx.x;
    const int bh = id % BH;
    id /= BH;
    const int seq = id % a.nseq;
    const int tile = tiles - 1 - id / a.nseq;
    const int b = bh / a.Htot, hf = bh % a.Htot;
    int qs, qe, ks, ke;
    seq_bounds(a, seq, qs, qe, ks, ke);
    const int Lq = qe - qs, Lk = ke - ks;
    const int row0 = tile * ROWS;
    if (tile < 0 || row0 >= Lq) return;
    const int64_t shift = a.bottom_right ? (int64_t)Lk - Lq : 0;
    const int row_last = min(row0 + ROWS, Lq) - 1;
    const int kbeg = clampk((int64_t)row0 + shift - a.wl, 0, Lk);
    const int kend = max(kbeg, clampk((int64_t)row_last + shift + a.wr + 1, 0, Lk));

    const int qrow = row0 + r;
    const bool live = qrow < Lq;
    const int klo = clampk((int64_t)qrow + shift - a.wl, 0, Lk);
    const int khi = clampk((int64_t)qrow + shift + a.wr, -1, Lk - 1);
    const int64_t qoff = (int64_t)b * a.sq.b + head_offset(a.sq, hf, a.Hin) + (int64_t)(qs + qrow) * a.sq.m;
    const int64_t ooff = (int64_t)b * a.so.b + head_offset(a.so, hf, a.Hin) + (int64_t)(qs + qrow) * a.so.m;
    const int64_t goff = (int64_t)b * a.sdo.b + head_offset(a.sdo, hf, a.Hin) + (int64_t)(qs + qrow) * a.sdo.m;
    const float *kp = (const float *)a.k + (int64_t)b * a.sk.b + head_offset(a.sk, hf, a.Hin) + (int64_t)ks * a.sk.m;
    const float *vp = (const float *)a.v + (int64_t)b * a.sv.b + head_offset(a.sv, hf, a.Hin) + (int64_t)ks * a.sv.m;

    float q[QK], g[QV], dq[QK];
    float dd = 0.f;
#pragma unroll
    for (int e = 0; e < QK; ++e) {
        const int d = part * QK + e;
        q[e] = (live && d < a.D) ? ((const float *)a.q)[qoff + d] : 0.f;
        dq[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < QV; ++e) {
        const int d = part * QV + e;
        const bool ok = live && d < a.Dv;
        g[e] = ok ? ((const float *)a.dout)[goff + d] : 0.f;
        dd = fmaf(g[e], ok ? ((const float *)a.o)[ooff + d] : 0.f, dd);
    }
    dd = row_sum(dd);
    float l2 = INFINITY;
    if (live) {
        const int64_t w = ((int64_t)b * a.Htot + hf) * a.Mq + qs + qrow;
        const float lse = a.lse[w];
        l2 = lse == -INFINITY ? INFINITY : lse * kLog2e;
        if (part == 0) {
            a.ws_d[w] = dd;
            a.ws_l2[w] = l2;
        }
    }
    const float c = a.scale_log2;

    for (int kt0 = kbeg; kt0 < kend; kt0 += TT) {
        __syncthreads();  // the previous tile is no longer read
        for (int i = tid; i < TT * KD; i += NT) {
            const int j = i / KD, d = i % KD;
            ks_[j][d] = (kt0 + j < kend && d < a.D) ? kp[(int64_t)(kt0 + j) * a.sk.m + d] : 0.f;
        }
        for (int i = tid; i < TT * KVD; i += NT) {
            const int j = i / KVD, d = i % KVD;
            vs_[j][d] = (kt0 + j < kend && d < a.Dv) ? vp[(int64_t)(kt0 + j) * a.sv.m + d] : 0.f;
        }
        __syncthreads();
        for (int j = 0; j < TT; ++j) {
            float s = 0.f, dp = 0.f;
#pragma unroll
            for (int e = 0; e < QK; ++e) s = fmaf(q[e], ks_[j][part * QK + e], s);
#pragma unroll
            for (int e = 0; e < QV; ++e) dp = fmaf(g[e], vs_[j][part * QV + e], dp);
            s = row_sum(s);
            dp = row_sum(dp);
            const int key = kt0 + j;
            const float p = (key >= klo && key <= khi) ? exp2f(fmaf(s, c, -l2)) : 0.f;
            const float ds = p * (dp - dd);
#pragma unroll
            for (int e = 0; e < QK; ++e) dq[e] = fmaf(ds, ks_[j][part * QK + e], dq[e]);
        }
    }

    if (live) {
        float *dqp = (float *)a.dq + (int64_t)b * a.sdq.b + head_offset(a.sdq, hf, a.Hin) + (int64_t)(qs + qrow) * a.sdq.m;
#pragma unroll
        for (int e = 0; e < QK; ++e) {
            const int d = part * QK + e;
            if (d < a.D) dqp[d] = dq[e] * a.scale;
        }
    }
}

// ------------------------------------------------------------------ 2. dk and dv

template <int KD, int KVD>
__global__ __launch_bounds__(NT) void bwd_f32_dkdv_kernel(BwdArgs a) {
    constexpr int QK = KD / RL, QV = KVD / RL;
    __shared__ __attribute__((aligned(16))) float qs_[TT][KD];
    __shared__ __attribute__((aligned(16))) float gs_[TT][KVD];
    __shared__ float ls_[TT], ds_[TT];

    const int tid = threadIdx.x, r = tid / RL, part = tid % RL;
    const int BH = a.B * a.Htot;
    int id = blockIdx.x;
    const int bh = id % BH;
    id /= BH;
    const int seq = id % a.nseq;
    const int ktile = id / a.nseq;
    const int b = bh / a.Htot, hf = bh % a.Htot;
    int qs, qe, ks, ke;
    seq_bounds(a, seq, qs, qe, ks, ke);
    const int Lq = qe - qs, Lk = ke - ks;
    const int k0 = ktile * ROWS;
    if (k0 >= Lk) return;
    const int k1 = min(k0 + ROWS, Lk);
    const int64_t shift = a.bottom_right ? (int64_t)Lk - Lq : 0;
    const int qbeg = clampk((int64_t)k0 - shift - a.wr, 0, Lq);
    const int qend = max(qbeg, clampk((int64_t)k1 - 1 - shift + a.wl + 1, 0, Lq));

    const int key = k0 + r;
    const bool live = key < Lk;
    const int qlo = clampk((int64_t)key - shift - a.wr, 0, Lq);
    const int qhi = clampk((int64_t)key - shift + a.wl, -1, Lq - 1);
    const int64_t koff = (int64_t)b * a.sk.b + head_offset(a.sk, hf, a.Hin) + (int64_t)(ks + key) * a.sk.m;
    const int64_t voff = (int64_t)b * a.sv.b + head_offset(a.sv, hf, a.Hin) + (int64_t)(ks + key) * a.sv.m;
    const float *qp = (const float *)a.q + (int64_t)b * a.sq.b + head_offset(a.sq, hf, a.Hin) + (int64_t)qs * a.sq.m;
    const float *gp = (const float *)a.dout + (int64_t)b * a.sdo.b + head_offset(a.sdo, hf, a.Hin) + (int64_t)qs * a.sdo.m;
    const int64_t wrow = ((int64_t)b * a.Htot + hf) * a.Mq + qs;

    float k[QK], v[QV], dk[QK], dv[QV];
#pragma unroll
    for (int e = 0; e < QK; ++e) {
        const int d = part * QK + e;
        k[e] = (live && d < a.D) ? ((const float *)a.k)[koff + d] : 0.f;
        dk[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < QV; ++e) {
        const int d = part * QV + e;
        v[e] = (live && d < a.Dv) ? ((const float *)a.v)[voff + d] : 0.f;
        dv[e] = 0.f;
    }
    const float c = a.scale_log2;

    for (int qt0 = qbeg; qt0 < qend; qt0 += TT) {
        __syncthreads();
        for (int i = tid; i < TT * KD; i += NT) {
            const int j = i / KD, d = i % KD;
            qs_[j][d] = (qt0 + j < qend && d < a.D) ? qp[(int64_t)(qt0 + j) * a.sq.m + d] : 0.f;
        }
        for (int i = tid; i < TT * KVD; i += NT) {
            const int j = i / KVD, d = i % KVD;
            gs_[j][d] = (qt0 + j < qend && d < a.Dv) ? gp[(int64_t)(qt0 + j) * a.sdo.m + d] : 0.f;
        }
        if (tid < TT) {
            const bool ok = qt0 + tid < qend;
            ls_[tid] = ok ? a.ws_l2[wrow + qt0 + tid] : INFINITY;
            ds_[tid] = ok ? a.ws_d[wrow + qt0 + tid] : 0.f;
        }
        __syncthreads();
        for (int i = 0; i < TT; ++i) {
            float s = 0.f, dp = 0.f;
#pragma unroll
            for (int e = 0; e < QK; ++e) s = fmaf(k[e], qs_[i][part * QK + e], s);
#pragma unroll
            for (int e = 0; e < QV; ++e) dp = fmaf(v[e], gs_[i][part * QV + e], dp);
            s = row_sum(s);
            dp = row_sum(dp);
            const int q = qt0 + i;
            const float p = (q >= qlo && q <= qhi) ? exp2f(fmaf(s, c, -ls_[i])) : 0.f;
            const float dsv = p * (dp - ds_[i]);
#pragma unroll
            for (int e = 0; e < QV; ++e) dv[e] = fmaf(p, gs_[i][part * QV + e], dv[e]);
#pragma unroll
            for (int e = 0; e < QK; ++e) dk[e] = fmaf(dsv, qs_[i][part * QK + e], dk[e]);
        }
    }

    if (live) {
        float *dkp = (float *)a.dk + (int64_t)b * a.sdk.b + head_offset(a.sdk, hf, a.Hin) + (int64_t)(ks + key) * a.sdk.m;
        float *dvp = (float *)a.dv + (int64_t)b * a.sdv.b + head_offset(a.sdv, hf, a.Hin) + (int64_t)(ks + key) * a.sdv.m;
#pragma unroll
        for (int e = 0; e < QK; ++e) {
            const int d = part * QK + e;
            if (d < a.D) dkp[d] = dk[e] * a.scale;
        }
#pragma unroll
        for (int e = 0; e < QV; ++e) {
            const int d = part * QV + e;
            if (d < a.Dv) dvp[d] = dv[e];
        }
    }
}

template <int KD, int KVD>
hipError_t launch(const BwdArgs &a, hipStream_t stream) {
    const int64_t gq = (int64_t)((a.max_seqlen_q + ROWS - 1) / ROWS) * a.nseq * a.B * a.Htot;
    const int64_t gkv = (int64_t)((a.max_seqlen_k + ROWS - 1) / ROWS) * a.nseq * a.B * a.Htot;
    if (gq > 0x7fffffff || gkv > 0x7fffffff) return hipErrorInvalidConfiguration;
    // the dq launch writes the per-row D and L that the dk/dv launch reads
    if (gq > 0) hipLaunchKernelGGL((bwd_f32_dq_kernel<KD, KVD>), dim3((unsigned)gq), dim3(NT), 0, stream, a);
    if (gkv > 0) hipLaunchKernelGGL((bwd_f32_dkdv_kernel<KD, KVD>), dim3((unsigned)gkv), dim3(NT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_f32(const BwdArgs &a, hipStream_t stream) {
    const bool k64 = a.D <= 64, v64 = a.Dv <= 64;
    if (k64 && v64) return launch<64, 64>(a, stream);
    if (k64) return launch<64, 128>(a, stream);
    if (v64) return launch<128, 64>(a, stream);
    return launch<128, 128>(a, stream);
}

}  // namespace attn
