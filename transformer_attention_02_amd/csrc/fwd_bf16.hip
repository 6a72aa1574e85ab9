// Fused attention forward for bf16 inputs on gfx950 matrix cores.
//
// Computes, per (batch, head) and query row i, out_i = softmax_j(scale q_i.k_j) v_j
// over the visible keys and lse_i = ln sum_j exp(scale q_i.k_j), without ever
// writing the score matrix to memory (MSLK kernel reference, "Attention - Core
// fMHA": memory_efficient_attention_forward_requires_grad and
// memory_efficient_attention_partial; masks from "Attention - Biases & masks":
// LowerTriangularMask, BlockDiagonalMask, BlockDiagonalCausalMask).
//
// Work decomposition
//   One workgroup = NW waves = 32*NW query rows of one (batch, head[, sequence]).
//   Each wave owns 32 query rows.  Key/value tiles of 64 rows stream through
//   LDS, double-buffered: while the waves run the matrix products on tile t,
//   the global loads of tile t+1 are in flight in registers.
//
// Matrix-core layout (v_mfma_f32_32x32x16_bf16, A 32x16, B 16x32, C 32x32)
//   S^T = K Q^T: A = K rows from LDS (m = key, k = head dim), B = Q^T held in
//   registers for the whole kernel (n = query row).  In the C layout lane l
//   owns query row l%32 and 16 keys, so the softmax row statistics need only
//   in-lane reductions plus one exchange with lane l^32.
//   O^T += V^T P^T: B = P^T straight from the S^T registers.  For that to work
//   without a register shuffle, K rows are stored in LDS under the permutation
//   key_perm (swap of the middle two groups of 4 in every 16 rows): then lane
//   half h holds 8 consecutive keys 16t+8h..16t+8h+7 of each 16-key step, which
//   is exactly the B-operand k layout.  V is transposed while being written to
//   LDS ([head dim][key]), so the A operand V^T is one 16-byte LDS read.
//   Both LDS tiles use an XOR swizzle of the 16-byte chunk index by the row to
//   spread the column reads over the banks.
//
// Online softmax in base 2: x = s * scale * log2(e); running max m and sum l
// per row; O is rescaled by 2^(m_old - m_new).  P is rounded to bf16 for the PV
// product; l accumulates the fp32 values.  lse = (m + log2 l) * ln 2.
// Causal tiles entirely above the diagonal are never visited; the element mask
// is evaluated only on tiles that cross the diagonal or the end of the keys.
#include "kernels.h"

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int BN = 64;  // keys per tile
constexpr float kLn2 = 0.69314718055994530942f;

// Involution on [0, 16): swaps rows 4..7 with 8..11 (and leaves the other two groups).
__device__ __forceinline__ int key_perm(int r) { return r ^ ((((r >> 2) ^ (r >> 3)) & 1) * 12); }

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

template <int HD, int NW, bool OUT_F32>
__global__ __launch_bounds__(NW * 64) void fwd_bf16_kernel(FwdArgs a) {
    constexpr int NT = NW * 64;
    constexpr int BM = NW * 32;
    constexpr int KCH = HD / 8;          // 16-byte chunks per K row
    constexpr int KS = HD / 16;          // k-steps of S^T over the head dim
    constexpr int MB = HD / 32;          // 32-row blocks of O^T over the head dim
    constexpr int KI = BN * KCH / NT;    // K chunks loaded per thread per tile
    constexpr int VI = (BN / 4) * KCH;   // V items (4 keys x 8 dims) per tile
    constexpr int K_BYTES = BN * HD * 2;
    constexpr int V_BYTES = HD * BN * 2;
    constexpr int BUF_BYTES = K_BYTES + V_BYTES;
    static_assert(KI >= 1 && KI * NT == BN * KCH, "K tile split");
    static_assert(VI <= NT, "V tile split");

    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * BUF_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hh = lane >> 5;

    // ---- which (tile, sequence, batch*head) this workgroup owns; heaviest tiles first
    const int BH = a.B * a.Htot;
    const int tiles = (a.max_seqlen_q + BM - 1) / BM;
    int id = blockIdx.x;
    const int bh = id % BH;
    id /= BH;
    const int seq = id % a.nseq;
    const int tile = tiles - 1 - id / a.nseq;
    const int b = bh / a.Htot, hf = bh % a.Htot;

    int qs = 0, qe = a.Mq, ks = 0, ke = a.Mkv;
    if (a.mask >= kMaskBlockDiag) {
        const int32_t *skp = a.seqstart_k ? a.seqstart_k : a.seqstart_q;
        qs = min(max(a.seqstart_q[seq], 0), a.Mq);
        qe = min(max(a.seqstart_q[seq + 1], qs), a.Mq);
        ks = min(max(skp[seq], 0), a.Mkv);
        ke = min(max(skp[seq + 1], ks), a.Mkv);
    }
    const int Lq = qe - qs, Lk = ke - ks;
    const int row0 = tile * BM;
    if (tile < 0 || row0 >= Lq) return;
    const bool causal = (a.mask == kMaskCausal || a.mask == kMaskBlockDiagCausal);
    const int nkeys = causal ? min(Lk, row0 + BM) : Lk;
    const int ntiles = (nkeys + BN - 1) / BN;

    const __bf16 *qp = (const __bf16 *)a.q + (int64_t)b * a.sq.b + head_offset(a.sq, hf, a.Hin) + (int64_t)qs * a.sq.m;
    const __bf16 *kp = (const __bf16 *)a.k + (int64_t)b * a.sk.b + head_offset(a.sk, hf, a.Hin) + (int64_t)ks * a.sk.m;
    const __bf16 *vp = (const __bf16 *)a.v + (int64_t)b * a.sv.b + head_offset(a.sv, hf, a.Hin) + (int64_t)ks * a.sv.m;

    // ---- Q^T fragments (B operand), resident for the whole kernel
    const int wrow0 = row0 + wave * 32;  // first local row of this wave
    const int qrow = wrow0 + l32;        // this lane's query row (local to the sequence)
    bf16x8 qf[KS];
    if (qrow < Lq) {
        const bf16x8 *src = (const bf16x8 *)(qp + (int64_t)qrow * a.sq.m + 8 * hh);
#pragma unroll
        for (int s = 0; s < KS; ++s) qf[s] = src[2 * s];
    } else {
#pragma unroll
        for (int s = 0; s < KS; ++s) qf[s] = bf16x8{};
    }

    // ---- global -> register staging of one K/V tile
    u32x4 kr[KI], vr[4];
    auto gload = [&](int kt0) {
#pragma unroll
        for (int i = 0; i < KI; ++i) {
            const int it = tid + i * NT, r = it / KCH, cc = it % KCH, j = kt0 + r;
            kr[i] = (j < Lk) ? *(const u32x4 *)(kp + (int64_t)j * a.sk.m + cc * 8) : u32x4{0, 0, 0, 0};
        }
        if (tid < VI) {
            const int a4 = tid / KCH, cc = tid % KCH;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int j = kt0 + 4 * a4 + u;
                vr[u] = (j < Lk) ? *(const u32x4 *)(vp + (int64_t)j * a.sv.m + cc * 8) : u32x4{0, 0, 0, 0};
            }
        }
    };
    // ---- register -> LDS: K permuted + swizzled, V transposed + swizzled
    auto lstore = [&](int buf) {
        unsigned char *kb = smem + buf * BUF_BYTES;
        unsigned char *vb = kb + K_BYTES;
#pragma unroll
        for (int i = 0; i < KI; ++i) {
            const int it = tid + i * NT, r = it / KCH, cc = it % KCH;
            const int rho = (r & ~15) | key_perm(r & 15);
            *(u32x4 *)(kb + rho * (HD * 2) + ((cc ^ (rho & (KCH - 1))) << 4)) = kr[i];
        }
        if (tid < VI) {
            const int a4 = tid / KCH, cc = tid % KCH;
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                const int w = d >> 1;
                unsigned lo, hi;
                if (d & 1) {
                    lo = (vr[0][w] >> 16) | (vr[1][w] & 0xffff0000u);
                    hi = (vr[2][w] >> 16) | (vr[3][w] & 0xffff0000u);
                } else {
                    lo = (vr[0][w] & 0xffffu) | (vr[1][w] << 16);
                    hi = (vr[2][w] & 0xffffu) | (vr[3][w] << 16);
                }
                const int row = cc * 8 + d;
                *(u32x2 *)(vb + row * (BN * 2) + ((((a4 >> 1) ^ (row & 7))) << 4) + ((a4 & 1) << 3)) = u32x2{lo, hi};
            }
        }
    };

    f32x16 o[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) o[i] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;
    const float c = a.scale_log2;

    if (ntiles > 0) gload(0);
    for (int t = 0; t < ntiles; ++t) {
        const int kt0 = t * BN;
        lstore(t & 1);
        __syncthreads();
        if (t + 1 < ntiles) gload(kt0 + BN);

        const unsigned char *kb = smem + (t & 1) * BUF_BYTES;
        const unsigned char *vb = kb + K_BYTES;

        // S^T = K Q^T for two 32-key blocks
        f32x16 st[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2) {
                const int rho = kb2 * 32 + l32;
                const int ch = (2 * s + hh) ^ (rho & (KCH - 1));
                const bf16x8 af = *(const bf16x8 *)(kb + rho * (HD * 2) + (ch << 4));
                st[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[s], st[kb2], 0, 0, 0);
            }
        }

        // scale, mask, row max
        const bool need_mask = (kt0 + BN > Lk) || (causal && kt0 + BN - 1 > wrow0);
        float mt = -INFINITY;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float x = st[kb2][r] * c;
                if (need_mask) {
                    const int key = kt0 + kb2 * 32 + key_perm(8 * (r >> 2) + 4 * hh + (r & 3));
                    if (key >= Lk || (causal && key > qrow)) x = -INFINITY;
                }
                st[kb2][r] = x;
                mt = fmaxf(mt, x);
            }
        }
        mt = fmaxf(mt, xor32(mt));
        const float m_new = fmaxf(m_run, mt);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        m_run = m_new;

        float ls = 0.f;
        bf16x8 pb[2][2];
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = __builtin_amdgcn_exp2f(st[kb2][r] - m_use);
                ls += p;
                pb[kb2][r >> 3][r & 7] = (__bf16)p;
            }
        }
        l_run = l_run * alpha + ls;
#pragma unroll
        for (int i = 0; i < MB; ++i) o[i] *= alpha;

        // O^T += V^T P^T
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const int row = mb * 32 + l32;
                    const int ch = (4 * kb2 + 2 * kt + hh) ^ (row & 7);
                    const bf16x8 af = *(const bf16x8 *)(vb + row * (BN * 2) + (ch << 4));
                    o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, pb[kb2][kt], o[mb], 0, 0, 0);
                }
            }
        }
    }

    // ---- normalise and store
    const float l_tot = l_run + xor32(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (qrow < Lq) {
        unsigned char *op = (unsigned char *)a.o;
        const int64_t obase = (int64_t)b * a.so.b + head_offset(a.so, hf, a.Hin) + (int64_t)(qs + qrow) * a.so.m;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = mb * 32 + 8 * g + 4 * hh;
                const float x0 = o[mb][4 * g] * inv, x1 = o[mb][4 * g + 1] * inv;
                const float x2 = o[mb][4 * g + 2] * inv, x3 = o[mb][4 * g + 3] * inv;
                if (OUT_F32) {
                    *(f32x4 *)(op + (obase + d0) * 4) = f32x4{x0, x1, x2, x3};
                } else {
                    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                    *(bf16x4 *)(op + (obase + d0) * 2) = bf16x4{(__bf16)x0, (__bf16)x1, (__bf16)x2, (__bf16)x3};
                }
            }
        }
        if (a.lse && hh == 0) {
            a.lse[((int64_t)b * a.Htot + hf) * a.Mq + qs + qrow] =
                l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
        }
    }
}

template <int HD, int NW, bool OUT_F32>
hipError_t launch(const FwdArgs &a, hipStream_t stream) {
    constexpr int BM = NW * 32;
    const int64_t tiles = (a.max_seqlen_q + BM - 1) / BM;
    const int64_t grid = tiles * a.nseq * (int64_t)a.B * a.Htot;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((fwd_bf16_kernel<HD, NW, OUT_F32>), dim3((unsigned)grid), dim3(NW * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs &a, bool out_f32, hipStream_t stream) {
    if (a.K == 128) return out_f32 ? launch<128, 4, true>(a, stream) : launch<128, 4, false>(a, stream);
    if (a.K == 64) return out_f32 ? launch<64, 4, true>(a, stream) : launch<64, 4, false>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace attn
