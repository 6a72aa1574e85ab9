// Fused attention backward for bf16 inputs on gfx950 matrix cores.
//
// Computes dq, dk, dv of the forward (MSLK kernel reference, "Attention - Core fMHA":
// memory_efficient_attention_backward consumes the upstream gradient, the forward's
// output and LSE and the original q, k, v; masks from "Attention - Biases & masks").
// With P_ij = exp(scale q_i.k_j - lse_i) on the visible keys:
//   dv_j = sum_i P_ij dout_i,  dS_ij = P_ij (dout_i.v_j - D_i),  D_i = dout_i.out_i,
//   dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i.
// The score matrix is never stored: P is rebuilt from the saved LSE tile by tile.
//
// Two launches:
//   1. bwd_dq_kernel: the forward's arrangement (8 waves, 32 query rows each; q and
//      dout in registers, 64-key tiles of K and V through LDS): S^T = K Q^T and
//      dP^T = V dout^T (lane l owns query row l%32), dS^T, then dQ^T += K^T dS^T.
//      Each lane first forms its row's D_i and base-2 LSE L_i = lse_i log2(e) (+inf for
//      a row with no visible key, so every rebuilt P of that row is exactly 0) and
//      stores both in a caller workspace for the second launch.
//   2. bwd_dkdv_pair_kernel: a workgroup owns 128 keys of one (batch, head, sequence), 32
//      per pair of waves; the pair keeps those keys' K and V rows in registers as
//      matrix-core operands while 64-row tiles of Q and dout (and their L, D) stream
//      through a 2-stage LDS ring.  Per tile and 32-row block: S = Q K^T and
//      dP = dout V^T (lane l owns key l%32 and 16 query rows), P and dS in fp32, then
//      dV^T += dout^T P and dK^T += Q^T dS with the A operands read transposed from the
//      row-major LDS tiles.
// P is rounded to bf16 for dV and dS for dK and dQ; every product accumulates in fp32.
// Same matrix-core layout as the forward (v_mfma_f32_32x32x16_bf16): a B operand taken
// from C-layout registers gives lane half h the rows {8a + 4h + 0..3} of each 16-row
// step, which fixes the k order, and the transposed A operand is read with
// ds_read_b64_tr_b16 from the same swizzled row-major tiles.
#include <type_traits>

#include "kernels.h"
#include "tile_common.h"

namespace attn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int BQ = 64;  // query rows per streamed tile (dK/dV kernel)
constexpr int BN = 64;  // keys per streamed tile (dQ kernel)

__device__ __forceinline__ int clampk(int64_t x, int64_t lo, int64_t hi) {
    return (int)(x < lo ? lo : (x > hi ? hi : x));
}

// Sequence bounds of workgroup sequence `seq`: query rows [qs, qe), key rows [ks, ke).
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

// ------------------------------------------------------------------ dK and dV

// Transposed-read LDS offsets inside a row-major [rows, HD] tile: lane i of 16-lane group G
// addresses row 4*hh + i/4 (+ 8e, + multiples of 16) and columns mb*32 + 16*(G&1) + 4*(i%4).
template <int HD, int MB>
__device__ __forceinline__ void tr_offsets(int lane, int (&taddr)[MB][2]) {
    constexpr int ROWB = HD * 2;
    const int hh = lane >> 5;
    const int trow = 4 * hh + ((lane & 15) >> 2);
    const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int row = trow + 8 * e, col = mb * 32 + tcol;
            taddr[mb][e] = row * ROWB + (((col >> 3) ^ swz<HD>(row)) << 4) + ((col & 4) << 1);
        }
}

// A operand (32 columns x 16 rows, transposed) at byte offset `off` of an LDS tile.
__device__ __forceinline__ bf16x8 tr_frag(const unsigned char LDS_AS *base, int off0, int off1) {
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 LDS_AS *)(base + off0));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 LDS_AS *)(base + off1));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// dK/dV kernel: 8 waves, 128 keys.  Waves w and w + 4 (which share a SIMD) own the same 32
// keys; wave w computes S = Q K^T, P and dV^T += dout^T P and passes P through LDS, wave
// w + 4 computes dP = dout V^T, dS = P (dP - D) and dK^T += Q^T dS.  Each wave holds one
// accumulator set and one resident operand (K or V), so two waves fit per SIMD and one's
// matrix-core ops overlap the other's LDS reads and fp32 work (a single wave doing all
// four products needs ~320 registers per lane and runs alone on its SIMD).
// With DS the dS side also writes its bf16 dS blocks to the key-major dS^T buffer for the
// dQ launch that follows (one sequence only: rows and keys count from 0).
template <int HD, int STAGES, bool DS = false>
__global__ __launch_bounds__(512) void bwd_dkdv_pair_kernel(BwdArgs a) {
    constexpr int NW = 8, NT = NW * 64, BK = 128;  // keys per workgroup (32 per wave pair)
    constexpr int ROWB = HD * 2;
    constexpr int CPR = HD / 8;
    constexpr int TILE_BYTES = BQ * ROWB;
    constexpr int LSD_BASE = STAGES * 2 * TILE_BYTES;       // per stage: 64 L values, 64 D values
    constexpr int PX_BASE = LSD_BASE + STAGES * 2 * BQ * 4;  // P exchange: [pair][2 buffers][4 KB]
    constexpr int PX_BYTES = 32 * 32 * 4;                    // one 32x32 fp32 block
    constexpr int ROUNDS = TILE_BYTES / 16 / NT;
    constexpr int KS = HD / 16, MB = HD / 32;
    static_assert(ROUNDS >= 1 && ROUNDS * NT * 16 == TILE_BYTES, "tile split");

    __shared__ __attribute__((aligned(1024))) unsigned char smem[PX_BASE + 4 * 2 * PX_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pair = wave & 3;
    const bool pside = wave < 4;  // S, P, dV side; the other wave of the pair does dP, dS, dK

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
    const int k0 = ktile * BK;
    if (k0 >= Lk) return;
    const int k1 = min(k0 + BK, Lk);
    const int64_t shift = a.bottom_right ? (int64_t)Lk - Lq : 0;
    const int qbeg = clampk((int64_t)k0 - shift - a.wr, 0, Lq);
    const int qend = clampk((int64_t)k1 - 1 - shift + a.wl + 1, 0, Lq);
    const int tb = qbeg / BQ;
    const int te = qend > qbeg ? (qend + BQ - 1) / BQ : tb;
    int ua = (clampk((int64_t)k1 - 1 - shift - a.wr, 0, Lq) + BQ - 1) / BQ;
    int ub = clampk(min((int64_t)k0 - shift + a.wl, (int64_t)Lq - 1) + 1, 0, Lq) / BQ;
    ua = min(max(ua, tb), te);
    ub = min(max(ub, ua), te);

    const __bf16 *qp = (const __bf16 *)a.q + (int64_t)b * a.sq.b + head_offset(a.sq, hf, a.Hin) + (int64_t)qs * a.sq.m;
    const __bf16 *gp =
        (const __bf16 *)a.dout + (int64_t)b * a.sdo.b + head_offset(a.sdo, hf, a.Hin) + (int64_t)qs * a.sdo.m;
    const __bf16 *kp = (const __bf16 *)a.k + (int64_t)b * a.sk.b + head_offset(a.sk, hf, a.Hin) + (int64_t)ks * a.sk.m;
    const __bf16 *vp = (const __bf16 *)a.v + (int64_t)b * a.sv.b + head_offset(a.sv, hf, a.Hin) + (int64_t)ks * a.sv.m;
    const int64_t wrow = ((int64_t)b * a.Htot + hf) * a.Mq + qs;
    const unsigned qstride = (unsigned)a.sq.m * 2u, gstride = (unsigned)a.sdo.m * 2u;

    unsigned qoff[ROUNDS], goff[ROUNDS];
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
        const int p = (r * NW + wave) * 64 + lane;
        const int row = p / CPR, c = (p % CPR) ^ swz<HD>(row);
        qoff[r] = row * qstride + c * 16;
        goff[r] = row * gstride + c * 16;
    }
    const unsigned smem_base = (unsigned)(unsigned long long)(unsigned char LDS_AS *)smem;
    auto issue = [&](int t) __attribute__((always_inline)) {
        const int q0 = t * BQ;
        const int nvalid = min(BQ, Lq - q0);
        const int stage = (t - tb) % STAGES;
        const unsigned st = smem_base + stage * 2 * TILE_BYTES;
        const i32x4 qr = make_rsrc(qp + (int64_t)q0 * a.sq.m, (nvalid - 1) * qstride + ROWB);
        const i32x4 gr = make_rsrc(gp + (int64_t)q0 * a.sdo.m, (nvalid - 1) * gstride + ROWB);
#pragma unroll
        for (int r = 0; r < ROUNDS; ++r) dma16(qr, qoff[r], st + (r * NW + wave) * 1024);
#pragma unroll
        for (int r = 0; r < ROUNDS; ++r) dma16(gr, goff[r], st + TILE_BYTES + (r * NW + wave) * 1024);
        if (wave == 0) {  // rows past the sequence read as 0 and are always masked
            const unsigned ls = smem_base + LSD_BASE + stage * 2 * BQ * 4;
            dma4(make_rsrc(a.ws_l2 + wrow + q0, nvalid * 4), lane * 4, ls);
            dma4(make_rsrc(a.ws_d + wrow + q0, nvalid * 4), lane * 4, ls + BQ * 4);
        }
    };

    // ---- this pair's 32 keys; the P side keeps K, the other side V, as B operands
    const int kw0 = k0 + pair * 32;
    const int key = kw0 + l32;
    bf16x8 rf[KS];
    if (key < Lk) {
        const u32x4 *src = (const u32x4 *)((pside ? kp + (int64_t)key * a.sk.m : vp + (int64_t)key * a.sv.m) + 8 * hh);
#pragma unroll
        for (int s = 0; s < KS; ++s) rf[s] = __builtin_bit_cast(bf16x8, src[2 * s]);
    } else {
#pragma unroll
        for (int s = 0; s < KS; ++s) rf[s] = bf16x8{};
    }
    const int qlo = clampk((int64_t)key - shift - a.wr, 0, Lq);
    const int qhi = clampk((int64_t)key - shift + a.wl, -1, Lq - 1);
    // both are non-decreasing in the key: the pair's last key has the largest lower bound, its
    // first key the smallest upper bound
    const int qlo_w = clampk((int64_t)kw0 + 31 - shift - a.wr, 0, Lq);
    const int qhi_w = clampk((int64_t)kw0 - shift + a.wl, -1, Lq - 1);
    const float c = a.scale_log2;

    int raddr[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) raddr[s] = l32 * ROWB + (((2 * s + hh) ^ swz<HD>(l32)) << 4);
    int taddr[MB][2];
    tr_offsets<HD, MB>(lane, taddr);
    // P exchange slot of this lane: float4 r4 of 16 values at [pair][buf][r4][lane]
    float LDS_AS *px = (float LDS_AS *)(smem + PX_BASE) + pair * 2 * (PX_BYTES / 4) + lane * 4;

    f32x16 acc[MB];  // dV^T on the P side, dK^T on the other
#pragma unroll
    for (int i = 0; i < MB; ++i) acc[i] = f32x16{};

    // dS of the last computed tile (DS, dS side), written after the next ring barrier: stores
    // count in vmcnt, and issued at once they would hold up that barrier.  The buffer holds
    // 32-key x 32-query blocks in the order the registers hold them ([2][64 lanes][8]: element
    // i of lane l in half kt is key l % 32 and query 16 kt + 8 (i / 4) + 4 (l / 32) + i % 4), so
    // every store instruction writes 1 KB of consecutive bytes.
    bf16x8 pend[2][2];
    int pend_q0 = -1;
    __bf16 *const dsw = DS ? (__bf16 *)a.ds + ((int64_t)b * a.Htot + hf) * a.ds_rows * a.ds_pitch +
                                 (int64_t)(kw0 >> 5) * (a.ds_pitch >> 5) * 1024 + lane * 8
                           : nullptr;
    auto flush_ds = [&]() __attribute__((always_inline)) {
        if (DS && pend_q0 >= 0) {
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)  // read once, by the dQ launch: streaming stores
                    __builtin_nontemporal_store(pend[qb][kt], (bf16x8 *)(dsw + ((pend_q0 >> 5) + qb) * 1024 + kt * 512));
            pend_q0 = -1;
        }
    };

    auto step = [&](int t, auto masked_tag) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(masked_tag)::value;
        const int q0 = t * BQ;
        const int stage = (t - tb) % STAGES;
        // tile t has landed (with STAGES - 1 tiles in flight, tile t + 1's loads may be pending)
        if (STAGES == 3 && t + 1 < te) wait_barrier<2 * ROUNDS>();
        else wait_barrier<0>();
        if (t + STAGES - 1 < te) issue(t + STAGES - 1);
        if (DS) flush_ds();
        // this pair's keys see no row of the tile: compute nothing, still meet every barrier
        const bool active = kw0 < Lk && !(MASKED && ((int64_t)kw0 > (int64_t)q0 + BQ - 1 + shift + a.wr ||
                                                      (int64_t)kw0 + 31 < (int64_t)q0 + shift - a.wl));
        const unsigned char LDS_AS *st = (const unsigned char LDS_AS *)smem + stage * 2 * TILE_BYTES;
        const float LDS_AS *ls = (const float LDS_AS *)(smem + LSD_BASE + stage * 2 * BQ * 4);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            float LDS_AS *pxb = px + ((2 * (t - tb) + qb) & 1) * (PX_BYTES / 4);
            f32x16 x = f32x16{};  // S on the P side, dP on the other
            bf16x8 ob[2];         // P (P side) or dS (other side) as bf16 B operands
            if (active) {
                const int aoff = pside ? 0 : TILE_BYTES;  // Q rows or dout rows
#pragma unroll
                for (int k = 0; k < KS; ++k) {
                    const bf16x8 fa = *(const bf16x8 LDS_AS *)(st + aoff + raddr[k] + qb * 32 * ROWB);
                    x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, rf[k], x, 0, 0, 0);
                }
                if (pside) {
                    float p[16];
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int row = qb * 32 + 8 * g + 4 * hh;
                        const f32x4 l2 = *(const f32x4 LDS_AS *)(ls + row);
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            p[4 * g + j] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[4 * g + j], c, -l2[j]));
                    }
                    if (MASKED) {
                        // element 4g + j is query q0 + 32 qb + 4 hh + 8g + j; only the bounds that
                        // cut this block for one of the pair's keys are tested
                        const int qb0 = q0 + qb * 32;
                        const int dlo = qlo - qb0 - 4 * hh, dhi = qhi - qb0 - 4 * hh;
                        const bool cut_lo = qb0 < qlo_w, cut_hi = qb0 + 31 > qhi_w;
                        if (cut_lo && cut_hi) {
#pragma unroll
                            for (int e = 0; e < 16; ++e) {
                                const int off = 8 * (e >> 2) + (e & 3);
                                if (off < dlo || off > dhi) p[e] = 0.f;
                            }
                        } else if (cut_hi) {
#pragma unroll
                            for (int e = 0; e < 16; ++e)
                                if (8 * (e >> 2) + (e & 3) > dhi) p[e] = 0.f;
                        } else if (cut_lo) {
#pragma unroll
                            for (int e = 0; e < 16; ++e)
                                if (8 * (e >> 2) + (e & 3) < dlo) p[e] = 0.f;
                        }
                    }
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        *(f32x4 LDS_AS *)(pxb + g * 256) = f32x4{p[4 * g], p[4 * g + 1], p[4 * g + 2], p[4 * g + 3]};
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                        for (int i = 0; i < 8; ++i) ob[kt][i] = (__bf16)p[8 * kt + i];
                }
            }
            // P of this block is in LDS; the other side's dP is in its registers
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            if (active) {
                if (!pside) {
                    float ds[16];
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int row = qb * 32 + 8 * g + 4 * hh;
                        const f32x4 dd = *(const f32x4 LDS_AS *)(ls + BQ + row);
                        const f32x4 pv = *(const f32x4 LDS_AS *)(pxb + g * 256);
#pragma unroll
                        for (int j = 0; j < 4; ++j) ds[4 * g + j] = pv[j] * (x[4 * g + j] - dd[j]);
                    }
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                        for (int i = 0; i < 8; ++i) ob[kt][i] = (__bf16)ds[8 * kt + i];
                    if (DS) {
                        pend[qb][0] = ob[0];
                        pend[qb][1] = ob[1];
                        pend_q0 = q0;
                    }
                }
                // dV^T += dout^T P (P side) or dK^T += Q^T dS (other side)
                const int toff = pside ? TILE_BYTES : 0;
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    const int roff = (qb * 32 + kt * 16) * ROWB;
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
                        const bf16x8 ft = tr_frag(st + toff, taddr[mb][0] + roff, taddr[mb][1] + roff);
                        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ft, ob[kt], acc[mb], 0, 0, 0);
                    }
                }
            }
        }
    };

    if (tb < te) issue(tb);
    if (STAGES == 3 && tb + 1 < te) issue(tb + 1);
    int t = tb;
    for (; t < ua; ++t) step(t, std::true_type{});
    for (; t < ub; ++t) step(t, std::false_type{});
    for (; t < te; ++t) step(t, std::true_type{});
    if (DS) flush_ds();

    {
        // gradient rows go out whole, staged in the now idle ring
        const Strides &so = pside ? a.sdv : a.sdk;
        __syncthreads();  // every wave has finished reading the Q/dout ring
        store_rows_bf16<HD>(acc, pside ? 1.f : a.scale, (unsigned char LDS_AS *)smem + wave * 32 * ROWB,
                            (unsigned char *)(pside ? a.dv : a.dk),
                            (int64_t)b * so.b + head_offset(so, hf, a.Hin) + (int64_t)(ks + kw0) * so.m, so.m, Lk - kw0);
    }
}

// ------------------------------------------------------------------ dQ (runs first)

template <int HD, int NW, int STAGES>
__global__ __launch_bounds__(NW * 64) void bwd_dq_kernel(BwdArgs a) {
    constexpr int NT = NW * 64;
    constexpr int BM = NW * 32;               // query rows per workgroup
    constexpr int ROWB = HD * 2;
    constexpr int CPR = HD / 8;
    constexpr int TILE_BYTES = BN * ROWB;     // one K or V tile
    constexpr int ROUNDS = TILE_BYTES / 16 / NT;
    constexpr int KS = HD / 16, MB = HD / 32;
    static_assert(ROUNDS >= 1 && ROUNDS * NT * 16 == TILE_BYTES, "tile split");

    __shared__ __attribute__((aligned(1024))) unsigned char smem[STAGES * 2 * TILE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // ---- which (query tile, sequence, batch*head); heaviest tiles first
    const int BH = a.B * a.Htot;
    const int tiles = (a.max_seqlen_q + BM - 1) / BM;
    int id = blockIdx.x;
    const int bh = id % BH;
    id /= BH;
    const int seq = id % a.nseq;
    const int tidx = id / a.nseq;  // 0: the sequence's heaviest row block
    const int b = bh / a.Htot, hf = bh % a.Htot;
    int qs, qe, ks, ke;
    seq_bounds(a, seq, qs, qe, ks, ke);
    const int Lq = qe - qs, Lk = ke - ks;
    // row blocks as in the forward: aligned to the sequence's last row when the remainder
    // Lq mod BM is at most BM - BN rows (the ragged block is then the first, which sees the fewest
    // keys under a causal mask), else to row 0; rows before row 0 hold nothing
    const int rem = Lq % BM;
    const bool end_aligned = rem != 0 && rem <= BM - BN;
    const int row0 = end_aligned ? Lq - (tidx + 1) * BM : (tiles - 1 - tidx) * BM;
    if (end_aligned ? row0 + BM <= 0 : row0 >= Lq) return;
    const int row0v = max(row0, 0);
    const int64_t shift = a.bottom_right ? (int64_t)Lk - Lq : 0;
    const int row_last = min(row0 + BM, Lq) - 1;
    const int kbeg = clampk((int64_t)row0v + shift - a.wl, 0, Lk);
    const int kend = clampk((int64_t)row_last + shift + a.wr + 1, 0, Lk);
    const int tb = kbeg / BN;
    const int te = kend > kbeg ? (kend + BN - 1) / BN : tb;
    int ua = (clampk((int64_t)row_last + shift - a.wl, 0, Lk) + BN - 1) / BN;
    int ub = clampk((int64_t)row0v + shift + a.wr + 1, 0, Lk) / BN;
    ua = min(max(ua, tb), te);
    ub = min(max(ub, ua), te);

    const __bf16 *qp = (const __bf16 *)a.q + (int64_t)b * a.sq.b + head_offset(a.sq, hf, a.Hin) + (int64_t)qs * a.sq.m;
    const __bf16 *gp =
        (const __bf16 *)a.dout + (int64_t)b * a.sdo.b + head_offset(a.sdo, hf, a.Hin) + (int64_t)qs * a.sdo.m;
    const __bf16 *kp = (const __bf16 *)a.k + (int64_t)b * a.sk.b + head_offset(a.sk, hf, a.Hin) + (int64_t)ks * a.sk.m;
    const __bf16 *vp = (const __bf16 *)a.v + (int64_t)b * a.sv.b + head_offset(a.sv, hf, a.Hin) + (int64_t)ks * a.sv.m;
    const unsigned kstride = (unsigned)a.sk.m * 2u, vstride = (unsigned)a.sv.m * 2u;

    unsigned koff[ROUNDS], voff[ROUNDS];
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
        const int p = (r * NW + wave) * 64 + lane;
        const int row = p / CPR, c = (p % CPR) ^ swz<HD>(row);
        koff[r] = row * kstride + c * 16;
        voff[r] = row * vstride + c * 16;
    }
    const unsigned smem_base = (unsigned)(unsigned long long)(unsigned char LDS_AS *)smem;
    auto issue = [&](int t) __attribute__((always_inline)) {
        const int kt0 = t * BN;
        const int nvalid = min(BN, Lk - kt0);
        const unsigned st = smem_base + ((t - tb) % STAGES) * 2 * TILE_BYTES;
        const i32x4 kr = make_rsrc(kp + (int64_t)kt0 * a.sk.m, (nvalid - 1) * kstride + ROWB);
        const i32x4 vr = make_rsrc(vp + (int64_t)kt0 * a.sv.m, (nvalid - 1) * vstride + ROWB);
#pragma unroll
        for (int r = 0; r < ROUNDS; ++r) dma16(kr, koff[r], st + (r * NW + wave) * 1024);
#pragma unroll
        for (int r = 0; r < ROUNDS; ++r) dma16(vr, voff[r], st + TILE_BYTES + (r * NW + wave) * 1024);
    };

    // ---- this lane's query row: q and dout as B operands, its L and D
    const int wrow0 = row0 + wave * 32;
    const int qrow = wrow0 + l32;
    const int klo = clampk((int64_t)qrow + shift - a.wl, 0, Lk);
    const int khi = clampk((int64_t)qrow + shift + a.wr, -1, Lk - 1);
    // non-decreasing in the row: the wave's last row has the largest lower bound, its first
    // row the smallest upper bound
    const int klo_w = clampk((int64_t)wrow0 + 31 + shift - a.wl, 0, Lk);
    const int khi_w = clampk((int64_t)wrow0 + shift + a.wr, -1, Lk - 1);
    bf16x8 qf[KS], gf[KS];
    float l2 = INFINITY, dd = 0.f;
    if (qrow >= 0 && qrow < Lq) {
        const u32x4 *qsrc = (const u32x4 *)(qp + (int64_t)qrow * a.sq.m + 8 * hh);
        const u32x4 *gsrc = (const u32x4 *)(gp + (int64_t)qrow * a.sdo.m + 8 * hh);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            qf[s] = __builtin_bit_cast(bf16x8, qsrc[2 * s]);
            gf[s] = __builtin_bit_cast(bf16x8, gsrc[2 * s]);
        }
        // D = dout.out over the row: this lane holds half of its columns, the lane 32 away the rest
        const u32x4 *osrc = (const u32x4 *)((const __bf16 *)a.o + (int64_t)b * a.so.b + head_offset(a.so, hf, a.Hin) +
                                            (int64_t)(qs + qrow) * a.so.m + 8 * hh);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const u32x4 ow = osrc[2 * s], gw = __builtin_bit_cast(u32x4, gf[s]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                dd = fmaf(__uint_as_float(ow[e] << 16), __uint_as_float(gw[e] << 16), dd);
                dd = fmaf(__uint_as_float(ow[e] & 0xffff0000u), __uint_as_float(gw[e] & 0xffff0000u), dd);
            }
        }
        const int64_t w = ((int64_t)b * a.Htot + hf) * a.Mq + qs + qrow;
        const float lse = a.lse[w];
        l2 = lse == -INFINITY ? INFINITY : lse * kLog2e;
    } else {
#pragma unroll
        for (int s = 0; s < KS; ++s) qf[s] = gf[s] = bf16x8{};
    }
    {
        auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(dd), __float_as_uint(dd), false, false);
        dd = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    }
    if (qrow >= 0 && qrow < Lq && hh == 0) {
        const int64_t w = ((int64_t)b * a.Htot + hf) * a.Mq + qs + qrow;
        a.ws_d[w] = dd;
        a.ws_l2[w] = l2;
    }
    const float c = a.scale_log2;

    int raddr[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) raddr[s] = l32 * ROWB + (((2 * s + hh) ^ swz<HD>(l32)) << 4);
    int taddr[MB][2];
    tr_offsets<HD, MB>(lane, taddr);

    f32x16 dq[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) dq[i] = f32x16{};

    auto step = [&](int t, auto masked_tag) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(masked_tag)::value;
        const int kt0 = t * BN;
        if (STAGES == 3 && t + 1 < te) wait_barrier<2 * ROUNDS>();
        else wait_barrier<0>();
        if (t + STAGES - 1 < te) issue(t + STAGES - 1);
        if (MASKED && ((int64_t)kt0 + BN - 1 < (int64_t)wrow0 + shift - a.wl ||
                       (int64_t)kt0 > (int64_t)wrow0 + 31 + shift + a.wr))
            return;
        const unsigned char LDS_AS *st = (const unsigned char LDS_AS *)smem + ((t - tb) % STAGES) * 2 * TILE_BYTES;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            // S^T = K Q^T and dP^T = V dout^T for 32 keys: lane owns query l32, keys 8g + 4hh + j
            f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                const bf16x8 ka = *(const bf16x8 LDS_AS *)(st + raddr[k] + kb * 32 * ROWB);
                const bf16x8 va = *(const bf16x8 LDS_AS *)(st + TILE_BYTES + raddr[k] + kb * 32 * ROWB);
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[k], s, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, gf[k], dp, 0, 0, 0);
            }
            float pr[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) pr[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -l2));
            if (MASKED) {
                // element r is key kt0 + 32 kb + 4 hh + off(r); only the bounds that cut this block
                // for one of the wave's rows are tested
                const int kb0 = kt0 + kb * 32;
                const int dlo = klo - kb0 - 4 * hh, dhi = khi - kb0 - 4 * hh;
                const bool cut_lo = kb0 < klo_w, cut_hi = kb0 + 31 > khi_w;
                if (cut_lo && cut_hi) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int off = 8 * (r >> 2) + (r & 3);
                        if (off < dlo || off > dhi) pr[r] = 0.f;
                    }
                } else if (cut_hi) {
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (8 * (r >> 2) + (r & 3) > dhi) pr[r] = 0.f;
                } else if (cut_lo) {
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (8 * (r >> 2) + (r & 3) < dlo) pr[r] = 0.f;
                }
            }
            float ds[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) ds[r] = pr[r] * (dp[r] - dd);
            bf16x8 dsb[2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 8; ++i) dsb[kt][i] = (__bf16)ds[8 * kt + i];
            // dQ^T += K^T dS^T over the two 16-key steps of this block
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                const int roff = (kb * 32 + kt * 16) * ROWB;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const bf16x8 kt_ = tr_frag(st, taddr[mb][0] + roff, taddr[mb][1] + roff);
                    dq[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt_, dsb[kt], dq[mb], 0, 0, 0);
                }
            }
        }
    };

    if (tb < te) issue(tb);
    if (STAGES == 3 && tb + 1 < te) issue(tb + 1);
    int t = tb;
    for (; t < ua; ++t) step(t, std::true_type{});
    for (; t < ub; ++t) step(t, std::false_type{});
    for (; t < te; ++t) step(t, std::true_type{});

    // dq rows go out whole, staged in the now idle ring
    __syncthreads();  // every wave has finished reading the K/V ring
    store_rows_bf16<HD>(dq, a.scale, (unsigned char LDS_AS *)smem + wave * 32 * ROWB, (unsigned char *)a.dq,
                        (int64_t)b * a.sdq.b + head_offset(a.sdq, hf, a.Hin) + (int64_t)(qs + wrow0) * a.sdq.m,
                        a.sdq.m, Lq - wrow0, -wrow0);
}

// ------------------------------------------------------------------ kept-dS form (one sequence)
//
// 1. bwd_prep_kernel: D_i and the base-2 LSE L_i of every query row, as the dQ kernel forms them.
// 2. bwd_dkdv_pair_kernel<DS>: dK, dV, and dS^T in bf16 (the values dK uses).
// 3. bwd_dq_ds_kernel: dQ^T += K^T dS^T, both operands read transposed from LDS tiles; S and dP
//    are computed once instead of twice.

// D and L of every query row: HD / 8 lanes per row, 16 bytes each, a lane-tree sum per row.
// Rows are numbered like the row arrays ((b * Htot + h) * Mq + m); a wave takes PREP_ITER groups
// of 64 / (HD / 8) consecutive rows, every load issued before the first sum, and writes its
// rows' D and L from consecutive lanes.
constexpr int PREP_ITER = 8;

template <int HD>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs a) {
    constexpr int LPR = HD / 8, RPW = 64 / LPR;  // lanes per row, rows per wave and group
    static_assert(RPW * PREP_ITER <= 64, "one lane per row of the wave at the end");
    const int lane = threadIdx.x & 63;
    const int64_t rows = (int64_t)a.B * a.Htot * a.Mq;
    const int64_t w0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * (RPW * PREP_ITER);
    const int c = (lane % LPR) * 8;
    u32x4 gw[PREP_ITER], ow[PREP_ITER];
#pragma unroll
    for (int it = 0; it < PREP_ITER; ++it) {
        const int64_t w = w0 + it * RPW + lane / LPR;
        gw[it] = ow[it] = u32x4{};
        if (w < rows) {
            const int m = (int)(w % a.Mq);
            const int64_t bh = w / a.Mq;
            const int hf = (int)(bh % a.Htot), b = (int)(bh / a.Htot);
            gw[it] = *(const u32x4 *)((const __bf16 *)a.dout + (int64_t)b * a.sdo.b + head_offset(a.sdo, hf, a.Hin) +
                                      (int64_t)m * a.sdo.m + c);
            ow[it] = *(const u32x4 *)((const __bf16 *)a.o + (int64_t)b * a.so.b + head_offset(a.so, hf, a.Hin) +
                                      (int64_t)m * a.so.m + c);
        }
    }
    float mine = 0.f;  // D of row w0 + lane
#pragma unroll
    for (int it = 0; it < PREP_ITER; ++it) {
        float dd = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            dd = fmaf(__uint_as_float(ow[it][e] << 16), __uint_as_float(gw[it][e] << 16), dd);
            dd = fmaf(__uint_as_float(ow[it][e] & 0xffff0000u), __uint_as_float(gw[it][e] & 0xffff0000u), dd);
        }
#pragma unroll
        for (int x = LPR / 2; x >= 1; x >>= 1) dd += __shfl_xor(dd, x, LPR);
        const float v = __shfl(dd, (lane % RPW) * LPR);
        if (lane / RPW == it) mine = v;
    }
    const int64_t w = w0 + lane;
    if (lane < RPW * PREP_ITER && w < rows) {
        const float lse = a.lse[w];
        a.ws_d[w] = mine;
        a.ws_l2[w] = lse == -INFINITY ? INFINITY : lse * kLog2e;
    }
}

// dQ from the kept dS: 8 waves, 32 query rows each (256 per workgroup), 64-key tiles of K and
// of dS (2 x 8 blocks of 32 keys x 32 queries, two runs of 16 KB in the buffer) through a
// 3-stage LDS ring.  The key tiles and the masked/unmasked split are those of bwd_dq_kernel; on
// masked tiles the dS elements of invisible (query, key) pairs are zeroed (the dK/dV launch
// writes only blocks that hold a visible pair, so anything else in the buffer is never used).
// In LDS the 16-byte chunk n of a block (half n / 64, lane n % 64) sits at n ^ (4 (2 (n / 64) +
// (n / 32) % 2)): the transposed reads of one half-wave then touch 16 chunks in distinct banks.
template <int HD, int STAGES>
__global__ __launch_bounds__(512) void bwd_dq_ds_kernel(BwdArgs a) {
    constexpr int NW = 8, NT = NW * 64;
    constexpr int BM = NW * 32;               // query rows per workgroup
    constexpr int ROWB = HD * 2, CPR = HD / 8;
    constexpr int KT_BYTES = BN * ROWB;       // one K tile
    constexpr int DT_BYTES = BN * BM * 2;     // one dS tile: 2 x 8 blocks of 2 KB
    constexpr int STAGE_BYTES = KT_BYTES + DT_BYTES;
    constexpr int KR = KT_BYTES / 16 / NT, DR = DT_BYTES / 16 / NT;
    constexpr int MB = HD / 32;
    static_assert(KR >= 1 && KR * NT * 16 == KT_BYTES && DR * NT * 16 == DT_BYTES, "tile split");
    static_assert(BM == 256 && DT_BYTES == 2 * 8 * 2048, "a dS tile is two runs of 8 blocks");

    __shared__ __attribute__((aligned(1024))) unsigned char smem[STAGES * STAGE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // ---- which (query tile, batch*head); heaviest tiles first
    const int BH = a.B * a.Htot;
    const int tiles = (a.Mq + BM - 1) / BM;
    const int bh = blockIdx.x % BH;
    const int tile = tiles - 1 - (int)(blockIdx.x / BH);
    const int b = bh / a.Htot, hf = bh % a.Htot;
    const int Lq = a.Mq, Lk = a.Mkv;
    const int row0 = tile * BM;
    if (tile < 0 || row0 >= Lq) return;
    const int64_t shift = a.bottom_right ? (int64_t)Lk - Lq : 0;
    const int row_last = min(row0 + BM, Lq) - 1;
    const int kbeg = clampk((int64_t)row0 + shift - a.wl, 0, Lk);
    const int kend = clampk((int64_t)row_last + shift + a.wr + 1, 0, Lk);
    const int tb = kbeg / BN;
    const int te = kend > kbeg ? (kend + BN - 1) / BN : tb;
    int ua = (clampk((int64_t)row_last + shift - a.wl, 0, Lk) + BN - 1) / BN;
    int ub = clampk((int64_t)row0 + shift + a.wr + 1, 0, Lk) / BN;
    ua = min(max(ua, tb), te);
    ub = min(max(ub, ua), te);

    const __bf16 *kp = (const __bf16 *)a.k + (int64_t)b * a.sk.b + head_offset(a.sk, hf, a.Hin);
    // block (key block kb, query block qb) starts at 2048 (kb * nqb + qb) bytes of the head's slab
    const unsigned nqb = (unsigned)(a.ds_pitch >> 5), run = nqb * 2048u;
    const unsigned char *dsp = (const unsigned char *)a.ds + (int64_t)bh * a.ds_rows * a.ds_pitch * 2 + (row0 >> 5) * 2048;
    const unsigned kstride = (unsigned)a.sk.m * 2u;

    unsigned koff[KR], doff[DR];
#pragma unroll
    for (int r = 0; r < KR; ++r) {
        const int p = (r * NW + wave) * 64 + lane;
        const int row = p / CPR, c = (p % CPR) ^ swz<HD>(row);
        koff[r] = row * kstride + c * 16;
    }
#pragma unroll
    for (int r = 0; r < DR; ++r) {
        // LDS chunk p of the tile: key half p / 1024, query block (p / 128) % 8, swizzled chunk p % 128
        const int p = (r * NW + wave) * 64 + lane;
        const int n = p & 127, src = n ^ ((2 * (n >> 6) + ((n >> 5) & 1)) << 2);
        doff[r] = (unsigned)(p >> 10) * run + (unsigned)(((p >> 7) & 7) * 128 + src) * 16u;
    }
    const unsigned smem_base = (unsigned)(unsigned long long)(unsigned char LDS_AS *)smem;
    auto issue = [&](int t) __attribute__((always_inline)) {
        const int kt0 = t * BN;
        const int nvalid = min(BN, Lk - kt0);
        const unsigned st = smem_base + ((t - tb) % STAGES) * STAGE_BYTES;
        const i32x4 kr = make_rsrc(kp + (int64_t)kt0 * a.sk.m, (nvalid - 1) * kstride + ROWB);
        // key blocks kt0 / 32 and kt0 / 32 + 1 < ds_rows / 32, query blocks row0 / 32 + 0..7 < nqb
        const i32x4 dr = make_rsrc(dsp + (int64_t)(kt0 >> 5) * run, run + 8 * 2048);
#pragma unroll
        for (int r = 0; r < KR; ++r) dma16(kr, koff[r], st + (r * NW + wave) * 1024);
#pragma unroll
        for (int r = 0; r < DR; ++r) dma16_nt(dr, doff[r], st + KT_BYTES + (r * NW + wave) * 1024);
    };

    const int wrow0 = row0 + wave * 32;
    const int qrow = wrow0 + l32;
    const int klo = clampk((int64_t)qrow + shift - a.wl, 0, Lk);
    const int khi = clampk((int64_t)qrow + shift + a.wr, -1, Lk - 1);
    const int klo_w = clampk((int64_t)wrow0 + 31 + shift - a.wl, 0, Lk);
    const int khi_w = clampk((int64_t)wrow0 + shift + a.wr, -1, Lk - 1);

    int taddr[MB][2];
    tr_offsets<HD, MB>(lane, taddr);
    // The transposed read of this wave's query block: lane l of 16-lane group G takes the 4
    // queries 16 (G % 2) + 4 (l % 4) .. + 3 of key 16 kt + 4 hh + (l % 16) / 4 + 8 e; in the block
    // those are bytes 8 ((l / 2) % 2) of the chunk of half G % 2, lane key + 32 (l % 2).
    int daddr[2][2];
    {
        const int g1 = (lane >> 4) & 1, hb = lane & 1;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int key = 16 * kt + 4 * hh + ((lane & 15) >> 2) + 8 * e;
                const int n = g1 * 64 + hb * 32 + key;
                daddr[kt][e] = wave * 2048 + ((n ^ ((2 * g1 + hb) << 2)) << 4) + ((lane >> 1) & 1) * 8;
            }
    }

    f32x16 dq[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) dq[i] = f32x16{};

    auto step = [&](int t, auto masked_tag) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(masked_tag)::value;
        const int kt0 = t * BN;
        if (STAGES == 3 && t + 1 < te) wait_barrier<KR + DR>();
        else wait_barrier<0>();
        if (t + STAGES - 1 < te) issue(t + STAGES - 1);
        if (MASKED && ((int64_t)kt0 + BN - 1 < (int64_t)wrow0 + shift - a.wl ||
                       (int64_t)kt0 > (int64_t)wrow0 + 31 + shift + a.wr))
            return;
        const unsigned char LDS_AS *st = (const unsigned char LDS_AS *)smem + ((t - tb) % STAGES) * STAGE_BYTES;
        const unsigned char LDS_AS *sd = st + KT_BYTES;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            // dS^T operand: lane owns query l32; element i of step kt is key kt0 + 32 kb + 16 kt +
            // 8 (i / 4) + 4 hh + i % 4, the k order of the K^T operand below
            bf16x8 dsb[2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) dsb[kt] = tr_frag(sd + kb * 16384, daddr[kt][0], daddr[kt][1]);
            if (MASKED) {
                const int kb0 = kt0 + kb * 32;
                const int dlo = klo - kb0 - 4 * hh, dhi = khi - kb0 - 4 * hh;
                const bool cut_lo = kb0 < klo_w, cut_hi = kb0 + 31 > khi_w;
                if (cut_lo || cut_hi) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int off = 8 * (r >> 2) + (r & 3);
                        if ((cut_lo && off < dlo) || (cut_hi && off > dhi)) dsb[r >> 3][r & 7] = (__bf16)0.f;
                    }
                }
            }
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                const int roff = (kb * 32 + kt * 16) * ROWB;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const bf16x8 kt_ = tr_frag(st, taddr[mb][0] + roff, taddr[mb][1] + roff);
                    dq[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt_, dsb[kt], dq[mb], 0, 0, 0);
                }
            }
        }
    };

    if (tb < te) issue(tb);
    if (STAGES == 3 && tb + 1 < te) issue(tb + 1);
    int t = tb;
    for (; t < ua; ++t) step(t, std::true_type{});
    for (; t < ub; ++t) step(t, std::false_type{});
    for (; t < te; ++t) step(t, std::true_type{});

    __syncthreads();  // every wave has finished reading the ring
    store_rows_bf16<HD>(dq, a.scale, (unsigned char LDS_AS *)smem + wave * 32 * ROWB, (unsigned char *)a.dq,
                        (int64_t)b * a.sdq.b + head_offset(a.sdq, hf, a.Hin) + (int64_t)wrow0 * a.sdq.m, a.sdq.m,
                        Lq - wrow0);
}

template <int HD>
hipError_t launch_hd(const BwdArgs &a, hipStream_t stream) {
    constexpr int NW_Q = 8;
    // LDS ring depth of the two kernels: 2 (one tile in flight while one is used); a third
    // stage was measured no faster for either and costs registers
#ifndef BWD_STAGES_Q
#define BWD_STAGES_Q 2
#endif
#ifndef BWD_STAGES_KV
#define BWD_STAGES_KV 2
#endif
    const int64_t gq = (int64_t)((a.max_seqlen_q + NW_Q * 32 - 1) / (NW_Q * 32)) * a.nseq * a.B * a.Htot;
    const int64_t gkv = (int64_t)((a.max_seqlen_k + 127) / 128) * a.nseq * a.B * a.Htot;
    if (gq > 0x7fffffff || gkv > 0x7fffffff) return hipErrorInvalidConfiguration;
    if constexpr (HD == 128) if (a.ds) {
        // one sequence: D and L first, then dK/dV (writing dS), then dQ from dS
        constexpr int PREP_ROWS = 4 * (64 / (HD / 8)) * PREP_ITER;  // rows per 256-thread workgroup
        const int64_t gp = ((int64_t)a.B * a.Htot * a.Mq + PREP_ROWS - 1) / PREP_ROWS;
        if (gp > 0x7fffffff) return hipErrorInvalidConfiguration;
        if (gp > 0) hipLaunchKernelGGL((bwd_prep_kernel<HD>), dim3((unsigned)gp), dim3(256), 0, stream, a);
        if (gkv > 0)
            hipLaunchKernelGGL((bwd_dkdv_pair_kernel<HD, BWD_STAGES_KV, true>), dim3((unsigned)gkv), dim3(512), 0, stream, a);
        if (gq > 0) hipLaunchKernelGGL((bwd_dq_ds_kernel<HD, 3>), dim3((unsigned)gq), dim3(512), 0, stream, a);
        return hipGetLastError();
    }
    // the dQ launch writes the per-row D and L that the dK/dV launch reads
    if (gq > 0) hipLaunchKernelGGL((bwd_dq_kernel<HD, NW_Q, BWD_STAGES_Q>), dim3((unsigned)gq), dim3(NW_Q * 64), 0, stream, a);
    if (gkv > 0) hipLaunchKernelGGL((bwd_dkdv_pair_kernel<HD, BWD_STAGES_KV>), dim3((unsigned)gkv), dim3(512), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs &a, hipStream_t stream) {
    if (a.D == 128) return launch_hd<128>(a, stream);
    if (a.D == 64) return launch_hd<64>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace attn
