// Split-KV decode: per-chunk partial attention for one query row per (batch, head)
// ("MSLK Kernel Library -- Complete Reference", Glossary, split-K / split-KV:
// parallelise the reduction over the KV sequence, then combine partials; the
// chunk results are exactly those of memory_efficient_attention_partial on
// each key chunk, and the merge kernel combines them).
//
// The work is a stream over the K/V cache, about one flop per byte, so the
// kernel is built for HBM bandwidth, not for the matrix cores:
//   * one workgroup (4 waves) per (chunk, batch, group of hpw neighbouring heads); hpw
//     is picked so that a cache row's segments of those heads are 512 contiguous bytes
//     (a lone 128- or 256-byte head segment per row streams markedly slower);
//   * a lane group of D/8 (bf16), D/16 (FP8) or D/32 (INT4) lanes reads one key row of one
//     head with 16-byte loads; K and V rows of the same keys are loaded together, eight
//     rows per lane (four for INT4) in flight before any arithmetic;
//   * every lane group keeps its own online softmax (base-2 running max, sum of
//     exponentials, p-weighted V columns) over the rows it reads, so there is no score
//     buffer and no barrier in the stream; at the end the states of a head's lane
//     groups are combined exactly through LDS (the same LSE-weighted merge as between
//     chunks);
//   * KV-cache layouts ("Attention - Biases & masks": BlockDiagonalPaddedKeysMask,
//     PagedBlockDiagonalPaddedKeysMask): per-sequence key counts on the device,
//     and for a paged cache the physical row of every key of a sub-chunk is
//     resolved once into LDS from the block table;
//   * quantised caches: row/group-wise FP8 ("Attention - operator protocol", InputsFp8),
//     MXFP8 (InputsMXFp8: one E8M0 scale 2^(e - 127) per block of 32, no shift) and
//     row/group-wise INT4 (triton_splitk.FwOp).  A lane takes 16 E4M3 codes (hardware
//     conversion) or 32 4-bit codes per 16-byte load, all inside one (scale, shift) group;
//     the group's pair is applied to the lane's partial dot product before the reduction
//     over the row's lanes, since q.(c*scale + shift) = scale*(q.c) + shift*sum(q), and on
//     the V side the weight p*scale multiplies the codes while p*shift is summed once per
//     row and lane.  On the K side INT4 codes become the bf16 values 128 + 8 * code (a shift
//     and one v_and_or_b32 per pair) and feed v_dot2_f32_bf16 against q's bf16 pairs (exact
//     products, fp32 sums); 128 * sum(q) is taken off afterwards.  The V side converts the
//     codes exactly and accumulates in fp32.
// Output: the chunk's normalised fp32 output and its natural-log LSE; an empty
// chunk gives 0 and -inf.
#include <type_traits>

#include "kernels.h"

namespace attn {
namespace {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr int NT = 256;
constexpr int SUB = 2048;  // keys per sub-chunk of a paged cache (their rows are resolved into LDS)
// Tuning (measured on the [16, 32768, 32, 128] decode): 8 key rows per lane in flight (4 for
// INT4), no software pipelining of rounds, 512 contiguous bytes per cache row and workgroup.
#ifndef DECODE_UNROLL
#define DECODE_UNROLL 8
#endif
#ifndef DECODE_UNROLL_INT4
#define DECODE_UNROLL_INT4 4
#endif
constexpr int U_DEF = DECODE_UNROLL;       // key rows per lane and round
constexpr int U_INT4 = DECODE_UNROLL_INT4;  // the same for INT4 caches (32 codes per lane and row)

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

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

// 16 OCP E4M3 codes (byte i of word j is element 4j+i) to fp32; exact.
__device__ __forceinline__ void unpack_fp8(const u32x4 &w, float *x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
        const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
        x[4 * i] = lo[0];
        x[4 * i + 1] = lo[1];
        x[4 * i + 2] = hi[0];
        x[4 * i + 3] = hi[1];
    }
}

template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the LPK consecutive lanes of a lane group.  Groups of 4, 8 and 16 lanes use DPP
// (no LDS round trip): each step adds a lane's value to its partner's under a pairing that is
// its own inverse (rotate by 8 in a 16-lane row, which is lane xor 8; mirror within 8 lanes;
// xor 2 and xor 1 inside quads), so every lane of the group ends with the same bits.
template <int LPK>
__device__ __forceinline__ float lane_group_sum(float x) {
    if constexpr (LPK == 4 || LPK == 8 || LPK == 16) {
        if constexpr (LPK == 16) x = dpp_add<0x128>(x);  // row_ror:8
        if constexpr (LPK >= 8) x = dpp_add<0x141>(x);   // row_half_mirror
        x = dpp_add<0x4E>(x);                            // quad_perm [2, 3, 0, 1]
        x = dpp_add<0xB1>(x);                            // quad_perm [1, 0, 3, 2]
        return x;
    } else {
#pragma unroll
        for (int o = LPK / 2; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
        return x;
    }
}

// 32 unsigned 4-bit codes (element 2i in the low nibble of byte i) to fp32; exact.  The masked
// words are hidden from the compiler so that each byte converts with one v_cvt_f32_ubyte{0..3}
// instead of a field extract plus a conversion.
__device__ __forceinline__ void unpack_int4(const u32x4 &w, float *x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        unsigned lo = w[i] & 0x0f0f0f0fu, hi = (w[i] >> 4) & 0x0f0f0f0fu;
        asm("" : "+v"(lo), "+v"(hi));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[8 * i + 2 * j] = (float)((lo >> (8 * j)) & 0xffu);
            x[8 * i + 2 * j + 1] = (float)((hi >> (8 * j)) & 0xffu);
        }
    }
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16x2 as_bf16x2(unsigned w) { return __builtin_bit_cast(bf16x2, w); }

// Two 4-bit codes as the bf16 values 128 + 8 * code: the code fills mantissa bits 3..6 of 2^7
// (0x4300), which keeps the offset only 2x the largest code term.  Shifting the word so that
// nibble s sits at bits 3..6 and masking with 0x00780078 picks elements s and 4 + s of the
// word's 8 (s = 0..3).  The two constants come in registers (m = 0x00780078, c = 0x43004300)
// that the compiler cannot see through, so the mask and the or fuse into one v_and_or_b32.
__device__ __forceinline__ unsigned int4_pair(unsigned w, int s, unsigned m, unsigned c) {
    const unsigned x = s == 0 ? w << 3 : w >> (4 * s - 3);
    return (x & m) | c;
}

template <int ELEM>
__device__ __forceinline__ void unpack_elem(const u32x4 &w, float *x) {
    if constexpr (ELEM == DECODE_FP8 || ELEM == DECODE_MXFP8)
        unpack_fp8(w, x);
    else if constexpr (ELEM == DECODE_INT4)
        unpack_int4(w, x);
    else
        unpack<ELEM == DECODE_F32>(w, x);
}

// (scale, shift) halves of a metadata word: two fp16 in 32 bits (scale in the low half), or two
// fp32 in 64 bits (scale in the low word)
__device__ __forceinline__ float ss_scale(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)); }
__device__ __forceinline__ float ss_shift(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }
__device__ __forceinline__ float ss_scale(uint64_t w) { return __uint_as_float((uint32_t)w); }
__device__ __forceinline__ float ss_shift(uint64_t w) { return __uint_as_float((uint32_t)(w >> 32)); }
// An E8M0 block scale 2^(e - 127) as fp32: the exponent field itself, 2^-127 (a subnormal) for
// e = 0, NaN for e = 255.
__device__ __forceinline__ float e8m0_scale(uint32_t e) {
    return __uint_as_float(e == 0 ? 0x00400000u : (e == 255 ? 0x7fc00000u : e << 23));
}

// Workgroups are dealt to the 8 XCDs round-robin (workgroup i to XCD i % 8).  Renumbered so
// that every XCD takes one contiguous range of the logical order: the workgroups of one cache
// row range (neighbouring heads, which share DRAM pages and the lines of quantisation metadata) then run
// on one XCD at about the same time.  A bijection on [0, n).
__device__ __forceinline__ int xcd_remap(int i, int n) {
    const int x = i & 7, k = i >> 3, q = n >> 3, r = n & 7;
    return x * q + min(x, r) + k;
}

// MODE 0: k/v [B, Mkv, ...], every sequence has Mkv keys.  MODE 1: padded lanes [B, cap, ...] with
// seqlens[b] valid keys.  MODE 2: paged cache [1, num_pages * page_size, ...]; key j of sequence b is
// row block_tables[b][j / page_size] * page_size + j % page_size (page numbers clamped to the cache).
// SS32 (FP8 and INT4 caches): (scale, shift) pairs of two fp32 instead of two fp16.
template <int HD, int ELEM, int MODE, bool SS32 = false>
__global__ __launch_bounds__(NT) void decode_kernel(DecodeArgs a) {
    constexpr bool F32 = ELEM == DECODE_F32, INT4 = ELEM == DECODE_INT4, MX = ELEM == DECODE_MXFP8;
    constexpr bool QUANT = ELEM == DECODE_FP8 || INT4 || MX;       // codes + (scale, shift) or E8M0 metadata
    static_assert(!SS32 || ELEM == DECODE_FP8 || INT4, "fp32 scale/shift pairs: FP8 and INT4 caches");
    constexpr int MES = MX ? 1 : (SS32 ? 4 : 2);                   // bytes per metadata stride unit
    using MetaW = typename std::conditional<SS32, uint64_t, uint32_t>::type;  // one group's metadata
    constexpr int EPL = F32 ? 4 : (INT4 ? 32 : (QUANT ? 16 : 8));  // elements per 16-byte load
    constexpr int LPK = HD / EPL;                                  // lanes per key row (a lane group)
    constexpr int KPP = NT / LPK;                                  // lane groups of the workgroup
    constexpr int U = INT4 ? U_INT4 : U_DEF;                       // key rows per lane and round
    // cache element type (bytes for the quantised caches; their strides count bytes) and q's
    using T = typename std::conditional<F32, float, typename std::conditional<QUANT, uint8_t, __bf16>::type>::type;
    using QT = typename std::conditional<F32, float, __bf16>::type;
    constexpr int TPL = 16 / (int)sizeof(T);  // cache elements of type T per 16-byte load

    __shared__ float acc_s[KPP][HD];
    __shared__ float m_s[KPP], l_s[KPP], w_s[KPP];
    __shared__ int rows_s[MODE == 2 ? SUB : 1];  // physical cache row of each key of the sub-chunk

    // Workgroup = (chunk s, batch b, hpw consecutive heads).  Lane group g works on head slot
    // g % hpw and row slot g / hpw, so one pass reads hpw neighbouring head segments of each row.
    const int lh = a.log2_hpw, hpw = 1 << lh, RPP = KPP >> lh, R = RPP * U;
    int id = xcd_remap(blockIdx.x, gridDim.x);
    const int hg = id % (a.Htot >> lh);
    id /= a.Htot >> lh;
    const int b = id % a.B;
    const int s = id / a.B;
    const int Lb = MODE == 0 ? a.Mkv : min(max(a.seqlens[b], 0), a.cap);
    const int jb = a.window > 0 ? max(0, Lb - a.window) : 0;  // first key the query sees
    const int j0 = min(Lb, jb + s * a.chunk);
    const int j1 = min(Lb, j0 + a.chunk);
    const int64_t kb = MODE == 2 ? 0 : (int64_t)b * a.sk.b, vb = MODE == 2 ? 0 : (int64_t)b * a.sv.b;

    const int tid = threadIdx.x, g = tid / LPK, cl = tid % LPK;
    const int hs = g & (hpw - 1), rs = g >> lh;
    const int hf = (hg << lh) + hs;
    const QT *qp = (const QT *)a.q + (int64_t)b * a.sq.b + head_offset(a.sq, hf, a.Hin) + cl * EPL;
    const T *kp = (const T *)a.k + kb + head_offset(a.sk, hf, a.Hin) + cl * TPL;
    const T *vp = (const T *)a.v + vb + head_offset(a.sv, hf, a.Hin) + cl * TPL;
    // quantised caches: the metadata of this lane's group in every row, a (scale, shift) word
    // addressed in fp16 (fp32 with SS32) units like a [.., G, 2] tensor, or an E8M0 byte of a
    // [.., D/32] tensor
    // (a lane's EPL elements never straddle two groups)
    const char *kss = nullptr, *vss = nullptr;
    const int gw = QUANT ? (MX ? 1 : 2) * ((cl * EPL) / a.group) : 0;
    if constexpr (QUANT) {
        kss = (const char *)a.kss + ((MODE == 2 ? 0 : (int64_t)b * a.skss.b) + head_offset(a.skss, hf, a.Hin) + gw) * MES;
        vss = (const char *)a.vss + ((MODE == 2 ? 0 : (int64_t)b * a.svss.b) + head_offset(a.svss, hf, a.Hin) + gw) * MES;
    }
    auto meta = [](const char *p) __attribute__((always_inline)) -> MetaW {
        if constexpr (SS32)
            return *(const uint64_t *)p;
        else
            return MX ? (uint32_t)*(const uint8_t *)p : *(const uint32_t *)p;
    };

    float qv[EPL];
    if constexpr (F32) {
        unpack<true>(*(const u32x4 *)qp, qv);
    } else {
#pragma unroll
        for (int i = 0; i < EPL / 8; ++i) unpack<false>(*(const u32x4 *)(qp + 8 * i), qv + 8 * i);
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) qv[e] *= a.scale_log2;
    // quantised caches: scale_log2 * (sum of this lane's q elements), the weight of its group's
    // shift; q.(c*scale + shift) summed over the lanes = sum of scale*(q.c) + shift*sum(q)
    float qsum = 0.f;
    if constexpr (QUANT) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) qsum += qv[e];
    }
    // INT4 K side on v_dot2: q's bf16 pairs in the order int4_pair() yields the codes (elements
    // 8i + s and 8i + 4 + s in pair 4i + s) and the sum of q (times 128, the codes' offset)
    unsigned q2[INT4 ? 16 : 1];
    float qraw = 0.f;
    unsigned m4 = 0x00780078u, c43 = 0x43004300u;
    asm("" : "+v"(m4), "+v"(c43));
    if constexpr (INT4) {
        const uint16_t *qh = (const uint16_t *)qp;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
                const unsigned lo = qh[8 * i + s2], hi = qh[8 * i + 4 + s2];
                q2[4 * i + s2] = lo | (hi << 16);
                qraw += __uint_as_float(lo << 16) + __uint_as_float(hi << 16);
            }
    }

    // Online softmax state of this lane group (the same in its LPK lanes): base-2 running max,
    // sum of exponentials, p-weighted values (this lane's EPL columns) and, for the quantised
    // caches, the sum of p * shift of this lane's group.
    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
    float m_run = -INFINITY, l_run = 0.f, sh_acc = 0.f;

    constexpr int NS = QUANT ? U : 1;
    u32x4 wk[U], wv[U];
    MetaW sk[NS], sv[NS];
    // lane32 path: uniform bases at head hf0 = hg * hpw, byte strides, 32-bit lane offsets
    // (head part + 16-byte column slice + row slot); the launcher checks that they fit
    const int hf0 = hg << lh;
    const char *kbase = (const char *)a.k + (kb + head_offset(a.sk, hf0, a.Hin)) * (int64_t)sizeof(T);
    const char *vbase = (const char *)a.v + (vb + head_offset(a.sv, hf0, a.Hin)) * (int64_t)sizeof(T);
    const int64_t kstr = a.sk.m * (int64_t)sizeof(T), vstr = a.sv.m * (int64_t)sizeof(T);
    const uint32_t klane = (uint32_t)((head_offset(a.sk, hf, a.Hin) - head_offset(a.sk, hf0, a.Hin) + cl * TPL) *
                                      (int64_t)sizeof(T) + rs * kstr);
    const uint32_t vlane = (uint32_t)((head_offset(a.sv, hf, a.Hin) - head_offset(a.sv, hf0, a.Hin) + cl * TPL) *
                                      (int64_t)sizeof(T) + rs * vstr);
    const char *ksbase = nullptr, *vsbase = nullptr;
    int64_t ksstr = 0, vsstr = 0;
    uint32_t kslane = 0, vslane = 0;
    if constexpr (QUANT) {
        const int64_t bk = MODE == 2 ? 0 : (int64_t)b * a.skss.b, bv = MODE == 2 ? 0 : (int64_t)b * a.svss.b;
        ksbase = (const char *)a.kss + (bk + head_offset(a.skss, hf0, a.Hin)) * MES;
        vsbase = (const char *)a.vss + (bv + head_offset(a.svss, hf0, a.Hin)) * MES;
        ksstr = a.skss.m * MES;
        vsstr = a.svss.m * MES;
        kslane = (uint32_t)((head_offset(a.skss, hf, a.Hin) - head_offset(a.skss, hf0, a.Hin) + gw) * MES + rs * ksstr);
        vslane = (uint32_t)((head_offset(a.svss, hf, a.Hin) - head_offset(a.svss, hf0, a.Hin) + gw) * MES + rs * vsstr);
    }

    // byte distance between row slot 0 of consecutive rows of a lane (RPP rows apart)
    const int64_t kstep = RPP * kstr, vstep = RPP * vstr, ksstep = RPP * ksstr, vsstep = RPP * vsstr;
    for (int sub0 = j0; sub0 < j1; sub0 += (MODE == 2 ? SUB : a.chunk)) {
        const int n = MODE == 2 ? min(SUB, j1 - sub0) : j1 - sub0;
        if (MODE == 2) {
            __syncthreads();  // the previous sub-chunk's rows are no longer read
            const int32_t *bt = a.block_tables + (int64_t)b * a.bt_stride;
            for (int i = tid; i < n; i += NT) {
                const int j = sub0 + i;
                const int pg = min(max(bt[j / a.page_size], 0), a.num_pages - 1);
                rows_s[i] = pg * a.page_size + j % a.page_size;
            }
            __syncthreads();
        }
        // K and V rows of the same keys are read together, in rounds of R keys (U per lane),
        // straight into the registers the round computes on.  A full round (every row < n) takes
        // no per-lane checks; with `lane32` the row part of each address is uniform and the
        // lane's part a 32-bit byte offset, so address arithmetic stays on the scalar unit.
        auto load = [&](int p, auto full_tag) __attribute__((always_inline)) {
            constexpr bool FULL = decltype(full_tag)::value;
            if constexpr (QUANT && MODE != 2 && FULL) {
                // quantised caches: the round's uniform row bases (row slot 0 of its first row) are
                // formed once, and each row adds a uniform step and the lanes' 32-bit offsets
                // (FP8 and INT4 4-6% faster than per-row bases; bf16 1% slower, so it keeps those)
                if (a.lane32) {
                    const int64_t r0 = sub0 + p;
                    const char *kr = kbase + r0 * kstr, *vr = vbase + r0 * vstr;
                    const char *ksr = ksbase + r0 * ksstr, *vsr = vsbase + r0 * vsstr;
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        wk[u] = *(const u32x4 *)(kr + u * kstep + klane);
                        wv[u] = *(const u32x4 *)(vr + u * vstep + vlane);
                        sk[u] = meta(ksr + u * ksstep + kslane);
                        sv[u] = meta(vsr + u * vsstep + vslane);
                    }
                    return;
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int r = p + u * RPP + rs;
                const bool ok = FULL || r < n;
                if (MODE != 2 && a.lane32 && FULL) {
                    const int64_t ru = sub0 + p + u * RPP;  // uniform row of this lane's row slot 0
                    wk[u] = *(const u32x4 *)(kbase + ru * kstr + klane);
                    wv[u] = *(const u32x4 *)(vbase + ru * vstr + vlane);
                    if constexpr (QUANT) {
                        sk[u] = meta(ksbase + ru * ksstr + kslane);
                        sv[u] = meta(vsbase + ru * vsstr + vslane);
                    }
                } else {
                    const int64_t row = MODE == 2 ? (ok ? rows_s[r] : 0) : sub0 + r;
                    wk[u] = ok ? *(const u32x4 *)(kp + row * a.sk.m) : u32x4{0, 0, 0, 0};
                    wv[u] = ok ? *(const u32x4 *)(vp + row * a.sv.m) : u32x4{0, 0, 0, 0};
                    if constexpr (QUANT) {
                        sk[u] = ok ? meta(kss + row * a.skss.m * MES) : 0u;
                        sv[u] = ok ? meta(vss + row * a.svss.m * MES) : 0u;
                    }
                }
            }
        };
        auto load_round = [&](int p) __attribute__((always_inline)) {
            if (p + R <= n)
                load(p, std::true_type{});
            else
                load(p, std::false_type{});
        };
        load_round(0);
        for (int p = 0; p < n; p += R) {
            float sc[U];
            float mx = -INFINITY;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float dot = 0.f;
                if constexpr (INT4) {
                    // sum of q * (128 + 8 code) over the lane's 32 elements, in two chains
                    float d0 = 0.f, d1 = 0.f;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int s2 = 0; s2 < 4; ++s2) {
                            float &d = (i & 1) ? d1 : d0;
                            d = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(int4_pair(wk[u][i], s2, m4, c43)),
                                                                as_bf16x2(q2[4 * i + s2]), d, false);
                        }
                    const float qc = ((d0 + d1) - 128.f * qraw) * 0.125f;  // q.code
                    dot = a.scale_log2 * fmaf(ss_scale(sk[u]), qc, ss_shift(sk[u]) * qraw);
                } else {
                    float x[EPL];
                    unpack_elem<ELEM>(wk[u], x);
#pragma unroll
                    for (int e = 0; e < EPL; ++e) dot = fmaf(qv[e], x[e], dot);
                    if constexpr (MX)
                        dot *= e8m0_scale(sk[u]);
                    else if constexpr (QUANT)
                        dot = fmaf(ss_scale(sk[u]), dot, ss_shift(sk[u]) * qsum);
                }
                dot = lane_group_sum<LPK>(dot);
                sc[u] = p + u * RPP + rs < n ? dot : -INFINITY;
                mx = fmaxf(mx, sc[u]);
            }
            const float m_new = fmaxf(m_run, mx);
            const float mu = m_new == -INFINITY ? 0.f : m_new;  // no row seen yet: keep exponents finite
            const float alpha = __builtin_amdgcn_exp2f(m_run - mu);
            m_run = m_new;
            l_run *= alpha;
            sh_acc *= alpha;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[e] *= alpha;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float pr = __builtin_amdgcn_exp2f(sc[u] - mu);
                l_run += pr;
                if constexpr (MX) {
                    pr *= e8m0_scale(sv[u]);
                } else if constexpr (QUANT) {
                    sh_acc = fmaf(pr, ss_shift(sv[u]), sh_acc);
                    pr *= ss_scale(sv[u]);
                }
                float x[EPL];
                unpack_elem<ELEM>(wv[u], x);
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[e] = fmaf(pr, x[e], acc[e]);
            }
            if (p + R < n) load_round(p + R);
        }
    }

    // exact combine of the lane groups' states, per head: groups hs, hs + hpw, ... hold head slot hs
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc_s[g][cl * EPL + e] = acc[e] + sh_acc;
    if (cl == 0) {
        m_s[g] = m_run;
        l_s[g] = l_run;
    }
    __syncthreads();
    if (tid < KPP) {
        float M = -INFINITY;
        for (int r = tid & (hpw - 1); r < KPP; r += hpw) M = fmaxf(M, m_s[r]);
        w_s[tid] = __builtin_amdgcn_exp2f(m_s[tid] - (M == -INFINITY ? 0.f : M));
    }
    __syncthreads();
    const int64_t obase = ((int64_t)s * a.B + b) * a.Htot + (hg << lh);  // first head of the workgroup
    for (int t = tid; t < HD << lh; t += NT) {
        const int h = t / HD, d = t % HD;
        float tot = 0.f, L = 0.f;
        for (int r = h; r < KPP; r += hpw) {
            tot = fmaf(acc_s[r][d], w_s[r], tot);
            L = fmaf(l_s[r], w_s[r], L);
        }
        a.ws_o[(obase + h) * HD + d] = L > 0.f ? tot / L : 0.f;
    }
    if (tid < hpw) {
        float M = -INFINITY, L = 0.f;
        for (int r = tid; r < KPP; r += hpw) M = fmaxf(M, m_s[r]);
        for (int r = tid; r < KPP; r += hpw) L = fmaf(l_s[r], w_s[r], L);
        a.ws_lse[obase + tid] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
    }
}

#ifndef DECODE_ROW_BYTES
#define DECODE_ROW_BYTES 512
#endif
template <int HD, int ELEM, int MODE, bool SS32 = false>
hipError_t launch(const DecodeArgs &args, hipStream_t stream) {
    // heads per workgroup: enough neighbouring head segments for DECODE_ROW_BYTES contiguous bytes
    // per cache row, a power of two that divides Htot and leaves every head at least one lane group
    constexpr bool FP8 = ELEM == DECODE_FP8 || ELEM == DECODE_MXFP8;
    constexpr int RB = ELEM == DECODE_F32 ? 4 * HD : (FP8 ? HD : (ELEM == DECODE_INT4 ? HD / 2 : 2 * HD));
    constexpr int KPP = NT / (RB / 16);  // lane groups: one 16-byte load per lane per row
    DecodeArgs a = args;
    a.log2_hpw = 0;
    while ((RB << (a.log2_hpw + 1)) <= DECODE_ROW_BYTES && (2 << a.log2_hpw) <= KPP &&
           a.Htot % (2 << a.log2_hpw) == 0)
        ++a.log2_hpw;
    // lane32: within every workgroup (hpw heads from a multiple of hpw, RPP row slots, LPK
    // 16-byte column slices) the offsets from the first head's row are >= 0 and < 2^32 bytes
    constexpr int EPL = ELEM == DECODE_F32 ? 4 : (ELEM == DECODE_INT4 ? 32 : (FP8 ? 16 : 8));
    constexpr int LPK = HD / EPL;
    const int64_t RPP = (NT / LPK) >> a.log2_hpw, hpw = 1 << a.log2_hpw;
    auto fits = [&](const Strides &st, int64_t es, int64_t col) {
        int64_t lo = 0, hi = 0;
        for (int h0 = 0; h0 < a.Htot; h0 += (int)hpw)
            for (int h = h0; h < h0 + hpw; ++h) {
                const int64_t d = head_offset(st, h, a.Hin) - head_offset(st, h0, a.Hin);
                lo = d < lo ? d : lo;
                hi = d > hi ? d : hi;
            }
        return lo >= 0 && (hi + col) * es + (RPP - 1) * st.m * es < (int64_t(1) << 32);
    };
    const int64_t es = ELEM == DECODE_F32 ? 4 : (ELEM == DECODE_BF16 ? 2 : 1);
    a.lane32 = MODE != 2 && fits(a.sk, es, 16 / es * (LPK - 1)) && fits(a.sv, es, 16 / es * (LPK - 1));
    if (ELEM == DECODE_FP8 || ELEM == DECODE_INT4)
        a.lane32 = a.lane32 && fits(a.skss, SS32 ? 4 : 2, 2 * ((LPK - 1) * EPL / a.group)) &&
                   fits(a.svss, SS32 ? 4 : 2, 2 * ((LPK - 1) * EPL / a.group));
    if (ELEM == DECODE_MXFP8)  // one E8M0 byte per block
        a.lane32 = a.lane32 && fits(a.skss, 1, (LPK - 1) * EPL / a.group) && fits(a.svss, 1, (LPK - 1) * EPL / a.group);
    const int64_t grid = (int64_t)a.S * a.B * (a.Htot >> a.log2_hpw);
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((decode_kernel<HD, ELEM, MODE, SS32>), dim3((unsigned)grid), dim3(NT), 0, stream, a);
    return hipGetLastError();
}

template <int HD, int ELEM, bool SS32 = false>
hipError_t launch_mode(const DecodeArgs &a, hipStream_t stream) {
    if (a.block_tables) return launch<HD, ELEM, 2, SS32>(a, stream);
    if (a.seqlens) return launch<HD, ELEM, 1, SS32>(a, stream);
    return launch<HD, ELEM, 0, SS32>(a, stream);
}

template <int HD>
hipError_t launch_elem(const DecodeArgs &a, int elem, hipStream_t stream) {
    switch (elem) {
    case DECODE_BF16: return launch_mode<HD, DECODE_BF16>(a, stream);
    case DECODE_F32: return launch_mode<HD, DECODE_F32>(a, stream);
    case DECODE_FP8: return a.ss32 ? launch_mode<HD, DECODE_FP8, true>(a, stream) : launch_mode<HD, DECODE_FP8>(a, stream);
    case DECODE_INT4: return a.ss32 ? launch_mode<HD, DECODE_INT4, true>(a, stream) : launch_mode<HD, DECODE_INT4>(a, stream);
    case DECODE_MXFP8: return launch_mode<HD, DECODE_MXFP8>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode_partials(const DecodeArgs &a, int elem, hipStream_t stream) {
    if (a.D == 128) return launch_elem<128>(a, elem, stream);
    if (a.D == 64) return launch_elem<64>(a, elem, stream);
    if (a.D == 256) return launch_elem<256>(a, elem, stream);
    return hipErrorInvalidValue;
}

}  // namespace attn
