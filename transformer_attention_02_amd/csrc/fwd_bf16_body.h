#pragma once
// Fused attention forward for bf16 inputs on gfx950 matrix cores: the kernel template and its
// launch helpers, shared by fwd_bf16.hip (value head dims up to 128) and fwd_bf16_v256.hip
// (value head dim 256), which are compiled with different instruction schedulers.
//
//
// Computes, per (batch, head) and query row i, out_i = softmax_j(scale q_i.k_j) v_j
// over the visible keys and lse_i = ln sum_j exp(scale q_i.k_j), without ever
// writing the score matrix to memory (MSLK kernel reference, "Attention - Core
// fMHA": memory_efficient_attention_forward_requires_grad and
// memory_efficient_attention_partial; masks from "Attention - Biases & masks":
// LowerTriangularMask, BlockDiagonalMask, BlockDiagonalCausalMask).
//
// Work decomposition
//   One workgroup = 8 waves = 256 query rows of one (batch, head[, sequence]);
//   each wave owns 32 rows, and two waves share each SIMD so that one wave's
//   softmax arithmetic runs while the other's matrix products execute.
//   Key/value tiles of 64 rows stream through an LDS ring filled by buffer
//   loads that write straight into LDS (no staging registers).  With 8 waves
//   the ring has 4 slots filled two tiles at a time: at the first tile of each
//   pair the waves wait for that pair and a barrier, then the next pair's loads
//   go into the slots just finished, so a pair is in flight while one is
//   computed.  Smaller workgroups keep a 3-slot ring with one barrier per tile
//   (tiles t+1 and t+2 in flight).  Rows past the end of the keys fall outside
//   the buffer descriptor's range and arrive as zeros.
//
// Matrix-core layout (v_mfma_f32_32x32x16_bf16, A 32x16, B 16x32, C 32x32)
//   S^T = K Q^T: A = K rows from LDS (m = key, k = head dim, one 16-byte read),
//   B = Q^T kept in registers (n = query row).  In the C layout lane l owns
//   query row l%32 and 16 keys of each 32-key block, so the softmax row
//   statistics are in-lane reductions plus one v_permlane32_swap.
//   O^T += V^T P^T: B = P^T straight from the S^T registers; the C layout gives
//   lane half h the keys {8a + 4h + 0..3}, which defines the k order of the
//   product.  The A operand V^T is read from row-major V with two
//   ds_read_b64_tr_b16 per 16-key step: inside each group of 16 lanes the
//   instruction returns to lane i element i%4 of the 8-byte pieces addressed by
//   lanes 4j + i/4, so lanes pointing at 4 consecutive key rows and 4-dim column
//   pieces deliver each lane 4 keys of its own head-dim column.
//   Both tiles are row-major with the 16-byte chunk index XOR-swizzled by the
//   row, so that 16 lanes reading one chunk of 16 rows (K) or 32-byte pieces of
//   4 rows (V) hit distinct LDS banks.
//
// Online softmax in base 2: x = s * scale * log2(e).  Each row keeps a
// reference maximum m and the sum l of 2^(x - m); the reference is raised
// (and O, l rescaled) only when a new x exceeds it by more than 8, so most
// tiles skip the rescale.  Once every row of a wave has a finite reference, a
// tile takes its exponentials against it straight away and checks afterwards:
// each lane's partial row sum bounds every value it summed, so a sum of at most
// 2^8 shows that no value needs the rescale and the tile's row maximum is never
// formed.  A tile that fails the check computes its scores again from the K
// tile still in LDS and takes the exact path (row maximum, rescale,
// exponentials).  P is rounded to bf16 for the product with V; l accumulates
// the fp32 values.  lse = (m + log2 l) * ln 2.
// Masks are one visible-key interval per row (causal, bottom-right, sliding
// windows).  Tiles outside every window of a wave's rows are skipped by that
// wave; the element mask is applied only on tiles that cut a window edge or
// the end of the keys.
#include <type_traits>

#include "kernels.h"
#include "tile_common.h"

namespace attn {
namespace {

constexpr int BN = 64;         // keys per tile
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescaleThreshold = 8.0f;  // log2 units
constexpr float kSumThreshold = 256.0f;    // 2^kRescaleThreshold

__device__ __forceinline__ float pair_max(float x) {
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// NW waves per workgroup; STAGES-deep LDS ring of K/V tiles; KD and VD are the head dims of
// q/k and of v/out.  KSPLIT waves share each 32-row block: with KSPLIT = 2 (and the paired ring)
// wave 2i takes the first tile of every resident pair and wave 2i + 1 the second, and their
// softmax states are merged exactly at the end.
// Entries of a sequence's block-table row resolved into LDS (32 KB): paged caches of up to this many
// pages per sequence.
constexpr int kMaxPages = 8192;

// VSPLIT waves share each 32-row block by value columns: with VSPLIT = 2 wave w + NW/2 keeps the
// second half of O^T.  Over a paged cache both waves compute the whole score tile and its softmax
// (the page table fills the LDS past the ring); otherwise (SSPLIT) each computes the scores of
// its own 32 keys of every tile, and the pair exchanges its row maxima and bf16 P halves through
// LDS, so that neither the matrix ops nor the exponentials of the scores are done twice.
template <int KD, int VD, int NW, int STAGES, bool OUT_F32, int KSPLIT, bool PAGED, int VSPLIT = 1>
__device__ __forceinline__ void fwd_bf16_body(const FwdArgs &a) {
    constexpr int NT = NW * 64;                  // threads per workgroup
    constexpr int BM = NW / KSPLIT / VSPLIT * 32;  // query rows per workgroup
    static_assert(VSPLIT == 1 || KSPLIT == 1, "keys or value columns are split, not both");
    static_assert(STAGES >= 2 && STAGES <= 4, "the unrolled tile loop names two to four LDS stages");
    // STAGES == 4: the ring is filled two tiles at a time, with one wait + barrier per two tiles
    constexpr bool PAIRS = STAGES == 4;
    static_assert(KSPLIT == 1 || (KSPLIT == 2 && PAIRS), "split keys need the paired ring");
    constexpr int KROWB = KD * 2, VROWB = VD * 2;    // bytes per K / V tile row
    constexpr int KCPR = KD / 8, VCPR = VD / 8;      // 16-byte chunks per row
    constexpr int KTILE = BN * KROWB, VTILE = BN * VROWB;
    constexpr int V_BASE = STAGES * KTILE;           // K tiles of all stages first, then the V tiles
    constexpr int KROUNDS = KTILE / 16 / NT;         // 16-byte loads per thread per K tile
    constexpr int VROUNDS = VTILE / 16 / NT;         // and per V tile
    constexpr int KS = KD / 16;                      // k-steps of S^T
    constexpr int MB = VD / 32 / VSPLIT;             // 32-row blocks of this wave's O^T
    constexpr int VW = VD / VSPLIT;                  // value columns of this wave
    static_assert(KROUNDS >= 1 && KROUNDS * NT * 16 == KTILE && VROUNDS >= 1 && VROUNDS * NT * 16 == VTILE,
                  "tile split");
    constexpr bool SSPLIT = VSPLIT == 2 && !PAGED;
    static_assert(!SSPLIT || (STAGES == 2 && NW == 8), "score halves pair wave w with wave w + 4");
    // score-split exchange area: per wave its bf16 P half ([2][64 lanes][16 bytes]), its 32 row
    // values (maxima, then the row sums) and its flag
    constexpr int XP_BYTES = NW * 2 * 64 * 16, XM_BYTES = NW * 32 * 4, XF_BYTES = NW * 4;

    __shared__ __attribute__((aligned(1024))) unsigned char smem[STAGES * (KTILE + VTILE)];
    // past the ring: a paged workgroup's page numbers, or the score-split exchange area
    __shared__ __attribute__((aligned(16))) unsigned char aux[PAGED ? kMaxPages * 4
                                                                   : (SSPLIT ? XP_BYTES + XM_BYTES + XF_BYTES : 16)];
    int LDS_AS *const ptab = (int LDS_AS *)aux;  // page numbers of this workgroup's key tiles
    unsigned char LDS_AS *const xp = (unsigned char LDS_AS *)aux;
    float LDS_AS *const xm = (float LDS_AS *)(aux + XP_BYTES);
    int LDS_AS *const xf = (int LDS_AS *)(aux + XP_BYTES + XM_BYTES);

    const int tid = threadIdx.x;
    const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // ---- which (key chunk, tile, sequence, batch*head) this workgroup owns; heaviest tiles first
    const int BH = a.B * a.Htot;
    const int tiles = (a.max_seqlen_q + BM - 1) / BM;
    int id = blockIdx.x;
    const int split = id % a.splits;
    id /= a.splits;
    int bh = id % BH;
    id /= BH;
    if (a.kv_groups > 0) {
        // expanded GQA: consecutive workgroup ids (round-robin over the XCDs) walk the groups
        // first, so that all heads of a group share an XCD and its L2 copy of the group's K/V
        const int r = bh % a.Htot;
        bh += (r % a.kv_groups) * a.Hin + r / a.kv_groups - r;
    }
    // expanded GQA over packed sequences: the query tiles of one sequence (longest first) run
    // together on the group's XCD, so they stream the sequence's keys in step and share them in
    // L2 (otherwise every tile level of every sequence in turn, heaviest first)
    const bool seq_major = a.kv_groups > 0 && a.nseq > 1;
    const int seq = seq_major ? id / tiles : id % a.nseq;
    const int tidx = seq_major ? id % tiles : id / a.nseq;  // 0: the sequence's heaviest row block
    const int b = bh / a.Htot, hf = bh % a.Htot;

    int qs = 0, qe = a.Mq, ks = 0, ke = a.Mkv;
    if (a.packed) {
        qs = min(max(a.seqstart_q[seq], 0), a.Mq);
        qe = min(max(a.seqstart_q[seq + 1], qs), a.Mq);
        if (a.seqlens_k) {
            // KV cache: the sequence's keys start at row 0 of its lane (or its first page), or at
            // row seqstart_k[seq] of the one k/v tensor (gappy lanes)
            ks = a.seqstart_k ? min(max(a.seqstart_k[seq], 0), a.Mkv) : 0;
            ke = ks + min(max(a.seqlens_k[seq], 0), a.cap - ks);
        } else {
            const int32_t *skp = a.seqstart_k ? a.seqstart_k : a.seqstart_q;
            ks = min(max(skp[seq], 0), a.Mkv);
            ke = min(max(skp[seq + 1], ks), a.Mkv);
        }
    }
    const int Lq = qe - qs, Lk = ke - ks;
    // Row blocks start at row 0, or end at the sequence's last row when its length leaves a
    // remainder r = Lq mod BM of at most BM - BN rows.  Aligned to the start, the ragged block is
    // the last one, which sees the most keys under a causal mask; aligned to the end, it is the
    // first one, which sees the fewest: (blocks - 1) (BM - ceil(r / BN) BN) / BN fewer key tiles.
    // With a larger remainder the tile counts are equal, and start alignment keeps the diagonal
    // on tile boundaries.  Either way tidx 0 is the block that ends at the last row.  A first
    // block aligned to the end starts before row 0; those rows hold nothing.
    const int rem = Lq % BM;
    const bool end_aligned = rem != 0 && rem <= BM - BN;
    const int row0 = end_aligned ? Lq - (tidx + 1) * BM : (tiles - 1 - tidx) * BM;
    if (end_aligned ? row0 + BM <= 0 : row0 >= Lq) return;  // no row of this sequence
    const int row0v = max(row0, 0);                          // the block's first row
    // this workgroup's key chunk [kc0, kc1) (the whole sequence unless the keys are split)
    const int kc0 = a.splits > 1 ? min(split * a.chunk, Lk) : 0;
    const int kc1 = a.splits > 1 ? min(kc0 + a.chunk, Lk) : Lk;
    // Visible keys of local row i: [lo(i), hi(i)] = [i + shift - wl, i + shift + wr] within [0, Lk),
    // both non-decreasing in i (64-bit: shift and the unbounded extents reach 2^31).
    const int64_t shift = a.bottom_right ? (int64_t)Lk - Lq : 0;
    auto clampk = [&](int64_t x, int64_t lo_, int64_t hi_) { return (int)(x < lo_ ? lo_ : (x > hi_ ? hi_ : x)); };
    const int row_last = min(row0 + BM, Lq) - 1;
    const int kbeg = clampk((int64_t)row0v + shift - a.wl, kc0, kc1);
    const int kend = clampk((int64_t)row_last + shift + a.wr + 1, kc0, kc1);
    // tiles [tb, te) hold every visible key; [ua, ub) need no mask for any row of the workgroup
    const int tb = kbeg / BN;
    const int te = kend > kbeg ? (kend + BN - 1) / BN : tb;
    int ua = (clampk((int64_t)row_last + shift - a.wl, 0, Lk) + BN - 1) / BN;
    int ub = clampk((int64_t)row0v + shift + a.wr + 1, 0, Lk) / BN;
    ua = min(max(ua, tb), te);
    ub = min(max(ub, ua), te);
    // Position p of the key loop takes the tile of [tb, te) congruent to p modulo the tile count: workgroups whose ranges have the same length and overlap (the query tiles of a
    // sliding window) then read each shared key tile at the same step, so the XCD's L2 serves the
    // later requests.  Ranges that start at tile 0 (causal, unmasked) keep their order.
    const int nt = te - tb;
    const int t_first = nt > 0 ? tb + (nt - tb % nt) % nt : tb;  // the tile at position 0
    int t_issue = t_first;  // the next tile to load (loads go out in position order)

    const __bf16 *qp = (const __bf16 *)a.q + (int64_t)b * a.sq.b + head_offset(a.sq, hf, a.Hin) + (int64_t)qs * a.sq.m;
    // K/V rows of key 0 (a KV cache's lane of this sequence; paged caches start at the cache)
    const int64_t kvb = a.seqlens_k && !PAGED && !a.seqstart_k ? seq : b;
    const __bf16 *kp = (const __bf16 *)a.k + (PAGED ? 0 : kvb * a.sk.b) + head_offset(a.sk, hf, a.Hin) + (int64_t)ks * a.sk.m;
    const __bf16 *vp = (const __bf16 *)a.v + (PAGED ? 0 : kvb * a.sv.b) + head_offset(a.sv, hf, a.Hin) + (int64_t)ks * a.sv.m;
    if constexpr (PAGED) {
        // page numbers of tiles [tb, te) (pages hold a whole number of 64-key tiles), clamped to the
        // cache; every wave reads them before its first tile load
        const int p0 = tb * BN / a.page_size, p1 = te > tb ? ((te * BN - 1) / a.page_size + 1) : p0;
        for (int i = p0 + tid; i < p1 && i - p0 < kMaxPages; i += NT)
            ptab[i - p0] = min(max(a.block_tables[(int64_t)seq * a.bt_stride + i], 0), a.num_pages - 1);
        __syncthreads();
    }
    const unsigned kstride = (unsigned)a.sk.m * 2u, vstride = (unsigned)a.sv.m * 2u;  // bytes per key row

    // ---- async tile loads: global -> LDS, 16 bytes per lane, OOB rows read as zeros
    // Slot p of a tile (16 bytes) holds row p / CPR, physical chunk p % CPR.
    unsigned koff[KROUNDS], voff[VROUNDS];
#pragma unroll
    for (int r = 0; r < KROUNDS; ++r) {
        const int p = (r * NW + wave) * 64 + lane;
        const int row = p / KCPR, c = (p % KCPR) ^ swz<KD>(row);
        koff[r] = row * kstride + c * 16;
    }
#pragma unroll
    for (int r = 0; r < VROUNDS; ++r) {
        const int p = (r * NW + wave) * 64 + lane;
        const int row = p / VCPR, c = (p % VCPR) ^ swz<VD>(row);
        voff[r] = row * vstride + c * 16;
    }
    const unsigned smem_base = (unsigned)(unsigned long long)(unsigned char LDS_AS *)smem;
    auto issue = [&](int p) __attribute__((always_inline)) {
        const int kt0 = t_issue * BN;
        t_issue = t_issue + 1 == te ? tb : t_issue + 1;
        const int nvalid = min(BN, Lk - kt0);
        const int slot = p % STAGES;
        const unsigned kst = smem_base + slot * KTILE, vst = smem_base + V_BASE + slot * VTILE;
        int64_t row = kt0;  // cache row of the tile's first key
        if constexpr (PAGED)
            row = (int64_t)min(max(ptab[kt0 / a.page_size - tb * BN / a.page_size], 0), a.num_pages - 1) * a.page_size +
                  kt0 % a.page_size;
        const i32x4 kr = make_rsrc(kp + row * a.sk.m, (nvalid - 1) * kstride + KROWB);
        const i32x4 vr = make_rsrc(vp + row * a.sv.m, (nvalid - 1) * vstride + VROWB);
#pragma unroll
        for (int r = 0; r < KROUNDS; ++r) dma16(kr, koff[r], kst + (r * NW + wave) * 1024);
#pragma unroll
        for (int r = 0; r < VROUNDS; ++r) dma16(vr, voff[r], vst + (r * NW + wave) * 1024);
    };

    // ---- Q^T fragments (B operand), resident for the whole kernel
    const int wsub = wave % KSPLIT;                // which tile of each pair this wave takes (KSPLIT = 2)
    const int vpart = wave / (NW / VSPLIT);        // which value columns this wave keeps (VSPLIT = 2)
    const int wrow0 = row0 + (wave % (NW / VSPLIT)) / KSPLIT * 32;  // first local row of this wave
    const int qrow = wrow0 + l32;        // this lane's query row (local to the sequence)
    const int klo = clampk((int64_t)qrow + shift - a.wl, 0, Lk);       // this row's visible keys
    const int khi = clampk((int64_t)qrow + shift + a.wr, -1, Lk - 1);  // (empty when khi < klo)
    // both bounds are non-decreasing in the row: the wave's last row has the largest lower
    // bound, its first row the smallest upper bound
    const int klo_w = clampk((int64_t)wrow0 + 31 + shift - a.wl, 0, Lk);
    const int khi_w = clampk((int64_t)wrow0 + shift + a.wr, -1, Lk - 1);
    float c = a.scale_log2;
    const unsigned qflip = c < 0.f ? 0x80008000u : 0u;  // negative scale: negate q, keep c > 0
    c = fabsf(c);
    bf16x8 qf[KS];
    if (qrow >= 0 && qrow < Lq) {
        const u32x4 *src = (const u32x4 *)(qp + (int64_t)qrow * a.sq.m + 8 * hh);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            u32x4 w = src[2 * s];
            w ^= u32x4{qflip, qflip, qflip, qflip};
            qf[s] = __builtin_bit_cast(bf16x8, w);
        }
    } else {
#pragma unroll
        for (int s = 0; s < KS; ++s) qf[s] = bf16x8{};
    }

    // ---- LDS read addresses (byte offsets inside a stage)
    int kaddr[KS];  // K: row kb*32 + l32 (kb adds 32 rows), chunk 2s + hh
#pragma unroll
    for (int s = 0; s < KS; ++s) kaddr[s] = l32 * KROWB + (((2 * s + hh) ^ swz<KD>(l32)) << 4);
    if constexpr (SSPLIT) {  // score halves: this wave reads K rows 32 vpart + l32
#pragma unroll
        for (int s = 0; s < KS; ++s) kaddr[s] += vpart * 32 * KROWB;
    }
    // V: lane i of 16-lane group G addresses key row 4*hh + i/4 (+ 8e + 16kt + 32kb) and
    // head-dim columns mb*32 + 16*(G&1) + 4*(i%4) .. +3.
    const int vrow = 4 * hh + ((lane & 15) >> 2);
    const int vcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    int vaddr[MB][2];  // [mb][e]; + (kb*32 + kt*16) rows keep the swizzle (rows shift by multiples of 16)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int row = vrow + 8 * e, col = vpart * VW + mb * 32 + vcol;
            vaddr[mb][e] = V_BASE + row * VROWB + ((((col >> 3) ^ swz<VD>(row))) << 4) + ((col & 4) << 1);
        }
    // score halves: V rows of this wave's 32 keys and of its partner's (32 rows keep the swizzle)
    int vown[SSPLIT ? MB : 1][2], vpar[SSPLIT ? MB : 1][2];
    if constexpr (SSPLIT) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                vown[mb][e] = vaddr[mb][e] + vpart * 32 * VROWB;
                vpar[mb][e] = vaddr[mb][e] + (1 - vpart) * 32 * VROWB;
            }
    }

    f32x16 o[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) o[i] = f32x16{};
    float m_ref = -INFINITY, l_run = 0.f;

    // Score-split tile (SSPLIT): this wave's 32 keys of the tile are keys kt0 + 32 vpart + ..., its
    // partner (wave ^ NW/2, the same 32 rows) has the other 32.  Both keep one reference maximum per
    // row: every change of it is decided from the maximum over both halves.  The fast path (no
    // rescale due, the same check as the whole-tile kernel) needs one exchange; when any wave of
    // the workgroup fails it or still has a row without a finite reference, every wave takes the
    // exact path (row maxima exchanged, then P).  Every barrier sits in workgroup-uniform control
    // flow: the decision is read from the LDS flags after a barrier, and waves whose rows see no key
    // of the tile still meet every barrier.
    auto step_halves = [&](int slot, int kt0, auto masked_tag) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(masked_tag)::value;
        const bool skip = MASKED && ((int64_t)kt0 + BN - 1 < (int64_t)wrow0 + shift - a.wl ||
                                     (int64_t)kt0 > (int64_t)wrow0 + 31 + shift + a.wr);
        const unsigned char LDS_AS *kst = (const unsigned char LDS_AS *)smem + slot * KTILE;  // + kaddr (own rows)
        const unsigned char LDS_AS *vst = (const unsigned char LDS_AS *)smem + slot * VTILE;
        const int partner = wave ^ (NW / 2);
        auto scores = [&](f32x16 &x) __attribute__((always_inline)) {
            x = f32x16{};
#pragma unroll
            for (int s = 0; s < KS; ++s)
                x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8 LDS_AS *)(kst + kaddr[s]), qf[s], x, 0, 0, 0);
            if (MASKED) {
                // element r holds key kt0 + 32 vpart + 4 hh + off(r)
                const int dlo = klo - kt0 - 32 * vpart - 4 * hh, dhi = khi - kt0 - 32 * vpart - 4 * hh;
                const bool cut_lo = kt0 < klo_w, cut_hi = kt0 + BN - 1 > khi_w;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int off = 8 * (r >> 2) + (r & 3);
                    if ((cut_lo && off < dlo) || (cut_hi && off > dhi)) x[r] = -INFINITY;
                }
            }
        };
        auto exponentials = [&](f32x16 &x, float m_use) __attribute__((always_inline)) {
#pragma unroll
            for (int r = 0; r < 16; ++r) x[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[r], c, -m_use));
            float ps[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) ps[i] = x[i] + x[i + 8];
#pragma unroll
            for (int w = 4; w >= 1; w >>= 1)
#pragma unroll
                for (int i = 0; i < w; ++i) ps[i] += ps[i + w];
            return ps[0];
        };
        bf16x8 pown[2];  // this wave's P half: B operands of its keys 32 vpart + 16 kt + ...
        auto put_p = [&](const f32x16 &x) __attribute__((always_inline)) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                for (int i = 0; i < 8; ++i) pown[kt][i] = (__bf16)x[8 * kt + i];
                *(bf16x8 LDS_AS *)(xp + ((wave * 2 + kt) * 64 + lane) * 16) = pown[kt];
            }
        };
        f32x16 x;
        float psum = 0.f;
        int need = 0;
        if (!skip) {
            scores(x);
            if (__builtin_amdgcn_ballot_w64(m_ref == -INFINITY)) {
                need = 1;
            } else {
                psum = exponentials(x, m_ref);
                if (__builtin_amdgcn_ballot_w64(!(psum <= kSumThreshold))) need = 1;
                else put_p(x);
            }
        }
        if (lane == 0) xf[wave] = need;
        lds_barrier();
        const i32x4 f0 = *(const i32x4 LDS_AS *)xf, f1 = *(const i32x4 LDS_AS *)(xf + 4);
        if ((f0[0] | f0[1] | f0[2] | f0[3] | f1[0] | f1[1] | f1[2] | f1[3]) != 0) {
            // exact path for the whole workgroup: scores again (K is still in LDS), row maxima of
            // both halves, one reference decision per row shared by the pair
            float mxh = -INFINITY;
            if (!skip) {
                __asm__ volatile("" ::: "memory");  // read K again rather than keep its fragments live
                scores(x);
                float m8[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) m8[i] = fmaxf(x[i], x[i + 8]);
#pragma unroll
                for (int w = 4; w >= 1; w >>= 1)
#pragma unroll
                    for (int i = 0; i < w; ++i) m8[i] = fmaxf(m8[i], m8[i + w]);
                mxh = pair_max(m8[0]);
                if (hh == 0) xm[wave * 32 + l32] = mxh;
            }
            lds_barrier();
            if (!skip) {
                const float mx = fmaxf(mxh, xm[partner * 32 + l32]) * c;
                const bool up = mx > m_ref + kRescaleThreshold;
                if (__builtin_amdgcn_ballot_w64(up)) {
                    const float alpha = up ? __builtin_amdgcn_exp2f(m_ref - mx) : 1.f;
                    m_ref = up ? mx : m_ref;
                    l_run *= alpha;
#pragma unroll
                    for (int i = 0; i < MB; ++i)
#pragma unroll
                        for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
                }
                psum = exponentials(x, (m_ref == -INFINITY) ? 0.f : m_ref);
                put_p(x);
            }
            lds_barrier();
        }
        if (skip) return;
        l_run += psum;
        // O^T += V^T P^T: this wave's 32 keys, then its partner's (V rows from vown / vpar)
#pragma unroll
        for (int side = 0; side < 2; ++side)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                const bf16x8 pk = side == 0 ? pown[kt]
                                            : *(const bf16x8 LDS_AS *)(xp + ((partner * 2 + kt) * 64 + lane) * 16);
                const int roff = kt * 16 * VROWB;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const int a0 = (side == 0 ? vown[mb][0] : vpar[mb][0]) + roff;
                    const int a1 = (side == 0 ? vown[mb][1] : vpar[mb][1]) + roff;
                    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 LDS_AS *)(vst + a0));
                    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 LDS_AS *)(vst + a1));
                    const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                    o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pk, o[mb], 0, 0, 0);
                }
            }
    };

    // One 64-key tile at loop position p: S^T, mask (MASKED only), online softmax, O^T update.
    // STAGE_C >= 0 names the LDS stage at compile time (p % STAGES == STAGE_C), so every LDS
    // offset becomes an instruction immediate; -1 computes it at run time.
    auto step = [&](int p, int t, auto masked_tag, auto stage_tag) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(masked_tag)::value;
        constexpr int STAGE_C = decltype(stage_tag)::value;
        const int slot = STAGE_C >= 0 ? STAGE_C : p % STAGES;
        const int kt0 = t * BN;
        if (PAIRS) {
            // even position of a pair: both tiles of the pair are in, and the two slots of the
            // previous pair, which every wave has finished, take the next pair
            if (((STAGE_C >= 0 ? STAGE_C : p) & 1) == 0) {
                wait_barrier<0>();
                if (p + 2 < nt) issue(p + 2);
                if (p + 3 < nt) issue(p + 3);
            }
        } else if (STAGES == 2) {
            // double buffer: tile p is in and every wave is past tile p - 1, whose slot takes p + 1
            wait_barrier<0>();
            if (p + 1 < nt) issue(p + 1);
        } else {
            if (p + 1 < nt) wait_barrier<KROUNDS + VROUNDS>();
            else wait_barrier<0>();
            if (p + 2 < nt) issue(p + 2);
        }
        if constexpr (SSPLIT) {
            step_halves(slot, kt0, masked_tag);
            return;
        }
        // split keys: the other wave of the block takes this tile
        if (KSPLIT > 1 && ((STAGE_C >= 0 ? STAGE_C : p) & 1) != wsub) return;
        // the whole tile lies before or after every window of this wave's 32 rows
        if (MASKED && ((int64_t)kt0 + BN - 1 < (int64_t)wrow0 + shift - a.wl ||
                       (int64_t)kt0 > (int64_t)wrow0 + 31 + shift + a.wr))
            return;
        const unsigned char LDS_AS *kst = (const unsigned char LDS_AS *)smem + slot * KTILE;  // K tile
        const unsigned char LDS_AS *vst = (const unsigned char LDS_AS *)smem + slot * VTILE;  // + vaddr (from V_BASE)

        // S^T = K Q^T for two 32-key blocks, masked on edge tiles
        auto scores = [&](f32x16 &sa, f32x16 &sb) __attribute__((always_inline)) {
            sa = f32x16{}; sb = f32x16{};
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const bf16x8 k0 = *(const bf16x8 LDS_AS *)(kst + kaddr[s]);
                const bf16x8 k1 = *(const bf16x8 LDS_AS *)(kst + kaddr[s] + 32 * KROWB);
                sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[s], sa, 0, 0, 0);
                sb = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[s], sb, 0, 0, 0);
            }
            if (MASKED) {
                // element r of sa holds key kt0 + 4 hh + off(r), of sb 32 keys later; only the bounds
                // that cut this tile for some row of the wave are tested
                const int dlo = klo - kt0 - 4 * hh, dhi = khi - kt0 - 4 * hh;
                const bool cut_lo = kt0 < klo_w, cut_hi = kt0 + BN - 1 > khi_w;
                if (cut_lo && cut_hi) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int off = 8 * (r >> 2) + (r & 3);
                        if (off < dlo || off > dhi) sa[r] = -INFINITY;
                        if (off + 32 < dlo || off + 32 > dhi) sb[r] = -INFINITY;
                    }
                } else if (cut_hi) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int off = 8 * (r >> 2) + (r & 3);
                        if (off > dhi) sa[r] = -INFINITY;
                        if (off + 32 > dhi) sb[r] = -INFINITY;
                    }
                } else if (cut_lo) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int off = 8 * (r >> 2) + (r & 3);
                        if (off < dlo) sa[r] = -INFINITY;
                        if (off + 32 < dlo) sb[r] = -INFINITY;
                    }
                }
            }
        };
        f32x16 sa, sb;
        scores(sa, sb);
        float psum;
        // Fast path once every row of the wave has a finite reference: exponentials first, then
        // the partial row sums decide whether any value exceeded 2^8 (the exponentials overwrite
        // the scores, so a failing tile computes them again and takes the exact path)
        auto exponentials = [&](float m_use) __attribute__((always_inline)) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                sa[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[r], c, -m_use));
                sb[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sb[r], c, -m_use));
            }
            float ps[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) ps[i] = sa[i] + sb[i];
#pragma unroll
            for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
                for (int i = 0; i < w; ++i) ps[i] += ps[i + w];
            return ps[0];
        };
        bool exact = __builtin_amdgcn_ballot_w64(m_ref == -INFINITY) != 0;
        if (!exact) {
            psum = exponentials(m_ref);
            if (__builtin_amdgcn_ballot_w64(!(psum <= kSumThreshold))) {
                exact = true;
                __asm__ volatile("" ::: "memory");  // read K again rather than keep its fragments live
                scores(sa, sb);
            }
        }
        if (exact) {
            // row maximum of the raw scores (c > 0), pairwise to keep dependency chains short
            float m8[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                m8[i] = fmaxf(fmaxf(sa[2 * i], sa[2 * i + 1]), fmaxf(sb[2 * i], sb[2 * i + 1]));
#pragma unroll
            for (int w = 4; w >= 1; w >>= 1)
#pragma unroll
                for (int i = 0; i < w; ++i) m8[i] = fmaxf(m8[i], m8[i + w]);
            const float mx = pair_max(m8[0]) * c;
            // raise the reference only when the row max grows by more than the threshold
            const bool up = mx > m_ref + kRescaleThreshold;
            if (__builtin_amdgcn_ballot_w64(up)) {
                // lanes that keep their reference scale by exactly 1 (m_ref may still be -inf there)
                const float alpha = up ? __builtin_amdgcn_exp2f(m_ref - mx) : 1.f;
                m_ref = up ? mx : m_ref;
                l_run *= alpha;
#pragma unroll
                for (int i = 0; i < MB; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
            }
            psum = exponentials((m_ref == -INFINITY) ? 0.f : m_ref);
        }
        bf16x8 pb[4];  // [kb*2 + kt]: keys 32kb + 16kt + {8*(i/4) + 4*hh + i%4}
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < 8; ++i) pb[j][i] = (__bf16)(j < 2 ? sa[8 * j + i] : sb[8 * (j - 2) + i]);
        l_run += psum;

        // O^T += V^T P^T over 4 steps of 16 keys
#pragma unroll
        for (int ksi = 0; ksi < 4; ++ksi) {
            const int roff = ksi * 16 * VROWB;  // kb*32 + kt*16 rows
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 LDS_AS *)(vst + vaddr[mb][0] + roff));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 LDS_AS *)(vst + vaddr[mb][1] + roff));
                const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[ksi], o[mb], 0, 0, 0);
            }
        }
    };

    if (nt > 0) issue(0);
    if (STAGES > 2 && nt > 1) issue(1);
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    using S3 = std::integral_constant<int, 3>;
    using SR = std::integral_constant<int, -1>;
    // The tiles [t, tend) of one unwrapped piece of the order, by class: the left edge of the
    // windows (masked), inner tiles (unmasked, unrolled by the ring's slots), then the diagonal,
    // right edge and key tail (masked).  The order is [t_first, te) then [tb, t_first).
    int p = 0;
    auto run = [&](int t, const int tend) __attribute__((always_inline)) {
        for (const int le = min(tend, ua); t < le; ++p, ++t) step(p, t, std::true_type{}, SR{});
        const int ie = min(tend, ub);
        for (; t < ie && p % STAGES != 0; ++p, ++t) step(p, t, std::false_type{}, SR{});
        for (; t + STAGES <= ie; p += STAGES, t += STAGES) {
            step(p, t, std::false_type{}, S0{});
            step(p + 1, t + 1, std::false_type{}, S1{});
            if constexpr (STAGES >= 3) step(p + 2, t + 2, std::false_type{}, S2{});
            if constexpr (STAGES == 4) step(p + 3, t + 3, std::false_type{}, S3{});
        }
        for (; t < ie; ++p, ++t) step(p, t, std::false_type{}, SR{});
        for (; t < tend; ++p, ++t) step(p, t, std::true_type{}, SR{});
    };
    run(t_first, te);
    run(tb, t_first);

    if constexpr (KSPLIT == 2) {
        // exact merge of the two waves' states of a block: the second wave leaves its (o, m, l)
        // in LDS (the ring is free once both waves are past the loop), the first rescales both
        // to the larger reference and adds them
        constexpr int REC = MB * 16 + 2;
        float *rec = (float *)smem + ((wave / 2) * 64 + lane) * REC;
        __syncthreads();
        if (wsub == 1) {
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) rec[16 * i + r] = o[i][r];
            rec[MB * 16] = m_ref;
            rec[MB * 16 + 1] = l_run;
        }
        __syncthreads();
        if (wsub == 1) return;
        const float m2 = rec[MB * 16], l2 = rec[MB * 16 + 1];
        const float mm = fmaxf(m_ref, m2);
        const float mu = mm == -INFINITY ? 0.f : mm;
        const float a1 = __builtin_amdgcn_exp2f(m_ref - mu), a2 = __builtin_amdgcn_exp2f(m2 - mu);
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[i][r] = o[i][r] * a1 + rec[16 * i + r] * a2;
        l_run = l_run * a1 + l2 * a2;
        m_ref = mm;
    }

    // ---- normalise and store
    float l_tot = pair_sum(l_run);
    if constexpr (SSPLIT) {
        // the pair's halves of each row sum (the same reference maximum): every wave meets this
        // barrier after its last tile
        if (hh == 0) xm[wave * 32 + l32] = l_tot;
        lds_barrier();
        l_tot += xm[(wave ^ (NW / 2)) * 32 + l32];
    }
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    unsigned char *const obase_p = (unsigned char *)a.o + split * a.o_split * (OUT_F32 ? 4 : 2);
    float *const lse_p = a.lse ? a.lse + split * a.lse_split : nullptr;
    if constexpr (!OUT_F32 && KSPLIT == 1) {
        // bf16 rows go out whole, staged in the now idle ring (16-byte stores, whole rows, instead
        // of 8 bytes per lane at 32 rows 8 KB apart)
        __syncthreads();  // every wave has finished reading the K/V ring
        store_rows_bf16<VW>(o, inv, (unsigned char LDS_AS *)smem + wave * 32 * VW * 2, obase_p,
                            (int64_t)b * a.so.b + head_offset(a.so, hf, a.Hin) + (int64_t)(qs + wrow0) * a.so.m +
                                vpart * VW,
                            a.so.m, Lq - wrow0, -wrow0);
        if (qrow >= 0 && qrow < Lq && lse_p && hh == 0 && vpart == 0)
            lse_p[((int64_t)b * a.Htot + hf) * a.Mq + qs + qrow] =
                l_tot > 0.f ? (m_ref + __log2f(l_tot)) * kLn2 : -INFINITY;
    } else if (qrow >= 0 && qrow < Lq) {
        unsigned char *op = obase_p;
        const int64_t obase = (int64_t)b * a.so.b + head_offset(a.so, hf, a.Hin) + (int64_t)(qs + qrow) * a.so.m;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = vpart * VW + mb * 32 + 8 * g + 4 * hh;
                const float x0 = o[mb][4 * g] * inv, x1 = o[mb][4 * g + 1] * inv;
                const float x2 = o[mb][4 * g + 2] * inv, x3 = o[mb][4 * g + 3] * inv;
                if (OUT_F32) {
                    *(f32x4 *)(op + (obase + d0) * 4) = f32x4{x0, x1, x2, x3};
                } else {
                    *(bf16x4 *)(op + (obase + d0) * 2) = bf16x4{(__bf16)x0, (__bf16)x1, (__bf16)x2, (__bf16)x3};
                }
            }
        }
        if (lse_p && hh == 0 && vpart == 0) {
            lse_p[((int64_t)b * a.Htot + hf) * a.Mq + qs + qrow] =
                l_tot > 0.f ? (m_ref + __log2f(l_tot)) * kLn2 : -INFINITY;
        }
    }
}

template <int KD, int VD, int NW, int STAGES, bool OUT_F32, bool PAGED>
__global__ __launch_bounds__(NW * 64) void fwd_bf16_kernel(FwdArgs a) {
    fwd_bf16_body<KD, VD, NW, STAGES, OUT_F32, 1, PAGED>(a);
}

// two waves per 32-row block, splitting its keys (paired ring)
template <int KD, int VD, bool OUT_F32, bool PAGED>
__global__ __launch_bounds__(128) void fwd_bf16_split_kernel(FwdArgs a) {
    fwd_bf16_body<KD, VD, 2, 4, OUT_F32, 2, PAGED>(a);
}

// 8 waves, two per 32-row block, each keeping half of the value columns (head dim 256)
template <int KD, int VD, bool OUT_F32, bool PAGED>
__global__ __launch_bounds__(512) void fwd_bf16_vsplit_kernel(FwdArgs a) {
    fwd_bf16_body<KD, VD, 8, 2, OUT_F32, 1, PAGED, 2>(a);
}

template <int KD, int VD, bool OUT_F32, bool PAGED>
hipError_t launch_vsplit(const FwdArgs &a, hipStream_t stream) {
    const int64_t grid = (a.max_seqlen_q + 127) / 128 * a.nseq * (int64_t)a.B * a.Htot * a.splits;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((fwd_bf16_vsplit_kernel<KD, VD, OUT_F32, PAGED>), dim3((unsigned)grid), dim3(512), 0, stream, a);
    return hipGetLastError();
}

template <int KD, int VD, int NW, int STAGES, bool OUT_F32, bool PAGED, int KSPLIT = 1>
hipError_t launch(const FwdArgs &a, hipStream_t stream) {
    constexpr int BM = NW / KSPLIT * 32;
    const int64_t tiles = (a.max_seqlen_q + BM - 1) / BM;
    const int64_t grid = tiles * a.nseq * (int64_t)a.B * a.Htot * a.splits;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    if constexpr (KSPLIT == 2)
        hipLaunchKernelGGL((fwd_bf16_split_kernel<KD, VD, OUT_F32, PAGED>), dim3((unsigned)grid), dim3(NW * 64), 0, stream,
                           a);
    else
        hipLaunchKernelGGL((fwd_bf16_kernel<KD, VD, NW, STAGES, OUT_F32, PAGED>), dim3((unsigned)grid), dim3(NW * 64), 0,
                           stream, a);
    return hipGetLastError();
}


// 8 waves (256 query rows) per workgroup, one workgroup per CU, a 4-slot K/V ring (128 KB of
// LDS for head dim 128) filled two tiles at a time, so that the waves meet at a barrier once
// per 128 keys (4% faster than a 3-stage ring with a barrier per tile).  Measured on MI355X
// against two 4-wave workgroups per CU with a 2-stage ring (30% slower) and against
// staggered two-group schedules (no faster).  Problems too small to give every CU a workgroup (few heads, short query
// ranges) take workgroups of 4 or 2 waves instead, so that more CUs share the work; below that,
// two waves share each 32-row block and split its keys between them.
#ifndef FWD_MIN_GRID
#define FWD_MIN_GRID 256
#endif
template <int KD, int VD, bool OUT_F32, bool PAGED>
hipError_t launch_nw(const FwdArgs &a, hipStream_t stream) {
    const int64_t units = (int64_t)a.nseq * a.B * a.Htot * a.splits;
    auto grid = [&](int bm) { return (a.max_seqlen_q + bm - 1) / bm * units; };
    if constexpr (VD == 256) {
        // 512-byte V rows and a 256-column O^T: a double-buffered ring (128 KB); 8 waves, two per
        // 32-row block splitting the value columns (both compute the scores), so that two waves
        // share each SIMD; on small grids 2 waves holding all 256 columns (one wave per SIMD)
        if (grid(128) >= FWD_MIN_GRID) return launch_vsplit<KD, VD, OUT_F32, PAGED>(a, stream);
        return launch<KD, VD, 2, 2, OUT_F32, PAGED>(a, stream);
    } else if constexpr (KD == 256) {
        // 512-byte K rows: a 3-slot ring (144 KB with 256-byte V rows) fits the LDS, a 4-slot one
        // does not, so every size keeps one barrier per tile (and no split-key form)
        if (grid(256) >= FWD_MIN_GRID) return launch<KD, VD, 8, 3, OUT_F32, PAGED>(a, stream);
        if (grid(128) >= FWD_MIN_GRID) return launch<KD, VD, 4, 3, OUT_F32, PAGED>(a, stream);
        return launch<KD, VD, 2, 3, OUT_F32, PAGED>(a, stream);
    } else {
    if (grid(256) >= FWD_MIN_GRID) return launch<KD, VD, 8, 4, OUT_F32, PAGED>(a, stream);
    if (grid(128) >= FWD_MIN_GRID) return launch<KD, VD, 4, 3, OUT_F32, PAGED>(a, stream);
    if (grid(64) >= FWD_MIN_GRID) return launch<KD, VD, 2, 3, OUT_F32, PAGED>(a, stream);
    // fewer than FWD_MIN_GRID blocks of 32 rows: two waves split each block's keys
    return launch<KD, VD, 2, 4, OUT_F32, PAGED, 2>(a, stream);
    }
}

template <int KD, int VD, bool PAGED>
hipError_t launch_out(const FwdArgs &a, bool out_f32, hipStream_t stream) {
    return out_f32 ? launch_nw<KD, VD, true, PAGED>(a, stream) : launch_nw<KD, VD, false, PAGED>(a, stream);
}

}  // namespace
}  // namespace attn
