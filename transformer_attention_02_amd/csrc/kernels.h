// Internal interface between the C-ABI front end (api.cpp) and the HIP kernels.
// Every struct is passed to a kernel by value.  Strides are in elements; a head
// index hf in [0, Htot) is split as (hf / Hin, hf % Hin) and addressed through
// (sg, sh), which covers [B,M,H,D] (sg unused) and [B,M,G,H,D] with any strides,
// including 0 for an explicitly expanded K/V head axis.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

struct Strides {
    int64_t b, m, g, h;
};

__host__ __device__ inline int64_t head_offset(const Strides &s, int hf, int Hin) {
    return (int64_t)(hf / Hin) * s.g + (int64_t)(hf % Hin) * s.h;
}

// "Unbounded" window extent; row/key indices stay below 2^31, so i + shift +- kWinInf
// is evaluated in 64-bit arithmetic.
constexpr int kWinInf = 1 << 30;

// Forward / partial attention over one key range per (batch, head).
struct FwdArgs {
    const void *q, *k, *v;
    void *o;
    float *lse;          // [B, Htot, Mlse] or null
    Strides sq, sk, sv, so;
    int B, Mq, Mkv, Htot, Hin, K, Kv;
    float scale_log2;    // scale * log2(e): scores are kept in base-2 units
    // Visible keys of local row i in a sequence of Lq rows and Lk keys:
    //   [i + shift - wl, i + shift + wr] intersected with [0, Lk),
    //   shift = bottom_right ? Lk - Lq : 0; kWinInf = unbounded.
    int packed;          // per-sequence blocks from seqstart_q / seqstart_k
    int bottom_right;
    int wl, wr;
    const int32_t *seqstart_q, *seqstart_k;  // device prefix sums, packed sequences only
    int nseq;            // 1 when not packed
    int max_seqlen_q;    // rows covered per sequence (Mq when not packed)
    // > 0: the K/V rows of a head depend only on its group hf / Hin (an explicitly expanded GQA
    // head axis); the kernels then order heads so that the kv_groups = Htot / Hin groups each land
    // on one XCD, whose L2 serves the group's K/V to all of its heads
    int kv_groups;
    // KV cache (packed query blocks against per-sequence keys), bf16 only; seqlens_k null otherwise.
    // Sequence s holds keys 0 .. seqlens_k[s] - 1 (clamped to [0, cap]): rows of its lane
    // k + s * sk.b (block_tables null), or rows block_tables[s][j / page_size] * page_size +
    // j % page_size of the cache k (page numbers clamped to [0, num_pages)).
    const int32_t *seqlens_k;
    const int32_t *block_tables;  // [nseq, bt_stride]
    int bt_stride, page_size, num_pages, cap;
    // keys cut into `splits` chunks of `chunk` keys (a multiple of the 64-key tile): chunk c of a
    // query block writes its fp32 partial output at o + c * o_split and its LSE at lse + c * lse_split
    int splits, chunk;
    int64_t o_split, lse_split;
};

// Split-KV decode partials: one query row per (batch, head), keys cut in S chunks.
struct DecodeArgs {
    const void *q, *k, *v;
    Strides sq, sk, sv;
    int B, Mkv, Htot, Hin, D;
    int S, chunk;        // chunk = ceil(Mkv / S)
    float scale_log2;
    float *ws_o;         // [S, B, Htot, D] fp32, normalised per chunk
    float *ws_lse;       // [S, B, Htot] fp32, natural log
    // Per-sequence key counts (padded lanes or pages), both device arrays; null = Mkv keys each.
    const int32_t *seqlens;       // [B], clamped to [0, cap]
    const int32_t *block_tables;  // [B, bt_stride] page numbers, or null (lanes [B, cap, ...])
    int bt_stride, page_size, num_pages, cap;
    int window;  // > 0: the query sees only its sequence's last `window` keys; chunks cover those
    // FP8 / INT4 caches only: (scale, shift) fp16 pairs per cache row, head and group of
    // `group` consecutive elements (a multiple of 16 or 32 dividing D); strides in fp16 units.
    // MXFP8: one E8M0 byte per row, head and block of 32; strides in bytes
    const void *kss, *vss;
    Strides skss, svss;
    int group;
    int ss32;      // FP8 / INT4: (scale, shift) pairs of two fp32 (8 bytes) instead of two fp16
    int log2_hpw;  // heads per workgroup = 1 << log2_hpw (set by the launcher)
    int lane32;    // every lane's offset from its workgroup's first head and row fits 32 bits (set by the launcher)
};

// Element type of a decode K/V cache (q is bf16 for the quantised caches, else the cache's type).
// INT4: two unsigned 4-bit codes per byte, element 2i in the low nibble of byte i.
// MXFP8: E4M3 codes with one E8M0 scale byte per block of 32 elements (group = 32, no shift).
enum DecodeElem : int { DECODE_BF16 = 0, DECODE_F32 = 1, DECODE_FP8 = 2, DECODE_INT4 = 3, DECODE_MXFP8 = 4 };

constexpr int kMaxChunks = 128;

// Exact merge of S chunk results that share one layout.
struct MergeArgs {
    const void *chunk[kMaxChunks];
    const float *lse[kMaxChunks];  // each [B, Htot, M]
    Strides sc;                    // chunk strides
    void *o;
    Strides so;
    float *lse_out;                // [B, Htot, M] or null
    int S, B, M, Htot, Hin, Kv;
    int chunk_f32, out_f32;
};

// Launchers return a hipError_t from the launch.
hipError_t launch_fwd_bf16(const FwdArgs &a, bool out_f32, hipStream_t stream);
hipError_t launch_fwd_bf16_v256(const FwdArgs &a, bool out_f32, hipStream_t stream);  // value head dim 256
hipError_t launch_fwd_f32(const FwdArgs &a, hipStream_t stream);
// Backward of the forward above: dq, dk, dv from dout, out and lse (same masks and layouts).
struct BwdArgs {
    const void *q, *k, *v, *o, *dout;
    void *dq, *dk, *dv;
    Strides sq, sk, sv, so, sdo, sdq, sdk, sdv;
    const float *lse;     // [B, Htot, Mq], natural log
    float *ws_d, *ws_l2;  // [B, Htot, Mq] each: dout.out per row, and lse * log2(e) (+inf for empty rows)
    int B, Mq, Mkv, Htot, Hin, D, Dv;  // D: q/k head dim, Dv: v/out head dim
    float scale, scale_log2;
    int packed, bottom_right, wl, wr;
    const int32_t *seqstart_q, *seqstart_k;
    int nseq, max_seqlen_q, max_seqlen_k;
    // bf16, one sequence: dS^T kept in bf16, [B * Htot][ds_rows][ds_pitch] (key-major rows of
    // ds_pitch query columns); NULL: dQ recomputes S and dP in its own launch
    void *ds;
    int64_t ds_pitch, ds_rows;
};

hipError_t launch_bwd_bf16(const BwdArgs &a, hipStream_t stream);
hipError_t launch_bwd_f32(const BwdArgs &a, hipStream_t stream);

hipError_t launch_decode_partials(const DecodeArgs &a, int elem, hipStream_t stream);
hipError_t launch_merge(const MergeArgs &a, hipStream_t stream);

}  // namespace attn
