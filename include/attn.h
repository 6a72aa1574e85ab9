/*
 * attn.h -- C ABI of a fused attention forward library for AMD MI355X (gfx950).
 *
 * Operations follow the MSLK pages ("MSLK - complete kernel reference for LLM
 * agents", section "Attention - Core fMHA", and "MSLK Kernel Library --
 * Complete Reference", sections Quick start, Conventions and Glossary):
 *
 *   attn_fwd            memory_efficient_attention_forward_requires_grad:
 *                       scaled Q K^T, an optional mask, softmax, product with
 *                       V, without materialising the attention matrix; returns
 *                       the output and the per-row log-sum-exp (LSE).
 *                       With lse == NULL it is memory_efficient_attention_forward.
 *   attn_partial        memory_efficient_attention_partial: the same over one
 *                       disjoint K/V shard, output kept in fp32 for merging.
 *   attn_merge          merge_attentions: exact LSE-weighted combination of
 *                       shard results (not an average).
 *   attn_decode_splitkv split-KV decode (Glossary, "split-K / split-KV"): one
 *                       query row per (batch, head); the keys are cut into
 *                       equal contiguous chunks, each chunk's partial result
 *                       goes to a caller-owned fp32 workspace, and a second
 *                       pass merges them.
 *
 *   Further entry points, each documented at its declaration below:
 *   attn_fwd_ex / attn_partial_ex (bottom-right and sliding-window masks),
 *   attn_fwd_kvcache (packed query blocks against padded or paged KV caches),
 *   attn_decode_splitkv_noalloc (the decode with library-held scratch, no workspace),
 *   attn_decode_num_splits (a split count for a decode shape),
 *   attn_decode_splitkv_paged (padded lanes or a paged KV cache),
 *   attn_decode_splitkv_fp8 / attn_decode_splitkv_int4 (quantised KV caches) and
 *   attn_bwd (gradients from the forward's output and LSE; with a larger workspace,
 *   attn_bwd_ds_workspace_bytes, it keeps dS instead of recomputing it).
 *
 * Conventions shared by every call
 *   - Tensors are described by attn_tensor: a device pointer, a dtype, 4 dims
 *     [B, M, H, D] or 5 dims [B, M, G, H, D] (grouped heads, flattened to
 *     H_total = G*H with flat head g*H + h), and strides in ELEMENTS.  The last
 *     dim must have stride 1 and the row start of every (b, m, head) must be
 *     16-byte aligned; other strides are free, including 0 (an explicitly
 *     expanded K/V head axis for GQA/MQA, "Conventions" and "Sharp edges:
 *     GQA broadcasting is explicit").  Tensors a call writes (out, the
 *     gradients) take no stride 0 on an axis of extent > 1.
 *   - out has q's layout with the last dim replaced by V's head dim.
 *   - lse is fp32, contiguous [B, H_total, Mq]; packed sequences use
 *     [1, H_total, M_total] indexed by packed row.  LSE is the natural log
 *     of sum_j exp(s_ij) over the visible keys of the SCALED scores s.
 *   - A row with no visible key gets out = 0 and lse = -inf.
 *   - scale: a NaN means 1/sqrt(K).
 *   - Ownership: the caller allocates and owns every buffer (inputs, outputs,
 *     lse, workspace, sequence offsets).  The library allocates nothing and
 *     never synchronises; calls enqueue on `stream` and return.  Results are
 *     ready once the stream has drained.
 *   - Errors: a non-zero status means nothing was launched and nothing was
 *     written; attn_last_error() gives the reason (thread-local).
 *     ATTN_ERR_INVALID_ARGUMENT: inconsistent shapes, dtypes, strides,
 *       alignment, null pointers, bad counts.
 *     ATTN_ERR_UNSUPPORTED: a valid request the library has no kernel for.
 *     ATTN_ERR_WORKSPACE_TOO_SMALL: workspace_bytes below the requirement.
 *     ATTN_ERR_LAUNCH: the HIP runtime refused the launch.
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *attn_stream_t; /* a hipStream_t; NULL = the null stream */

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_INVALID_ARGUMENT = 1,
    ATTN_ERR_UNSUPPORTED = 2,
    ATTN_ERR_WORKSPACE_TOO_SMALL = 3,
    ATTN_ERR_LAUNCH = 4
} attn_status;

typedef enum {
    ATTN_DTYPE_F32 = 0,
    ATTN_DTYPE_BF16 = 1,
    ATTN_DTYPE_FP8_E4M3 = 2, /* OCP E4M3 ("FN": bias 7, no infinities, S.1111.111 = NaN); K/V caches of
                                attn_decode_splitkv_fp8 only */
    ATTN_DTYPE_F16 = 3,      /* IEEE half; the scale/shift metadata of the quantised decodes only */
    ATTN_DTYPE_INT4X2 = 4,   /* two unsigned 4-bit codes per byte, element 2i in the low nibble of byte i;
                                shape and strides of such a tensor count bytes (last dim = D / 2);
                                K/V caches of attn_decode_splitkv_int4 only */
    ATTN_DTYPE_E8M0 = 5      /* one byte e per block: the scale 2^(e - 127), e = 255 NaN (the MX formats'
                                shared exponent); block scales of attn_decode_splitkv_mxfp8 only */
} attn_dtype;

/* Masks ("Attention - Biases & masks" on the kernel reference page).  For a
 * (sequence of) Lq query rows and Lk keys, with local row i and local key j, the
 * visible keys are those with  -wl <= j - i - shift <= wr,  where shift = Lk - Lq
 * for the bottom-right kinds (the diagonal ends in the last key) and 0 otherwise.
 * The BLOCKDIAG kinds apply this inside every packed sequence (attn_varlen). */
typedef enum {
    ATTN_MASK_NONE = 0,
    ATTN_MASK_CAUSAL = 1,            /* LowerTriangularMask: top-left aligned, key j visible iff j <= i */
    ATTN_MASK_BLOCKDIAG = 2,         /* BlockDiagonalMask: a query row sees its own packed sequence */
    ATTN_MASK_BLOCKDIAG_CAUSAL = 3,  /* BlockDiagonalCausalMask: top-left causal inside every block */
    ATTN_MASK_CAUSAL_BOTTOMRIGHT = 4,            /* LowerTriangularFromBottomRightMask: j <= i + Lk - Lq */
    ATTN_MASK_BLOCKDIAG_CAUSAL_BOTTOMRIGHT = 5,  /* BlockDiagonalCausalFromBottomRightMask (per block);
                                                    a block with fewer keys than queries leaves its
                                                    first Lq - Lk rows empty */
    ATTN_MASK_LOCAL_BOTTOMRIGHT = 6,             /* LocalAttentionFromBottomRightMask(window_left,
                                                    window_right): wl = window_left, wr = window_right */
    ATTN_MASK_CAUSAL_LOCAL_BOTTOMRIGHT = 7,      /* LowerTriangularFromBottomRightLocalAttentionMask(
                                                    window_size): the window_size keys ending at the
                                                    diagonal (wl = window_size - 1, wr = 0) */
    ATTN_MASK_BLOCKDIAG_CAUSAL_LOCAL = 8,        /* BlockDiagonalCausalLocalAttentionMask(window_size):
                                                    top-left, per block */
    ATTN_MASK_BLOCKDIAG_CAUSAL_LOCAL_BOTTOMRIGHT = 9  /* BlockDiagonalCausalLocalAttentionFromBottomRightMask */
} attn_mask_kind;

/* A mask with its window parameters (kinds 6-9 need them; 0-5 ignore them).
 * window_size >= 1 for kinds 7-9; window_left, window_right >= 0 for kind 6. */
typedef struct {
    int32_t kind;
    int32_t window_size;
    int32_t window_left;
    int32_t window_right;
} attn_mask;

typedef struct {
    void *data;        /* device pointer */
    int32_t dtype;     /* attn_dtype */
    int32_t ndim;      /* 4: [B, M, H, D]; 5: [B, M, G, H, D] */
    int64_t shape[5];
    int64_t stride[5]; /* in elements */
} attn_tensor;

/* Packed variable-length sequences ("Glossary: varlen"; BlockDiagonalMask.from_seqlens).
 * Required for the BLOCKDIAG masks, ignored otherwise.  B must be 1.
 * seqstart_q/seqstart_k are DEVICE int32 prefix sums [nseq + 1]: 0, L0, L0+L1,
 * ..., M_total.  seqstart_k NULL means seqstart_k = seqstart_q.
 * max_seqlen_q must be >= every query length; max_seqlen_k, read by attn_bwd only,
 * >= every key length, or <= 0 when not known (Mkv is then assumed).  The offsets
 * live on the device and are not read by the host: offsets that are not monotone,
 * do not start at 0, or exceed max_seqlen_q / max_seqlen_k give unspecified output
 * values but never an out-of-bounds access (the kernels clamp them to [0, M]).
 * Rows outside every sequence are not written. */
typedef struct {
    const int32_t *seqstart_q;
    const int32_t *seqstart_k;
    int32_t nseq;
    int32_t max_seqlen_q;
    int32_t max_seqlen_k;
} attn_varlen;

/* memory_efficient_attention_forward_requires_grad ("Attention - Core fMHA").
 *   mask: an attn_mask_kind without window parameters (0-5); attn_fwd_ex takes any kind.
 *   q [B, Mq, (G,) H, K], k [B, Mkv, (G,) H, K], v [B, Mkv, (G,) H, Kv]; one dtype.
 *   out [B, Mq, (G,) H, Kv] with q's dtype.
 *   lse fp32 [B, H_total, Mq] device buffer, or NULL to skip it.
 *   varlen: NULL unless mask is one of the block-diagonal kinds.
 * Built kernels: bf16 with K and Kv each in {64, 128, 256} (MFMA; ck_splitk.FwOp in "Attention -
 * Backend operators" takes head dims up to 256); fp32 with K, Kv <= 128. */
attn_status attn_fwd(const attn_tensor *q, const attn_tensor *k, const attn_tensor *v,
                     int32_t mask, const attn_varlen *varlen, float scale,
                     const attn_tensor *out, float *lse, attn_stream_t stream);

/* memory_efficient_attention_partial ("Attention - Core fMHA").
 * Same inputs as attn_fwd; k/v are the shard (the mask treats the shard as the
 * whole key sequence).  out may be fp32 (the default for merging) or q's dtype.
 * lse is required.  An empty shard (Mkv = 0) gives out = 0, lse = -inf. */
attn_status attn_partial(const attn_tensor *q, const attn_tensor *k, const attn_tensor *v,
                         int32_t mask, const attn_varlen *varlen, float scale,
                         const attn_tensor *out, float *lse, attn_stream_t stream);

/* attn_fwd / attn_partial with a full mask descriptor (any kind, including the
 * windowed ones).  Everything else as above. */
attn_status attn_fwd_ex(const attn_tensor *q, const attn_tensor *k, const attn_tensor *v,
                        const attn_mask *mask, const attn_varlen *varlen, float scale,
                        const attn_tensor *out, float *lse, attn_stream_t stream);
attn_status attn_partial_ex(const attn_tensor *q, const attn_tensor *k, const attn_tensor *v,
                            const attn_mask *mask, const attn_varlen *varlen, float scale,
                            const attn_tensor *out, float *lse, attn_stream_t stream);

/* merge_attentions ("Attention - Core fMHA"; "Exact softmax merge" in Quick start).
 *   n_chunks in [1, ATTN_MAX_CHUNKS]; out_chunks: n_chunks host descriptors
 *   [B, M, (G,) H, Kv] (fp32 or bf16, all with the same dtype and strides, e.g.
 *   views of one stacked tensor); lse_chunks: n_chunks device pointers, each
 *   fp32 contiguous [B, H_total, M].
 *   out [B, M, (G,) H, Kv] fp32 or bf16; lse_out fp32 [B, H_total, M] or NULL
 *   (merge_attentions' write_lse=False).
 *   L = M* + ln sum_c exp(lse_c - M*),  out = sum_c exp(lse_c - L) out_c;
 *   chunks at -inf weigh 0; if every chunk is -inf, out = 0 and lse = -inf. */
#define ATTN_MAX_CHUNKS 128
attn_status attn_merge(int32_t n_chunks, const attn_tensor *out_chunks,
                       const float *const *lse_chunks, const attn_tensor *out, float *lse_out,
                       attn_stream_t stream);

/* Bytes of device workspace attn_fwd_kvcache needs with num_splits >= 2 (fp32 partial outputs
 * [num_splits, Mq, H_total, Kv] and LSEs [num_splits, H_total, Mq], 256-byte aligned); 0 for 1. */
size_t attn_fwd_kvcache_workspace_bytes(int64_t Mq, int64_t H_total, int64_t Kv, int32_t num_splits);

/* Packed query blocks against a KV cache ("Attention - Biases & masks": BlockDiagonalPaddedKeysMask,
 * BlockDiagonalCausalWithOffsetPaddedKeysMask, BlockDiagonalLocalAttentionPaddedKeysMask,
 * BlockDiagonalCausalLocalAttentionPaddedKeysMask and their Paged... forms, "packed Q blocks attending
 * fixed-capacity padded K/V lanes" mapped to physical cache pages): chunked prefill and several
 * queries per sequence, e.g. speculative decoding.
 *   q [1, Mq, (G,) H, K] bf16: sequence s owns query rows seqstart_q[s] .. seqstart_q[s+1]-1
 *     (DEVICE int32 [nseq + 1] prefix sums; every block at most max_seqlen_q rows).
 *   seqlens_k: DEVICE int32 [nseq], keys held by each sequence (clamped to [0, cap]).
 *   seqstart_k non-NULL (gappy lanes: BlockDiagonalGappyKeysMask,
 *     BlockDiagonalCausalWithOffsetGappyKeysMask, BlockDiagonalLocalAttentionFromBottomRightGappyKeysMask,
 *     "K/V lanes with arbitrary starts and independently used lengths"): DEVICE int32 [nseq];
 *     k/v are one tensor [1, Mk, (G,) H, K/Kv] and sequence s owns its rows seqstart_k[s] ..
 *     seqstart_k[s] + seqlens_k[s] - 1 (clamped to [0, Mk]; lanes may overlap or leave gaps);
 *     block_tables must be NULL (the paged gappy form is not built); cap = Mk.
 *   block_tables NULL (and seqstart_k NULL): k/v are padded lanes [B >= nseq, cap, (G,) H, K/Kv];
 *     sequence s owns keys 0 .. seqlens_k[s]-1 of lane s.
 *   block_tables non-NULL: DEVICE int32 [nseq, max_blocks_per_seq] page numbers; k/v are the cache
 *     [1, num_pages * page_size, (G,) H, D] (K == Kv); key j of sequence s is cache row
 *     block_tables[s][j / page_size] * page_size + j % page_size; page_size a multiple of 64 and
 *     max_blocks_per_seq <= 8192 (cap = max_blocks_per_seq * page_size).
 *   mask: ATTN_MASK_NONE (all of the sequence's keys), ATTN_MASK_CAUSAL_BOTTOMRIGHT (the "with
 *     offset" causal form: the block's Lq queries are the sequence's last ones, query i sees keys
 *     j <= i + Lk - Lq), ATTN_MASK_LOCAL_BOTTOMRIGHT (window_left, window_right around that
 *     diagonal) or ATTN_MASK_CAUSAL_LOCAL_BOTTOMRIGHT (window_size); per sequence, with Lk =
 *     seqlens_k[s] and Lq its query count.  Rows that see no key get out = 0, lse = -inf.
 *   num_splits in [1, ATTN_MAX_CHUNKS]: the keys are cut into chunks of ceil(max_seqlen_k /
 *     num_splits) rounded up to 64 keys; with num_splits >= 2 the chunks' fp32 partial results go to
 *     `workspace` (device, 256-byte aligned, >= attn_fwd_kvcache_workspace_bytes) and a merge
 *     launch combines them (for few query blocks over long caches).
 *   out [1, Mq, (G,) H, Kv] bf16; lse fp32 [1, H_total, Mq] or NULL.  K, Kv in {64, 128, 256}
 *     (a paged cache: K == Kv).
 *   Device metadata is not read by the host; bad values give unspecified results, never an
 *   out-of-bounds access.  Errors as attn_fwd. */
attn_status attn_fwd_kvcache(const attn_tensor *q, const attn_tensor *k, const attn_tensor *v, const attn_mask *mask,
                             const int32_t *seqstart_q, int32_t nseq, int32_t max_seqlen_q, const int32_t *seqstart_k,
                             const int32_t *seqlens_k,
                             const int32_t *block_tables, int32_t max_blocks_per_seq, int32_t page_size,
                             int32_t max_seqlen_k, int32_t num_splits, float scale, void *workspace,
                             size_t workspace_bytes, const attn_tensor *out, float *lse, attn_stream_t stream);

/* Bytes of device workspace attn_bwd needs: two fp32 rows per query row and head
 * ([B, H_total, Mq] each, 256-byte aligned). */
size_t attn_bwd_workspace_bytes(int64_t B, int64_t H_total, int64_t Mq);

/* Bytes of device workspace with which the bf16 backward at head dim 128 of one sequence per
 * batch element (no block-diagonal mask) keeps dS instead of recomputing it:
 * attn_bwd_workspace_bytes(B, H_total, Mq) followed by a bf16 dS buffer of round_up(Mkv, 128) x
 * round_up(Mq, 256) elements per (batch, head).  SIZE_MAX when Mq exceeds 2^24 (that form then
 * never runs). */
size_t attn_bwd_ds_workspace_bytes(int64_t B, int64_t H_total, int64_t Mq, int64_t Mkv);

/* memory_efficient_attention_backward ("Attention - Core fMHA"): the gradients of the
 * forward for an upstream gradient, from the forward's output and LSE and the original
 * q, k, v (no dropout, no bias gradient).  With P_ij = exp(scale q_i.k_j - lse_i) on the
 * visible keys: dv_j = sum_i P_ij dout_i; dS_ij = P_ij (dout_i.v_j - dout_i.out_i);
 * dq_i = scale sum_j dS_ij k_j; dk_j = scale sum_i dS_ij q_i.
 *   q [B, Mq, (G,) H, K]; k [B, Mkv, (G,) H, K]; v [B, Mkv, (G,) H, Kv];
 *     dout, out [B, Mq, (G,) H, Kv]; one dtype: bf16 with K == Kv in {64, 128} (matrix
 *     cores) or fp32 with K, Kv <= 128; lse fp32 [B, H_total, Mq] as attn_fwd wrote it.
 *   mask, varlen, scale: exactly those of the forward call.
 *   dq, dk, dv: shapes of q, k, v, q's dtype, any strides that do not make two elements
 *     share memory (a stride-0 expanded head axis is rejected: for expanded GQA keys
 *     pass dk/dv of the expanded shape and sum over each group's heads).
 *   workspace: device, 256-byte aligned, >= attn_bwd_workspace_bytes(B, H_total, Mq).
 *   Two launches on `stream`: dQ (recomputing S and dP per key tile), then dK and dV.
 *   bf16 at head dim 128 without a block-diagonal mask and with workspace_bytes >=
 *   attn_bwd_ds_workspace_bytes(B, H_total, Mq, Mkv): three launches instead (each row's D and LSE; dK and dV, keeping dS in
 *   bf16 in the workspace; dQ = scale dS K), so S and dP are computed once.  Both forms round P and
 *   dS to bf16 before the products that use them.
 *   The two forms measured within a few percent of each other.
 *   Errors as attn_fwd; nothing is written on error. */
attn_status attn_bwd(const attn_tensor *dout, const attn_tensor *q, const attn_tensor *k,
                     const attn_tensor *v, const attn_tensor *out, const float *lse,
                     const attn_mask *mask, const attn_varlen *varlen, float scale, void *workspace,
                     size_t workspace_bytes, const attn_tensor *dq, const attn_tensor *dk,
                     const attn_tensor *dv, attn_stream_t stream);

/* A split count for the split-KV decodes (the pages' get_split_k(B, H, Mk) of ck_splitk.FwOp and
 * triton_splitk.FwOp): the smallest power of two S <= ATTN_MAX_CHUNKS with B * H_total * S at least
 * eight per compute unit of the current device, while chunks keep >= 256 keys (S = 1 for empty
 * shapes).  Measured on MI355X within a few percent of the best split over 1..128 for B*H_total
 * from 16 to 4096 and Mkv from 1 K to 128 K keys.  Host-only: reads the device's compute-unit
 * count once per device (256 when no device answers), enqueues nothing. */
int32_t attn_decode_num_splits(int64_t B, int64_t H_total, int64_t Mkv);

/* Bytes of device workspace attn_decode_splitkv needs (fp32 partial outputs
 * [num_splits, B, H_total, Kv] and LSEs [num_splits, B, H_total], 256-byte aligned). */
size_t attn_decode_workspace_bytes(int64_t B, int64_t H_total, int64_t Kv, int32_t num_splits);

/* Split-KV decode (Glossary "split-K / split-KV"; ck_splitk.FwOp_S* fixes the split count).
 *   q [B, 1, (G,) H, K], k/v [B, Mkv, (G,) H, K]; bf16 or fp32, K == Kv in {64, 128, 256}
 *   (ck_splitk.FwOp: head dims up to 256).
 *   num_splits in [1, ATTN_MAX_CHUNKS]: chunk s covers keys
 *   [s*c, min(Mkv, (s+1)*c)) with c = ceil(Mkv / num_splits); a chunk may be empty.
 *   workspace: device, 256-byte aligned, >= attn_decode_workspace_bytes(...).
 *   out [B, 1, (G,) H, Kv] with q's dtype; lse fp32 [B, H_total, 1] or NULL.
 *   Two launches on `stream`: per-chunk partials, then the merge. */
attn_status attn_decode_splitkv(const attn_tensor *q, const attn_tensor *k, const attn_tensor *v,
                                int32_t num_splits, float scale, void *workspace,
                                size_t workspace_bytes, const attn_tensor *out, float *lse,
                                attn_stream_t stream);

/* attn_decode_splitkv for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The per-chunk partials go to a
 * static device array of ATTN_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs
 * on until the process ends (its address is looked up once per device, on that device's first
 * call, with the device current: the stream must belong to the current device).  No allocation
 * of any kind happens in the call.
 *   Arguments, layouts, results and errors as attn_decode_splitkv, without the workspace.  A call
 *   whose attn_decode_workspace_bytes(B, H_total, Kv, num_splits) exceeds the scratch returns
 *   ATTN_ERR_UNSUPPORTED and launches nothing.
 *   Every call on one GPU shares that GPU's scratch: calls that may overlap on one GPU (other
 *   streams, other threads) race and must be ordered by the caller.  Each call writes every
 *   scratch entry it reads, so nothing needs clearing between calls. */
#define ATTN_NOALLOC_SCRATCH_BYTES (32u << 20)
attn_status attn_decode_splitkv_noalloc(const attn_tensor *q, const attn_tensor *k, const attn_tensor *v,
                                        int32_t num_splits, float scale, const attn_tensor *out, float *lse,
                                        attn_stream_t stream);

/* Split-KV decode against a KV cache ("Attention - Biases & masks": BlockDiagonalPaddedKeysMask
 * and PagedBlockDiagonalPaddedKeysMask, one query per sequence; "MSLK Kernel Library --
 * Complete Reference", Glossary "paged KV": cache rows addressed through a block table
 * and a fixed page size).
 *   q [B, 1, (G,) H, D]; seqlens: DEVICE int32 [B], keys held by each sequence.
 *   block_tables NULL: k/v are padded lanes [B, cap, (G,) H, D], sequence b owns keys
 *     0 .. seqlens[b]-1 of its lane (cap = k's row count).
 *   block_tables non-NULL: DEVICE int32 [B, max_blocks_per_seq] (row-major) of page
 *     numbers; k/v are the cache [1, num_pages * page_size, (G,) H, D]; key j of sequence
 *     b is cache row block_tables[b][j / page_size] * page_size + j % page_size
 *     (cap = max_blocks_per_seq * page_size).
 *   max_seqlen_k in [0, cap] bounds every seqlens[b]; the keys are cut into num_splits
 *     chunks of ceil(max_seqlen_k / num_splits), so shorter sequences have empty chunks.
 *   window_size 0: every key of the sequence.  window_size W >= 1: the query (its sequence's
 *     last position) sees only the sequence's last W keys (BlockDiagonalCausalLocalAttention-
 *     PaddedKeysMask and PagedBlockDiagonalCausalLocalPaddedKeysMask with one query per
 *     sequence); the chunks then cut those keys, ceil(min(max_seqlen_k, W) / num_splits) each.
 *   Device metadata is not read by the host: seqlens are clamped to [0, cap] and page
 *   numbers to the cache, so bad metadata gives unspecified values, never an
 *   out-of-bounds access; keys past num_splits chunks are not seen.
 *   Workspace, out, lse, scale and errors as in attn_decode_splitkv. */
attn_status attn_decode_splitkv_paged(const attn_tensor *q, const attn_tensor *k, const attn_tensor *v,
                                      const int32_t *seqlens, const int32_t *block_tables,
                                      int32_t max_blocks_per_seq, int32_t page_size, int32_t max_seqlen_k,
                                      int32_t window_size,
                                      int32_t num_splits, float scale, void *workspace, size_t workspace_bytes,
                                      const attn_tensor *out, float *lse, attn_stream_t stream);

/* Split-KV decode against a row-wise quantised FP8 K/V cache ("Attention - operator protocol",
 * InputsFp8: row/group quantised FP8 K/V caches whose scale/shift metadata the split-K decode
 * backends read directly; triton_splitk.FwOp: row-wise FP8 caches).  Stored row r of head h
 * holds D codes and G (scale, shift) pairs; its values are  fp8(code) * scale + shift  of
 * each element's group, and the result is that of attn_decode_splitkv / _paged on those
 * values.
 *   q [B, 1, (G,) H, D] bf16, D in {64, 128, 256}.
 *   k, v: ATTN_DTYPE_FP8_E4M3 caches laid out as in attn_decode_splitkv (seqlens and
 *     block_tables both NULL: every sequence holds all of its lane), or as in
 *     attn_decode_splitkv_paged (seqlens given: padded lanes; block_tables too: paged).
 *   k_scale_shift, v_scale_shift: ATTN_DTYPE_F16, the shape of k with D replaced by 2G,
 *     stride-1 last axis and 4-byte aligned rows: G (scale, shift) pairs of every cache row
 *     and head, one per group of D/G consecutive elements (G = 1: row-wise; D/G a multiple
 *     of 16), each one 32-bit word with the scale in its low half; element d's value is
 *     fp8(code) * scale_g + shift_g with g = d / (D/G).  Or ATTN_DTYPE_F32 (InputsFp8's
 *     use_fp32_scales), the same shape with 8-byte aligned rows: each pair two fp32, scale
 *     first.  k and v metadata share one dtype.
 *   out [B, 1, (G,) H, D] bf16 or fp32; lse fp32 [B, H_total, 1] or NULL.
 *   The codes and metadata are read as they are; NaN codes or metadata propagate.
 *   Workspace, splits, window_size, scale, device-metadata handling and errors as in
 *   attn_decode_splitkv_paged (with seqlens NULL every sequence holds its whole lane). */
attn_status attn_decode_splitkv_fp8(const attn_tensor *q, const attn_tensor *k, const attn_tensor *v,
                                    const attn_tensor *k_scale_shift, const attn_tensor *v_scale_shift,
                                    const int32_t *seqlens, const int32_t *block_tables,
                                    int32_t max_blocks_per_seq, int32_t page_size, int32_t max_seqlen_k,
                                    int32_t window_size,
                                    int32_t num_splits, float scale, void *workspace, size_t workspace_bytes,
                                    const attn_tensor *out, float *lse, attn_stream_t stream);

/* Split-KV decode against a row/group-wise INT4 K/V cache (triton_splitk.FwOp: fused
 * row/group INT4 caches stored through int32 words).  Row r of head h holds D codes
 * 0..15, eight per 32-bit word, and G (scale, shift) pairs, one per group of D/G
 * consecutive elements; element d is  code_d * scale_g + shift_g  with g = d / (D/G).
 *   q [B, 1, (G,) H, D] bf16, D in {64, 128, 256}.
 *   k, v: ATTN_DTYPE_INT4X2 caches, last dim D/2 bytes, laid out as in
 *     attn_decode_splitkv_fp8 (lanes, padded lanes or pages).
 *   k_scale_shift, v_scale_shift: ATTN_DTYPE_F16, the shape of k with the last axis 2G
 *     (G pairs, scale first), stride-1 last axis, 4-byte aligned rows; D/G must be a
 *     multiple of 32 (G in {1, 2, 4} for D = 128; {1, 2} for D = 64).  Or ATTN_DTYPE_F32
 *     pairs with 8-byte aligned rows, as for attn_decode_splitkv_fp8.
 *   Everything else as in attn_decode_splitkv_fp8. */
attn_status attn_decode_splitkv_int4(const attn_tensor *q, const attn_tensor *k, const attn_tensor *v,
                                     const attn_tensor *k_scale_shift, const attn_tensor *v_scale_shift,
                                     const int32_t *seqlens, const int32_t *block_tables,
                                     int32_t max_blocks_per_seq, int32_t page_size, int32_t max_seqlen_k,
                                     int32_t window_size,
                                     int32_t num_splits, float scale, void *workspace, size_t workspace_bytes,
                                     const attn_tensor *out, float *lse, attn_stream_t stream);

/* Split-KV decode against an MXFP8 K/V cache ("Attention - operator protocol": InputsMXFp8, FP8 K/V
 * with E8M0 block scales k_fp8_scale / v_fp8_scale).  Row r of head h holds D E4M3 codes and D/32
 * E8M0 scales, one per block of 32 consecutive elements (the MX standard block); element d's value
 * is  fp8(code_d) * 2^(e_{d/32} - 127).
 *   q [B, 1, (G,) H, D] bf16, D in {64, 128, 256}.
 *   k, v: ATTN_DTYPE_FP8_E4M3 caches laid out as in attn_decode_splitkv_fp8 (lanes, padded
 *     lanes or pages).
 *   k_scale, v_scale: ATTN_DTYPE_E8M0, the shape of k with the last axis D/32, stride-1 last axis.
 *   Everything else as in attn_decode_splitkv_fp8. */
attn_status attn_decode_splitkv_mxfp8(const attn_tensor *q, const attn_tensor *k, const attn_tensor *v,
                                      const attn_tensor *k_scale, const attn_tensor *v_scale,
                                      const int32_t *seqlens, const int32_t *block_tables,
                                      int32_t max_blocks_per_seq, int32_t page_size, int32_t max_seqlen_k,
                                      int32_t window_size,
                                      int32_t num_splits, float scale, void *workspace, size_t workspace_bytes,
                                      const attn_tensor *out, float *lse, attn_stream_t stream);

/* Reason for the last non-OK status returned on this thread ("" if none). */
const char *attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
