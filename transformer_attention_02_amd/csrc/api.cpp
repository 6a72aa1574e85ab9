// C-ABI front end: validates descriptors on the host (integer checks only, no
// device access, no allocation, no synchronisation), picks a kernel and launches
// it on the caller's stream.  Any failure returns before a launch, with the
// reason in a thread-local string (the pages' not_supported_reasons idea,
// "Attention - Backend operator classes" in the MSLK kernel reference).
#include "../../include/attn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <atomic>
#include <mutex>

#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

attn_status fail(attn_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

attn_status ok() {
    g_err[0] = '\0';
    return ATTN_OK;
}

size_t dtype_size(int dt) {
    return dt == ATTN_DTYPE_F32 ? 4
                                : ((dt == ATTN_DTYPE_FP8_E4M3 || dt == ATTN_DTYPE_INT4X2 || dt == ATTN_DTYPE_E8M0) ? 1 : 2);
}

constexpr unsigned DT_FLOAT = (1u << ATTN_DTYPE_F32) | (1u << ATTN_DTYPE_BF16);  // q/k/v/out of every path

// A tensor normalised to [B, M, Htot, D] with head addressing (sg, sh, Hin).
struct View {
    void *p;
    int dtype;
    int ndim;
    int64_t B, M, G, H, D;
    attn::Strides s;
};

// `dtypes`: bit set of the attn_dtype values accepted; `align`: byte alignment of row starts.
attn_status make_view(const attn_tensor *t, const char *name, View *v, unsigned dtypes = DT_FLOAT, int align = 16) {
    if (!t) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: descriptor is NULL", name);
    if (t->dtype < 0 || t->dtype > ATTN_DTYPE_E8M0 || !((dtypes >> t->dtype) & 1u))
        return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: dtype %d is not accepted here", name, t->dtype);
    if (t->ndim != 4 && t->ndim != 5)
        return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: ndim must be 4 [B,M,H,D] or 5 [B,M,G,H,D], got %d", name, t->ndim);
    for (int i = 0; i < t->ndim; ++i) {
        if (t->shape[i] < 0) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: negative shape[%d]", name, i);
        if (t->shape[i] > 0x7fffffff) return fail(ATTN_ERR_UNSUPPORTED, "%s: shape[%d] exceeds 2^31-1", name, i);
        if (t->stride[i] < 0) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: negative stride[%d]", name, i);
    }
    const int last = t->ndim - 1;
    if (t->stride[last] != 1)
        return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: the last dimension must have stride 1 (got %lld)", name,
                    (long long)t->stride[last]);
    v->p = t->data;
    v->dtype = t->dtype;
    v->ndim = t->ndim;
    v->B = t->shape[0];
    v->M = t->shape[1];
    if (t->ndim == 4) {
        v->G = 1;
        v->H = t->shape[2];
        v->s = attn::Strides{t->stride[0], t->stride[1], 0, t->stride[2]};
    } else {
        v->G = t->shape[2];
        v->H = t->shape[3];
        v->s = attn::Strides{t->stride[0], t->stride[1], t->stride[2], t->stride[3]};
    }
    v->D = t->shape[last];
    if (v->G * v->H > 0x7fffffff) return fail(ATTN_ERR_UNSUPPORTED, "%s: too many heads", name);
    const int64_t n = v->B * v->M * v->G * v->H * v->D;
    if (n > 0) {
        if (!v->p) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: data pointer is NULL", name);
        // aligned row starts: base pointer and every outer stride in bytes
        const size_t es = dtype_size(v->dtype);
        if (((uintptr_t)v->p) % align != 0)
            return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: data pointer is not %d-byte aligned", name, align);
        for (int i = 0; i < last; ++i)
            if ((t->stride[i] * (int64_t)es) % align != 0)
                return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: stride[%d]=%lld elements is not a multiple of %d bytes",
                            name, i, (long long)t->stride[i], align);
    }
    return ATTN_OK;
}

int64_t htot(const View &v) { return v.G * v.H; }

bool same_heads(const View &a, const View &b) { return a.ndim == b.ndim && a.G == b.G && a.H == b.H; }

// Tensors the kernels write get each element written once: an axis of extent > 1 with
// stride 0 would have several workgroups store to the same address.
attn_status check_written(const char *fn, const char *name, const View &x) {
    const int64_t ext[4] = {x.B, x.M, x.G, x.H};
    const int64_t str[4] = {x.s.b, x.s.m, x.s.g, x.s.h};
    for (int i = 0; i < 4; ++i)
        if (ext[i] > 1 && str[i] == 0)
            return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: %s must not have stride-0 axes", fn, name);
    return ATTN_OK;
}

attn_status launch_status(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(ATTN_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

// Mask kind -> (packed, bottom_right, wl, wr) of the kernels' visible-key interval.
struct MaskSpec {
    int packed, bottom_right, wl, wr;
};

attn_status mask_spec(const char *fn, const attn_mask &m, MaskSpec *out) {
    const int inf = attn::kWinInf;
    auto clampw = [&](int64_t w) { return (int)(w >= inf ? inf : w); };
    switch (m.kind) {
    case ATTN_MASK_NONE: *out = {0, 0, inf, inf}; break;
    case ATTN_MASK_CAUSAL: *out = {0, 0, inf, 0}; break;
    case ATTN_MASK_BLOCKDIAG: *out = {1, 0, inf, inf}; break;
    case ATTN_MASK_BLOCKDIAG_CAUSAL: *out = {1, 0, inf, 0}; break;
    case ATTN_MASK_CAUSAL_BOTTOMRIGHT: *out = {0, 1, inf, 0}; break;
    case ATTN_MASK_BLOCKDIAG_CAUSAL_BOTTOMRIGHT: *out = {1, 1, inf, 0}; break;
    case ATTN_MASK_LOCAL_BOTTOMRIGHT:
        if (m.window_left < 0 || m.window_right < 0)
            return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: window_left and window_right must be >= 0", fn);
        *out = {0, 1, clampw(m.window_left), clampw(m.window_right)};
        break;
    case ATTN_MASK_CAUSAL_LOCAL_BOTTOMRIGHT:
    case ATTN_MASK_BLOCKDIAG_CAUSAL_LOCAL:
    case ATTN_MASK_BLOCKDIAG_CAUSAL_LOCAL_BOTTOMRIGHT:
        if (m.window_size < 1) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: window_size must be >= 1", fn);
        *out = {m.kind != ATTN_MASK_CAUSAL_LOCAL_BOTTOMRIGHT, m.kind != ATTN_MASK_BLOCKDIAG_CAUSAL_LOCAL,
                clampw((int64_t)m.window_size - 1), 0};
        break;
    default:
        return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: unknown mask kind %d", fn, m.kind);
    }
    return ATTN_OK;
}

// Shared validation and launch for attn_fwd / attn_partial (and the _ex forms).
attn_status forward(const char *fn, bool partial, const attn_tensor *qt, const attn_tensor *kt,
                    const attn_tensor *vt, const attn_mask &mask, const attn_varlen *varlen, float scale,
                    const attn_tensor *ot, float *lse, attn_stream_t stream) {
    View q, k, v, o;
    attn_status st;
    if ((st = make_view(qt, "q", &q)) != ATTN_OK) return st;
    if ((st = make_view(kt, "k", &k)) != ATTN_OK) return st;
    if ((st = make_view(vt, "v", &v)) != ATTN_OK) return st;
    if ((st = make_view(ot, "out", &o)) != ATTN_OK) return st;
    if (k.dtype != q.dtype || v.dtype != q.dtype)
        return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: q, k and v must share one dtype", fn);
    if (partial) {
        if (o.dtype != ATTN_DTYPE_F32 && o.dtype != q.dtype)
            return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: out must be fp32 or q's dtype", fn);
        if (!lse) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: lse is required", fn);
    } else if (o.dtype != q.dtype) {
        return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: out must have q's dtype", fn);
    }
    if (!same_heads(q, k) || !same_heads(q, v) || !same_heads(q, o))
        return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: q, k, v and out must have the same rank and head axes", fn);
    if (k.B != q.B || v.B != q.B || o.B != q.B) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: batch sizes differ", fn);
    if (v.M != k.M) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: k and v have different key counts", fn);
    if (o.M != q.M) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: out must have q's row count", fn);
    if (k.D != q.D) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: q and k head dims differ", fn);
    if (o.D != v.D) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: out head dim must equal v's", fn);
    if ((st = check_written(fn, "out", o)) != ATTN_OK) return st;
    MaskSpec ms;
    if ((st = mask_spec(fn, mask, &ms)) != ATTN_OK) return st;
    const bool packed = ms.packed;
    if (packed) {
        if (!varlen) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: block-diagonal masks need varlen", fn);
        if (q.B != 1) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: packed sequences need B == 1", fn);
        if (varlen->nseq < 1 || !varlen->seqstart_q)
            return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: varlen needs nseq >= 1 and seqstart_q", fn);
        if (varlen->max_seqlen_q < 0 || varlen->max_seqlen_q > q.M)
            return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: max_seqlen_q must be in [0, Mq]", fn);
        if ((((uintptr_t)varlen->seqstart_q) % 4) || (((uintptr_t)varlen->seqstart_k) % 4))
            return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: seqstart arrays must be 4-byte aligned", fn);
    }
    if (!(std::isnan(scale) || std::isfinite(scale)))
        return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: scale must be finite (or NaN for 1/sqrt(K))", fn);
    if (lse && ((uintptr_t)lse) % 4) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: lse must be 4-byte aligned", fn);
    if (q.D < 1 || v.D < 1) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: head dims must be >= 1", fn);

    if (q.dtype == ATTN_DTYPE_BF16) {
        auto dim_ok = [](int64_t d) { return d == 64 || d == 128 || d == 256; };
        if (!(dim_ok(q.D) && dim_ok(v.D)))
            return fail(ATTN_ERR_UNSUPPORTED, "%s: bf16 kernels need K and Kv in {64, 128, 256} (got K=%lld, Kv=%lld)",
                        fn, (long long)q.D, (long long)v.D);
        // key tiles are fetched through buffer descriptors whose range ends at the last valid key row
        if (k.M > 1 && (k.s.m < k.D || v.s.m < v.D))
            return fail(ATTN_ERR_UNSUPPORTED, "%s: bf16 kernels need key/value row strides >= the head dim", fn);
        if ((k.s.m * 2 * 64 + k.D * 2) >= (int64_t)1 << 31 || (v.s.m * 2 * 64 + v.D * 2) >= (int64_t)1 << 31)
            return fail(ATTN_ERR_UNSUPPORTED, "%s: key/value row stride too large for 32-bit tile offsets", fn);
    } else {
        if (q.D > 128 || v.D > 128)
            return fail(ATTN_ERR_UNSUPPORTED, "%s: fp32 kernel needs K, Kv <= 128 (got K=%lld, Kv=%lld)", fn,
                        (long long)q.D, (long long)v.D);
    }
    if (q.B == 0 || q.M == 0 || htot(q) == 0) return ok();  // nothing to compute

    attn::FwdArgs a;
    a.q = q.p;
    a.k = k.p;
    a.v = v.p;
    a.o = o.p;
    a.lse = lse;
    a.sq = q.s;
    a.sk = k.s;
    a.sv = v.s;
    a.so = o.s;
    a.B = (int)q.B;
    a.Mq = (int)q.M;
    a.Mkv = (int)k.M;
    a.Htot = (int)htot(q);
    a.Hin = (int)q.H;
    a.K = (int)q.D;
    a.Kv = (int)v.D;
    const double sc = std::isnan(scale) ? 1.0 / std::sqrt((double)q.D) : (double)scale;
    a.scale_log2 = (float)(sc * 1.4426950408889634);
    if (std::fabs(a.scale_log2) < 1e-30f) a.scale_log2 = std::copysign(1e-30f, a.scale_log2);  // keeps -inf masking exact
    a.packed = ms.packed;
    a.bottom_right = ms.bottom_right;
    a.wl = ms.wl;
    a.wr = ms.wr;
    if (packed) {
        a.seqstart_q = varlen->seqstart_q;
        a.seqstart_k = varlen->seqstart_k;
        a.nseq = varlen->nseq;
        a.max_seqlen_q = varlen->max_seqlen_q;
    } else {
        a.seqstart_q = a.seqstart_k = nullptr;
        a.nseq = 1;
        a.max_seqlen_q = a.Mq;
    }
    a.kv_groups = (k.s.h == 0 && v.s.h == 0 && q.H > 1) ? (int)(htot(q) / q.H) : 0;
    a.seqlens_k = nullptr;
    a.block_tables = nullptr;
    a.bt_stride = a.page_size = a.num_pages = a.cap = 0;
    a.splits = 1;
    a.chunk = 0;
    a.o_split = a.lse_split = 0;
    hipError_t e;
    if (q.dtype == ATTN_DTYPE_BF16)
        e = attn::launch_fwd_bf16(a, o.dtype == ATTN_DTYPE_F32, (hipStream_t)stream);
    else
        e = attn::launch_fwd_f32(a, (hipStream_t)stream);
    return launch_status(e, fn);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

extern "C" {

const char *attn_last_error(void) { return g_err; }

static attn_status plain_mask(const char *fn, int32_t kind, attn_mask *m) {
    if (kind >= ATTN_MASK_LOCAL_BOTTOMRIGHT && kind <= ATTN_MASK_BLOCKDIAG_CAUSAL_LOCAL_BOTTOMRIGHT)
        return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: mask kind %d needs window sizes: use the _ex entry point", fn,
                    kind);
    *m = attn_mask{kind, 0, 0, 0};
    return ATTN_OK;
}

attn_status attn_fwd(const attn_tensor *q, const attn_tensor *k, const attn_tensor *v, int32_t mask,
                     const attn_varlen *varlen, float scale, const attn_tensor *out, float *lse,
                     attn_stream_t stream) {
    attn_mask m;
    attn_status st = plain_mask("attn_fwd", mask, &m);
    return st != ATTN_OK ? st : forward("attn_fwd", false, q, k, v, m, varlen, scale, out, lse, stream);
}

attn_status attn_partial(const attn_tensor *q, const attn_tensor *k, const attn_tensor *v, int32_t mask,
                         const attn_varlen *varlen, float scale, const attn_tensor *out, float *lse,
                         attn_stream_t stream) {
    attn_mask m;
    attn_status st = plain_mask("attn_partial", mask, &m);
    return st != ATTN_OK ? st : forward("attn_partial", true, q, k, v, m, varlen, scale, out, lse, stream);
}

attn_status attn_fwd_ex(const attn_tensor *q, const attn_tensor *k, const attn_tensor *v, const attn_mask *mask,
                        const attn_varlen *varlen, float scale, const attn_tensor *out, float *lse,
                        attn_stream_t stream) {
    if (!mask) return fail(ATTN_ERR_INVALID_ARGUMENT, "attn_fwd_ex: mask is NULL");
    return forward("attn_fwd_ex", false, q, k, v, *mask, varlen, scale, out, lse, stream);
}

attn_status attn_partial_ex(const attn_tensor *q, const attn_tensor *k, const attn_tensor *v, const attn_mask *mask,
                            const attn_varlen *varlen, float scale, const attn_tensor *out, float *lse,
                            attn_stream_t stream) {
    if (!mask) return fail(ATTN_ERR_INVALID_ARGUMENT, "attn_partial_ex: mask is NULL");
    return forward("attn_partial_ex", true, q, k, v, *mask, varlen, scale, out, lse, stream);
}

attn_status attn_merge(int32_t n_chunks, const attn_tensor *out_chunks, const float *const *lse_chunks,
                       const attn_tensor *out, float *lse_out, attn_stream_t stream) {
    const char *fn = "attn_merge";
    if (n_chunks < 1) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: need at least one chunk", fn);
    if (n_chunks > ATTN_MAX_CHUNKS)
        return fail(ATTN_ERR_UNSUPPORTED, "%s: at most %d chunks per call", fn, ATTN_MAX_CHUNKS);
    if (!out_chunks || !lse_chunks) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: chunk arrays are NULL", fn);
    View c0, o;
    attn_status st;
    if ((st = make_view(&out_chunks[0], "out_chunks[0]", &c0)) != ATTN_OK) return st;
    if ((st = make_view(out, "out", &o)) != ATTN_OK) return st;
    for (int i = 1; i < n_chunks; ++i) {
        View ci;
        char nm[32];
        snprintf(nm, sizeof nm, "out_chunks[%d]", i);
        if ((st = make_view(&out_chunks[i], nm, &ci)) != ATTN_OK) return st;
        if (ci.dtype != c0.dtype || ci.ndim != c0.ndim || ci.B != c0.B || ci.M != c0.M || ci.G != c0.G ||
            ci.H != c0.H || ci.D != c0.D)
            return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: chunk %d differs from chunk 0 in dtype or shape", fn, i);
        if (ci.s.b != c0.s.b || ci.s.m != c0.s.m || ci.s.g != c0.s.g || ci.s.h != c0.s.h)
            return fail(ATTN_ERR_UNSUPPORTED, "%s: chunk %d has different strides from chunk 0", fn, i);
    }
    if (!same_heads(o, c0) || o.B != c0.B || o.M != c0.M || o.D != c0.D)
        return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: out shape differs from the chunks'", fn);
    if ((st = check_written(fn, "out", o)) != ATTN_OK) return st;
    const int64_t rows = c0.B * c0.M * htot(c0);
    for (int i = 0; i < n_chunks; ++i)
        if (rows > 0 && (!lse_chunks[i] || ((uintptr_t)lse_chunks[i]) % 4))
            return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: lse_chunks[%d] is NULL or misaligned", fn, i);
    if (lse_out && ((uintptr_t)lse_out) % 4) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: lse_out misaligned", fn);
    if (rows == 0 || c0.D == 0) return ok();

    attn::MergeArgs a;
    memset(&a, 0, sizeof a);
    for (int i = 0; i < n_chunks; ++i) {
        a.chunk[i] = out_chunks[i].data;
        a.lse[i] = lse_chunks[i];
    }
    a.sc = c0.s;
    a.o = o.p;
    a.so = o.s;
    a.lse_out = lse_out;
    a.S = n_chunks;
    a.B = (int)c0.B;
    a.M = (int)c0.M;
    a.Htot = (int)htot(c0);
    a.Hin = (int)c0.H;
    a.Kv = (int)c0.D;
    a.chunk_f32 = c0.dtype == ATTN_DTYPE_F32;
    a.out_f32 = o.dtype == ATTN_DTYPE_F32;
    return launch_status(attn::launch_merge(a, (hipStream_t)stream), fn);
}

size_t attn_fwd_kvcache_workspace_bytes(int64_t Mq, int64_t H_total, int64_t Kv, int32_t num_splits) {
    if (Mq < 0 || H_total < 0 || Kv < 0 || num_splits < 2) return 0;
    const size_t rows = (size_t)num_splits * (size_t)Mq * (size_t)H_total;
    return align256(rows * (size_t)Kv * 4) + align256(rows * 4);
}

attn_status attn_fwd_kvcache(const attn_tensor *qt, const attn_tensor *kt, const attn_tensor *vt, const attn_mask *mask,
                             const int32_t *seqstart_q, int32_t nseq, int32_t max_seqlen_q, const int32_t *seqstart_k,
                             const int32_t *seqlens_k,
                             const int32_t *block_tables, int32_t max_blocks_per_seq, int32_t page_size,
                             int32_t max_seqlen_k, int32_t num_splits, float scale, void *workspace,
                             size_t workspace_bytes, const attn_tensor *ot, float *lse, attn_stream_t stream) {
    const char *fn = "attn_fwd_kvcache";
    View q, k, v, o;
    attn_status st;
    if ((st = make_view(qt, "q", &q)) != ATTN_OK) return st;
    if ((st = make_view(kt, "k", &k)) != ATTN_OK) return st;
    if ((st = make_view(vt, "v", &v)) != ATTN_OK) return st;
    if ((st = make_view(ot, "out", &o)) != ATTN_OK) return st;
    if (!mask) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: mask is NULL", fn);
    if (q.dtype != ATTN_DTYPE_BF16 || k.dtype != q.dtype || v.dtype != q.dtype || o.dtype != q.dtype)
        return fail(ATTN_ERR_UNSUPPORTED, "%s: q, k, v and out must be bf16", fn);
    if (!same_heads(q, k) || !same_heads(q, v) || !same_heads(q, o))
        return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: q, k, v and out must have the same rank and head axes", fn);
    if (q.B != 1 || o.B != 1) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: packed queries need B == 1", fn);
    if (o.M != q.M) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: out must have q's row count", fn);
    if (k.D != q.D) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: q and k head dims differ", fn);
    if (o.D != v.D) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: out head dim must equal v's", fn);
    if (v.M != k.M || v.B != k.B) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: k and v caches differ in shape", fn);
    if ((st = check_written(fn, "out", o)) != ATTN_OK) return st;
    // the padded-keys masks: every one aligned from the bottom right of its sequence
    const int kind = mask->kind;
    if (kind != ATTN_MASK_NONE && kind != ATTN_MASK_CAUSAL_BOTTOMRIGHT && kind != ATTN_MASK_LOCAL_BOTTOMRIGHT &&
        kind != ATTN_MASK_CAUSAL_LOCAL_BOTTOMRIGHT)
        return fail(ATTN_ERR_INVALID_ARGUMENT,
                    "%s: mask kind %d; the KV-cache forward takes NONE, CAUSAL_BOTTOMRIGHT, LOCAL_BOTTOMRIGHT or "
                    "CAUSAL_LOCAL_BOTTOMRIGHT",
                    fn, kind);
    MaskSpec ms;
    if ((st = mask_spec(fn, *mask, &ms)) != ATTN_OK) return st;
    if (nseq < 1 || !seqstart_q || !seqlens_k)
        return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: needs nseq >= 1, seqstart_q and seqlens_k", fn);
    if ((((uintptr_t)seqstart_q) % 4) || (((uintptr_t)seqlens_k) % 4) || (((uintptr_t)block_tables) % 4) ||
        (((uintptr_t)seqstart_k) % 4))
        return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: index arrays must be 4-byte aligned", fn);
    if (seqstart_k && block_tables)
        return fail(ATTN_ERR_UNSUPPORTED, "%s: gappy lanes (seqstart_k) over a paged cache are not built", fn);
    if (max_seqlen_q < 0 || max_seqlen_q > q.M)
        return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: max_seqlen_q must be in [0, Mq]", fn);
    const bool paged = block_tables != nullptr;
    int64_t cap;
    if (paged) {
        if (k.B != 1) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: a paged cache has batch 1", fn);
        if (page_size < 64 || page_size % 64)
            return fail(ATTN_ERR_UNSUPPORTED, "%s: page_size must be a multiple of 64 (got %d)", fn, page_size);
        if (max_blocks_per_seq < 1) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: max_blocks_per_seq must be >= 1", fn);
        if (max_blocks_per_seq > 8192)
            return fail(ATTN_ERR_UNSUPPORTED, "%s: at most 8192 pages per sequence (got %d)", fn, max_blocks_per_seq);
        if (k.M % page_size || k.M == 0)
            return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: the cache must hold a whole number of pages", fn);
        if (k.D != v.D) return fail(ATTN_ERR_UNSUPPORTED, "%s: a paged cache needs equal head dims", fn);
        if (k.D != 64 && k.D != 128 && k.D != 256)
            return fail(ATTN_ERR_UNSUPPORTED, "%s: paged head dims must be 64, 128 or 256", fn);
        cap = (int64_t)max_blocks_per_seq * page_size;
        if (cap > 0x7fffffff) return fail(ATTN_ERR_UNSUPPORTED, "%s: sequences too long", fn);
    } else if (seqstart_k) {
        if (k.B != 1) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: gappy lanes index one k/v tensor (B == 1)", fn);
        cap = k.M;
    } else {
        if (k.B < nseq) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: k/v need a lane per sequence (B >= nseq)", fn);
        cap = k.M;
    }
    if (max_seqlen_k < 0 || max_seqlen_k > cap)
        return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: max_seqlen_k must be in [0, %lld]", fn, (long long)cap);
    if (num_splits < 1 || num_splits > ATTN_MAX_CHUNKS)
        return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: num_splits must be in [1, %d]", fn, ATTN_MAX_CHUNKS);
    if (!(std::isnan(scale) || std::isfinite(scale)))
        return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: scale must be finite (or NaN for 1/sqrt(K))", fn);
    if (lse && ((uintptr_t)lse) % 4) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: lse must be 4-byte aligned", fn);
    auto dim_ok = [](int64_t d) { return d == 64 || d == 128 || d == 256; };
    if (!(dim_ok(q.D) && dim_ok(v.D)))
        return fail(ATTN_ERR_UNSUPPORTED, "%s: head dims K and Kv must be in {64, 128, 256}", fn);
    if ((k.M > 1 && (k.s.m < k.D || v.s.m < v.D)) || (k.s.m * 2 * 64 + k.D * 2) >= (int64_t)1 << 31 ||
        (v.s.m * 2 * 64 + v.D * 2) >= (int64_t)1 << 31)
        return fail(ATTN_ERR_UNSUPPORTED, "%s: key/value row strides must be >= the head dim and < 2^24 bytes", fn);
    const int64_t Htot = htot(q);
    const size_t need = attn_fwd_kvcache_workspace_bytes(q.M, Htot, v.D, num_splits);
    if (q.M == 0 || Htot == 0) return ok();
    if (num_splits > 1) {
        if (!workspace || ((uintptr_t)workspace) % 256)
            return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: workspace is NULL or not 256-byte aligned", fn);
        if (workspace_bytes < need)
            return fail(ATTN_ERR_WORKSPACE_TOO_SMALL, "%s: workspace needs %zu bytes, got %zu", fn, need,
                        workspace_bytes);
    }

    attn::FwdArgs a;
    a.q = q.p;
    a.k = k.p;
    a.v = v.p;
    a.sq = q.s;
    a.sk = k.s;
    a.sv = v.s;
    a.B = 1;
    a.Mq = (int)q.M;
    a.Mkv = (int)k.M;
    a.Htot = (int)Htot;
    a.Hin = (int)q.H;
    a.K = (int)q.D;
    a.Kv = (int)v.D;
    const double sc = std::isnan(scale) ? 1.0 / std::sqrt((double)q.D) : (double)scale;
    a.scale_log2 = (float)(sc * 1.4426950408889634);
    if (std::fabs(a.scale_log2) < 1e-30f) a.scale_log2 = std::copysign(1e-30f, a.scale_log2);
    a.packed = 1;
    a.bottom_right = 1;
    a.wl = ms.wl;
    a.wr = ms.wr;
    a.seqstart_q = seqstart_q;
    a.seqstart_k = seqstart_k;  // gappy lanes (with seqlens_k): the sequences' first key rows
    a.nseq = nseq;
    a.max_seqlen_q = max_seqlen_q;
    a.kv_groups = (k.s.h == 0 && v.s.h == 0 && q.H > 1) ? (int)(Htot / q.H) : 0;
    a.seqlens_k = seqlens_k;
    a.block_tables = block_tables;
    a.bt_stride = paged ? max_blocks_per_seq : 0;
    a.page_size = paged ? page_size : 0;
    a.num_pages = paged ? (int)(k.M / page_size) : 0;
    a.cap = (int)cap;
    a.splits = num_splits;
    // chunks of whole 64-key tiles
    a.chunk = (int)(((int64_t)max_seqlen_k + num_splits - 1) / num_splits + 63) / 64 * 64;
    const int64_t rows = q.M * Htot;
    const attn::Strides part{rows * v.D, Htot * v.D, q.H * v.D, v.D};  // [1, Mq, (G,) H, Kv] fp32, per chunk
    if (num_splits == 1) {
        a.o = o.p;
        a.so = o.s;
        a.lse = lse;
        a.o_split = a.lse_split = 0;
        return launch_status(attn::launch_fwd_bf16(a, false, (hipStream_t)stream), fn);
    }
    float *ws_o = (float *)workspace;
    float *ws_lse = (float *)((char *)workspace + align256((size_t)num_splits * rows * v.D * 4));
    a.o = ws_o;
    a.so = part;
    a.lse = ws_lse;
    a.o_split = rows * v.D;
    a.lse_split = rows;
    hipError_t e = attn::launch_fwd_bf16(a, true, (hipStream_t)stream);
    if (e != hipSuccess) return launch_status(e, fn);
    attn::MergeArgs m;
    memset(&m, 0, sizeof m);
    for (int c = 0; c < num_splits; ++c) {
        m.chunk[c] = ws_o + (size_t)c * rows * v.D;
        m.lse[c] = ws_lse + (size_t)c * rows;
    }
    m.sc = part;
    m.o = o.p;
    m.so = o.s;
    m.lse_out = lse;
    m.S = num_splits;
    m.B = 1;
    m.M = (int)q.M;
    m.Htot = (int)Htot;
    m.Hin = (int)q.H;
    m.Kv = (int)v.D;
    m.chunk_f32 = 1;
    m.out_f32 = 0;
    return launch_status(attn::launch_merge(m, (hipStream_t)stream), fn);
}

size_t attn_bwd_workspace_bytes(int64_t B, int64_t H_total, int64_t Mq) {
    if (B < 0 || H_total < 0 || Mq < 0) return 0;
    return 2 * align256((size_t)B * (size_t)H_total * (size_t)Mq * 4);
}

// dS^T buffer of the kept-dS backward: per (batch, head) round_up(Mkv, 128) key rows of
// round_up(Mq, 256) bf16 query columns, after the two row arrays
static const int64_t kDsMaxPitch = (int64_t)1 << 24;  // 64 rows of a dS^T tile stay below 2^31 bytes

size_t attn_bwd_ds_workspace_bytes(int64_t B, int64_t H_total, int64_t Mq, int64_t Mkv) {
    if (B < 0 || H_total < 0 || Mq < 0 || Mkv < 0) return 0;
    const int64_t pitch = (Mq + 255) / 256 * 256, krows = (Mkv + 127) / 128 * 128;
    if (pitch > kDsMaxPitch) return SIZE_MAX;
    typedef unsigned __int128 u128;
    const u128 ds = (u128)B * (u128)H_total * (u128)krows * (u128)pitch * 2u;
    const u128 total = (u128)attn_bwd_workspace_bytes(B, H_total, Mq) + (ds + 255) / 256 * 256;
    return total >= (u128)SIZE_MAX ? SIZE_MAX : (size_t)total;
}

attn_status attn_bwd(const attn_tensor *dot, const attn_tensor *qt, const attn_tensor *kt, const attn_tensor *vt,
                     const attn_tensor *ot, const float *lse, const attn_mask *mask, const attn_varlen *varlen,
                     float scale, void *workspace, size_t workspace_bytes, const attn_tensor *dqt,
                     const attn_tensor *dkt, const attn_tensor *dvt, attn_stream_t stream) {
    const char *fn = "attn_bwd";
    View g, q, k, v, o, dq, dk, dv;
    attn_status st;
    if ((st = make_view(dot, "dout", &g)) != ATTN_OK) return st;
    if ((st = make_view(qt, "q", &q)) != ATTN_OK) return st;
    if ((st = make_view(kt, "k", &k)) != ATTN_OK) return st;
    if ((st = make_view(vt, "v", &v)) != ATTN_OK) return st;
    if ((st = make_view(ot, "out", &o)) != ATTN_OK) return st;
    if ((st = make_view(dqt, "dq", &dq)) != ATTN_OK) return st;
    if ((st = make_view(dkt, "dk", &dk)) != ATTN_OK) return st;
    if ((st = make_view(dvt, "dv", &dv)) != ATTN_OK) return st;
    if (!mask) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: mask is NULL", fn);
    for (const View *x : {&g, &k, &v, &o, &dq, &dk, &dv})
        if (x->dtype != q.dtype) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: all tensors must share q's dtype", fn);
    for (const View *x : {&g, &k, &v, &o, &dq, &dk, &dv})
        if (!same_heads(*x, q)) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: rank and head axes must match q's", fn);
    auto same_shape = [](const View &a_, const View &b_) { return a_.B == b_.B && a_.M == b_.M && a_.D == b_.D; };
    if (!same_shape(dq, q)) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: dq must have q's shape", fn);
    if (!same_shape(dk, k)) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: dk must have k's shape", fn);
    if (!same_shape(dv, v)) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: dv must have v's shape", fn);
    if (g.B != q.B || g.M != q.M || o.B != q.B || o.M != q.M || g.D != v.D || o.D != v.D)
        return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: dout and out must be [B, Mq, ..., Kv]", fn);
    if (v.B != k.B || v.M != k.M) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: k and v have different key counts", fn);
    if (k.B != q.B) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: batch sizes differ", fn);
    if (k.D != q.D) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: q and k head dims differ", fn);
    for (const View *x : {&dq, &dk, &dv})
        if ((st = check_written(fn, "gradient tensors", *x)) != ATTN_OK) return st;
    if (q.D < 1 || v.D < 1) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: head dims must be >= 1", fn);
    if (q.dtype == ATTN_DTYPE_BF16) {
        if (!((q.D == 64 || q.D == 128) && v.D == q.D))
            return fail(ATTN_ERR_UNSUPPORTED, "%s: the bf16 backward needs K == Kv in {64, 128}", fn);
        // tiles of q/dout (key-side kernel) and k/v (query-side kernel) go through buffer descriptors
        for (const View *x : {&q, &g, &k, &v}) {
            if (x->M > 1 && x->s.m < x->D)
                return fail(ATTN_ERR_UNSUPPORTED, "%s: row strides must be >= the head dim", fn);
            if (x->s.m * 2 * 64 + x->D * 2 >= (int64_t)1 << 31)
                return fail(ATTN_ERR_UNSUPPORTED, "%s: row stride too large for 32-bit tile offsets", fn);
        }
    } else if (q.D > 128 || v.D > 128) {
        return fail(ATTN_ERR_UNSUPPORTED, "%s: the fp32 backward needs K, Kv <= 128", fn);
    }
    MaskSpec ms;
    if ((st = mask_spec(fn, *mask, &ms)) != ATTN_OK) return st;
    if (ms.packed) {
        if (!varlen) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: block-diagonal masks need varlen", fn);
        if (q.B != 1) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: packed sequences need B == 1", fn);
        if (varlen->nseq < 1 || !varlen->seqstart_q)
            return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: varlen needs nseq >= 1 and seqstart_q", fn);
        if (varlen->max_seqlen_q < 0 || varlen->max_seqlen_q > q.M)
            return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: max_seqlen_q must be in [0, Mq]", fn);
        if (varlen->max_seqlen_k > k.M)
            return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: max_seqlen_k must be <= Mkv", fn);
        if ((((uintptr_t)varlen->seqstart_q) % 4) || (((uintptr_t)varlen->seqstart_k) % 4))
            return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: seqstart arrays must be 4-byte aligned", fn);
    }
    if (!(std::isnan(scale) || std::isfinite(scale)))
        return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: scale must be finite (or NaN for 1/sqrt(K))", fn);
    const int64_t rows = q.B * htot(q) * q.M;
    if (rows > 0 && (!lse || ((uintptr_t)lse) % 4))
        return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: lse is NULL or not 4-byte aligned", fn);
    const size_t need = attn_bwd_workspace_bytes(q.B, htot(q), q.M);
    if (rows > 0 && (!workspace || ((uintptr_t)workspace) % 256))
        return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: workspace is NULL or not 256-byte aligned", fn);
    if (rows > 0 && workspace_bytes < need)
        return fail(ATTN_ERR_WORKSPACE_TOO_SMALL, "%s: workspace needs %zu bytes, got %zu", fn, need, workspace_bytes);
    if (q.B == 0 || htot(q) == 0 || (q.M == 0 && k.M == 0)) return ok();

    attn::BwdArgs a;
    a.q = q.p;
    a.k = k.p;
    a.v = v.p;
    a.o = o.p;
    a.dout = g.p;
    a.dq = dq.p;
    a.dk = dk.p;
    a.dv = dv.p;
    a.sq = q.s;
    a.sk = k.s;
    a.sv = v.s;
    a.so = o.s;
    a.sdo = g.s;
    a.sdq = dq.s;
    a.sdk = dk.s;
    a.sdv = dv.s;
    a.lse = lse;
    a.ws_d = (float *)workspace;
    a.ws_l2 = (float *)((char *)workspace + need / 2);
    a.B = (int)q.B;
    a.Mq = (int)q.M;
    a.Mkv = (int)k.M;
    a.Htot = (int)htot(q);
    a.Hin = (int)q.H;
    a.D = (int)q.D;
    a.Dv = (int)v.D;
    const double sc = std::isnan(scale) ? 1.0 / std::sqrt((double)q.D) : (double)scale;
    a.scale = (float)sc;
    a.scale_log2 = (float)(sc * 1.4426950408889634);
    a.packed = ms.packed;
    a.bottom_right = ms.bottom_right;
    a.wl = ms.wl;
    a.wr = ms.wr;
    if (ms.packed) {
        a.seqstart_q = varlen->seqstart_q;
        a.seqstart_k = varlen->seqstart_k;
        a.nseq = varlen->nseq;
        a.max_seqlen_q = varlen->max_seqlen_q;
        a.max_seqlen_k = varlen->max_seqlen_k > 0 ? varlen->max_seqlen_k : (int)k.M;
    } else {
        a.seqstart_q = a.seqstart_k = nullptr;
        a.nseq = 1;
        a.max_seqlen_q = a.Mq;
        a.max_seqlen_k = a.Mkv;
    }
    a.ds = nullptr;
    a.ds_pitch = a.ds_rows = 0;
    const size_t need_ds = attn_bwd_ds_workspace_bytes(q.B, htot(q), q.M, k.M);
    // head dim 128 only: at 64 the dS round trip costs more than the recomputation it saves
    if (q.dtype == ATTN_DTYPE_BF16 && q.D == 128 && !ms.packed && need_ds != SIZE_MAX && workspace_bytes >= need_ds) {
        a.ds = (char *)workspace + need;
        a.ds_pitch = (q.M + 255) / 256 * 256;
        a.ds_rows = (k.M + 127) / 128 * 128;
    }
    return launch_status(q.dtype == ATTN_DTYPE_BF16 ? attn::launch_bwd_bf16(a, (hipStream_t)stream)
                                                    : attn::launch_bwd_f32(a, (hipStream_t)stream),
                         fn);
}

int32_t attn_decode_num_splits(int64_t B, int64_t H_total, int64_t Mkv) {
    if (B <= 0 || H_total <= 0 || Mkv <= 0) return 1;
    // compute units of the current device (256 on MI355X; that value when no device answers)
    static std::atomic<int> cus[64];  // per device, 0 until first asked; racing threads store the same value
    int dev = 0, n = 256;
    if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64) {
        n = cus[dev].load(std::memory_order_relaxed);
        if (!n) {
            int c = 0;
            n = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && c > 0 ? c : 256;
            cus[dev].store(n, std::memory_order_relaxed);
        }
    } else {
        (void)hipGetLastError();  // leave no error behind for the caller's next HIP call
    }
    // enough (split, batch, head) rows for 8 per compute unit, chunks of at least 256 keys
    const int64_t units = B * H_total, target = 8 * (int64_t)n;
    int32_t S = 1;
    while (S < ATTN_MAX_CHUNKS && units * S < target && Mkv / (2 * S) >= 256) S *= 2;
    return S;
}

size_t attn_decode_workspace_bytes(int64_t B, int64_t H_total, int64_t Kv, int32_t num_splits) {
    if (B < 0 || H_total < 0 || Kv < 0 || num_splits < 1) return 0;
    const size_t rows = (size_t)num_splits * (size_t)B * (size_t)H_total;
    return align256(rows * (size_t)Kv * 4) + align256(rows * 4);
}

}  // extern "C"

namespace {

// Shared validation and launches of the split-KV decode entry points.  Without block tables
// k/v are [B, cap, (G,) H, D] lanes; with them k/v are the paged cache [1, pages * page_size, ...].
// `quant`: 0 = k/v share q's dtype; ATTN_DTYPE_FP8_E4M3 / ATTN_DTYPE_INT4X2 = k/v are codes of that
// type with (scale, shift) metadata ksst / vsst; `mx`: FP8 codes with E8M0 block scales instead.
attn_status decode(const char *fn, int quant, const attn_tensor *qt, const attn_tensor *kt, const attn_tensor *vt,
                   const attn_tensor *ksst, const attn_tensor *vsst, const int32_t *seqlens,
                   const int32_t *block_tables, int32_t max_blocks_per_seq, int32_t page_size, int32_t max_seqlen_k,
                   int32_t window_size, int32_t num_splits, float scale, void *workspace, size_t workspace_bytes,
                   const attn_tensor *ot, float *lse, attn_stream_t stream, bool mx = false) {
    View q, k, v, o, kss{}, vss{};
    attn_status st;
    const unsigned kv_dt = quant ? 1u << quant : DT_FLOAT;
    if ((st = make_view(qt, "q", &q)) != ATTN_OK) return st;
    if ((st = make_view(kt, "k", &k, kv_dt)) != ATTN_OK) return st;
    if ((st = make_view(vt, "v", &v, kv_dt)) != ATTN_OK) return st;
    if ((st = make_view(ot, "out", &o)) != ATTN_OK) return st;
    int group = 0;  // elements per (scale, shift) group or E8M0 block
    if (mx) {
        if ((st = make_view(ksst, "k_scale", &kss, 1u << ATTN_DTYPE_E8M0, 1)) != ATTN_OK) return st;
        if ((st = make_view(vsst, "v_scale", &vss, 1u << ATTN_DTYPE_E8M0, 1)) != ATTN_OK) return st;
        if (q.dtype != ATTN_DTYPE_BF16) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: q must be bf16", fn);
        if (k.D % 32 || kss.D != k.D / 32 || vss.D != kss.D)
            return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: block scales need D a multiple of 32 and a last axis D/32",
                        fn);
        for (const View *m : {&kss, &vss})
            if (!same_heads(*m, k) || m->B != k.B || m->M != k.M)
                return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: block scales must have k's shape with the last axis D/32",
                            fn);
        group = 32;
    } else if (quant) {
        // (scale, shift) pairs of two fp16 (one 32-bit word) or, InputsFp8's use_fp32_scales, of two
        // fp32 (one 64-bit word, rows 8-byte aligned)
        const unsigned ss_dt = (1u << ATTN_DTYPE_F16) | (1u << ATTN_DTYPE_F32);
        if ((st = make_view(ksst, "k_scale_shift", &kss, ss_dt, 4)) != ATTN_OK) return st;
        if ((st = make_view(vsst, "v_scale_shift", &vss, ss_dt, 4)) != ATTN_OK) return st;
        if (kss.dtype != vss.dtype)
            return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: k and v scale/shift tensors must share one dtype", fn);
        if (kss.dtype == ATTN_DTYPE_F32) {
            if ((st = make_view(ksst, "k_scale_shift", &kss, ss_dt, 8)) != ATTN_OK) return st;
            if ((st = make_view(vsst, "v_scale_shift", &vss, ss_dt, 8)) != ATTN_OK) return st;
        }
        if (q.dtype != ATTN_DTYPE_BF16) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: q must be bf16", fn);
        // INT4 rows are D/2 bytes: compare head dims in elements
        if (quant == ATTN_DTYPE_INT4X2) {
            k.D *= 2;
            v.D *= 2;
        }
        const int64_t G = kss.D / 2;
        if (kss.D % 2 || kss.D != vss.D)
            return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: scale/shift last axes must be 2G (equal for k and v)", fn);
        for (const View *m : {&kss, &vss})
            if (!same_heads(*m, k) || m->B != k.B || m->M != k.M)
                return fail(ATTN_ERR_INVALID_ARGUMENT,
                            "%s: scale/shift tensors must have k's shape with the last axis 2G", fn);
        // a lane reads 16 FP8 codes or 32 INT4 codes of one row: each lane's codes share a group
        const int64_t lane_elems = quant == ATTN_DTYPE_FP8_E4M3 ? 16 : 32;
        if (G < 1 || k.D % G || (k.D / G) % lane_elems)
            return fail(ATTN_ERR_UNSUPPORTED, "%s: groups of D/G elements must be a multiple of %lld", fn,
                        (long long)lane_elems);
        group = (int)(k.D / G);
    } else if (k.dtype != q.dtype || v.dtype != q.dtype || o.dtype != q.dtype) {
        return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: q, k, v and out must share one dtype", fn);
    }
    if (!same_heads(q, k) || !same_heads(q, v) || !same_heads(q, o))
        return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: q, k, v and out must have the same rank and head axes", fn);
    const bool paged = block_tables != nullptr;
    if (o.B != q.B) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: batch sizes differ", fn);
    if (paged) {
        if (k.B != 1 || v.B != 1) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: a paged cache has batch 1", fn);
    } else if (k.B != q.B || v.B != q.B) {
        return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: batch sizes differ", fn);
    }
    if (q.M != 1 || o.M != 1) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: decode takes one query row (M == 1)", fn);
    if ((st = check_written(fn, "out", o)) != ATTN_OK) return st;
    if (v.M != k.M) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: k and v have different key counts", fn);
    if (k.D != q.D || v.D != q.D || o.D != q.D)
        return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: q, k, v and out head dims must match", fn);
    if (!(q.D == 64 || q.D == 128 || q.D == 256))
        return fail(ATTN_ERR_UNSUPPORTED, "%s: head dim must be 64, 128 or 256", fn);
    if (num_splits < 1) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: num_splits must be >= 1", fn);
    if (num_splits > ATTN_MAX_CHUNKS)
        return fail(ATTN_ERR_UNSUPPORTED, "%s: num_splits must be <= %d", fn, ATTN_MAX_CHUNKS);
    if (window_size < 0) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: window_size must be >= 0 (0: none)", fn);
    if (!(std::isnan(scale) || std::isfinite(scale)))
        return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: scale must be finite (or NaN for 1/sqrt(K))", fn);
    if (lse && ((uintptr_t)lse) % 4) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: lse must be 4-byte aligned", fn);
    int64_t cap = k.M;  // keys a sequence may hold
    if (seqlens || paged) {
        if (!seqlens || ((uintptr_t)seqlens) % 4)
            return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: seqlens must be a 4-byte aligned device array", fn);
        if (paged) {
            if (((uintptr_t)block_tables) % 4)
                return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: block_tables must be 4-byte aligned", fn);
            if (page_size < 1 || max_blocks_per_seq < 1)
                return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: page_size and max_blocks_per_seq must be >= 1", fn);
            if (k.M % page_size != 0 || k.M == 0)
                return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: the cache must hold a whole number of pages", fn);
            cap = (int64_t)max_blocks_per_seq * page_size;
            if (cap > 0x7fffffff) return fail(ATTN_ERR_UNSUPPORTED, "%s: sequences too long", fn);
        }
        if (max_seqlen_k < 0 || max_seqlen_k > cap)
            return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: max_seqlen_k must be in [0, %lld]", fn, (long long)cap);
    } else {
        max_seqlen_k = (int32_t)k.M;
    }
    const size_t need = attn_decode_workspace_bytes(q.B, htot(q), q.D, num_splits);
    if (q.B == 0 || htot(q) == 0) return ok();
    if (!workspace || ((uintptr_t)workspace) % 256)
        return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: workspace is NULL or not 256-byte aligned", fn);
    if (workspace_bytes < need)
        return fail(ATTN_ERR_WORKSPACE_TOO_SMALL, "%s: workspace needs %zu bytes, got %zu", fn, need, workspace_bytes);
    const int64_t rows = (int64_t)num_splits * q.B * htot(q);
    if (rows > 0x7fffffff) return fail(ATTN_ERR_UNSUPPORTED, "%s: too many (split, batch, head) rows", fn);

    attn::DecodeArgs d;
    d.q = q.p;
    d.k = k.p;
    d.v = v.p;
    d.sq = q.s;
    d.sk = k.s;
    d.sv = v.s;
    d.B = (int)q.B;
    d.Mkv = (int)k.M;
    d.Htot = (int)htot(q);
    d.Hin = (int)q.H;
    d.D = (int)q.D;
    d.S = num_splits;
    // with a window the chunks cover the last window_size keys of each sequence
    const int64_t span = window_size > 0 ? std::min<int64_t>(max_seqlen_k, window_size) : max_seqlen_k;
    d.chunk = (int)((span + num_splits - 1) / num_splits);
    d.window = window_size;
    const double sc = std::isnan(scale) ? 1.0 / std::sqrt((double)q.D) : (double)scale;
    d.scale_log2 = (float)(sc * 1.4426950408889634);
    d.ws_o = (float *)workspace;
    d.ws_lse = (float *)((char *)workspace + align256((size_t)rows * q.D * 4));
    d.seqlens = seqlens;
    d.block_tables = block_tables;
    d.bt_stride = max_blocks_per_seq;
    d.page_size = page_size;
    d.num_pages = paged ? (int)(k.M / page_size) : 0;
    d.cap = (int)cap;
    d.kss = kss.p;
    d.vss = vss.p;
    d.skss = kss.s;
    d.svss = vss.s;
    d.group = group;
    d.ss32 = quant && !mx && kss.dtype == ATTN_DTYPE_F32;
    const int elem = mx ? attn::DECODE_MXFP8
                     : quant == ATTN_DTYPE_FP8_E4M3 ? attn::DECODE_FP8
                     : quant == ATTN_DTYPE_INT4X2 ? attn::DECODE_INT4
                     : (q.dtype == ATTN_DTYPE_F32 ? attn::DECODE_F32 : attn::DECODE_BF16);
    hipError_t e = attn::launch_decode_partials(d, elem, (hipStream_t)stream);
    if (e != hipSuccess) return launch_status(e, fn);

    attn::MergeArgs m;
    memset(&m, 0, sizeof m);
    const int64_t per = q.B * htot(q);
    for (int s = 0; s < num_splits; ++s) {
        m.chunk[s] = d.ws_o + (size_t)s * per * q.D;
        m.lse[s] = d.ws_lse + (size_t)s * per;
    }
    // workspace chunk layout [B, 1, Htot, D] contiguous, addressed like [B, M, G, H, D]
    m.sc = attn::Strides{htot(q) * q.D, htot(q) * q.D, q.H * q.D, q.D};
    m.o = o.p;
    m.so = o.s;
    m.lse_out = lse;
    m.S = num_splits;
    m.B = (int)q.B;
    m.M = 1;
    m.Htot = (int)htot(q);
    m.Hin = (int)q.H;
    m.Kv = (int)q.D;
    m.chunk_f32 = 1;
    m.out_f32 = o.dtype == ATTN_DTYPE_F32;
    return launch_status(attn::launch_merge(m, (hipStream_t)stream), fn);
}

}  // namespace

// Device scratch of attn_decode_splitkv_noalloc: the decode's per-chunk partial outputs and LSEs
// live here instead of in a caller workspace.  Every GPU the library runs on holds its own copy
// until the process ends.  In host code `scratch` names a host-side stand-in, not device memory:
// its device address comes from hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxDevices] = {};

// Device address of the current device's scratch, looked up on the device's first call.
attn_status scratch_address(const char *fn, void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(ATTN_ERR_LAUNCH, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(ATTN_ERR_UNSUPPORTED, "%s: device %d out of range", fn, dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(ATTN_ERR_LAUNCH, "%s: hipGetSymbolAddress(scratch) failed on device %d: %s", fn, dev,
                        hipGetErrorString(e));
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return ATTN_OK;
}

}  // namespace

extern "C" {

attn_status attn_decode_splitkv_noalloc(const attn_tensor *qt, const attn_tensor *kt, const attn_tensor *vt,
                                        int32_t num_splits, float scale, const attn_tensor *ot, float *lse,
                                        attn_stream_t stream) {
    const char *fn = "attn_decode_splitkv_noalloc";
    View q;
    attn_status st;
    if ((st = make_view(qt, "q", &q)) != ATTN_OK) return st;
    const size_t need = attn_decode_workspace_bytes(q.B, htot(q), q.D, num_splits);
    if (need > (size_t)ATTN_NOALLOC_SCRATCH_BYTES)
        return fail(ATTN_ERR_UNSUPPORTED,
                    "%s: the call needs %zu bytes of scratch, more than the library's static %zu; "
                    "use attn_decode_splitkv with a caller workspace",
                    fn, need, (size_t)ATTN_NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    if ((st = scratch_address(fn, &ws)) != ATTN_OK) return st;
    return decode(fn, 0, qt, kt, vt, nullptr, nullptr, nullptr, nullptr, 0, 0, 0, 0, num_splits, scale, ws,
                  (size_t)ATTN_NOALLOC_SCRATCH_BYTES, ot, lse, stream);
}

attn_status attn_decode_splitkv(const attn_tensor *qt, const attn_tensor *kt, const attn_tensor *vt,
                                int32_t num_splits, float scale, void *workspace, size_t workspace_bytes,
                                const attn_tensor *ot, float *lse, attn_stream_t stream) {
    return decode("attn_decode_splitkv", 0, qt, kt, vt, nullptr, nullptr, nullptr, nullptr, 0, 0, 0, 0, num_splits,
                  scale, workspace, workspace_bytes, ot, lse, stream);
}

attn_status attn_decode_splitkv_paged(const attn_tensor *q, const attn_tensor *k, const attn_tensor *v,
                                      const int32_t *seqlens, const int32_t *block_tables,
                                      int32_t max_blocks_per_seq, int32_t page_size, int32_t max_seqlen_k,
                                      int32_t window_size,
                                      int32_t num_splits, float scale, void *workspace, size_t workspace_bytes,
                                      const attn_tensor *out, float *lse, attn_stream_t stream) {
    return decode("attn_decode_splitkv_paged", 0, q, k, v, nullptr, nullptr, seqlens, block_tables,
                  max_blocks_per_seq, page_size, max_seqlen_k, window_size, num_splits, scale, workspace,
                  workspace_bytes, out, lse, stream);
}

attn_status attn_decode_splitkv_fp8(const attn_tensor *q, const attn_tensor *k, const attn_tensor *v,
                                    const attn_tensor *k_scale_shift, const attn_tensor *v_scale_shift,
                                    const int32_t *seqlens, const int32_t *block_tables,
                                    int32_t max_blocks_per_seq, int32_t page_size, int32_t max_seqlen_k,
                                    int32_t window_size,
                                    int32_t num_splits, float scale, void *workspace, size_t workspace_bytes,
                                    const attn_tensor *out, float *lse, attn_stream_t stream) {
    const char *fn = "attn_decode_splitkv_fp8";
    if (block_tables && !seqlens) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: block_tables need seqlens", fn);
    return decode(fn, ATTN_DTYPE_FP8_E4M3, q, k, v, k_scale_shift, v_scale_shift, seqlens, block_tables,
                  max_blocks_per_seq, page_size, max_seqlen_k, window_size, num_splits, scale, workspace,
                  workspace_bytes, out, lse, stream);
}

attn_status attn_decode_splitkv_int4(const attn_tensor *q, const attn_tensor *k, const attn_tensor *v,
                                     const attn_tensor *k_scale_shift, const attn_tensor *v_scale_shift,
                                     const int32_t *seqlens, const int32_t *block_tables,
                                     int32_t max_blocks_per_seq, int32_t page_size, int32_t max_seqlen_k,
                                     int32_t window_size,
                                     int32_t num_splits, float scale, void *workspace, size_t workspace_bytes,
                                     const attn_tensor *out, float *lse, attn_stream_t stream) {
    const char *fn = "attn_decode_splitkv_int4";
    if (block_tables && !seqlens) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: block_tables need seqlens", fn);
    return decode(fn, ATTN_DTYPE_INT4X2, q, k, v, k_scale_shift, v_scale_shift, seqlens, block_tables,
                  max_blocks_per_seq, page_size, max_seqlen_k, window_size, num_splits, scale, workspace,
                  workspace_bytes, out, lse, stream);
}

attn_status attn_decode_splitkv_mxfp8(const attn_tensor *q, const attn_tensor *k, const attn_tensor *v,
                                      const attn_tensor *k_scale, const attn_tensor *v_scale,
                                      const int32_t *seqlens, const int32_t *block_tables,
                                      int32_t max_blocks_per_seq, int32_t page_size, int32_t max_seqlen_k,
                                      int32_t window_size,
                                      int32_t num_splits, float scale, void *workspace, size_t workspace_bytes,
                                      const attn_tensor *out, float *lse, attn_stream_t stream) {
    const char *fn = "attn_decode_splitkv_mxfp8";
    if (block_tables && !seqlens) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: block_tables need seqlens", fn);
    return decode(fn, ATTN_DTYPE_FP8_E4M3, q, k, v, k_scale, v_scale, seqlens, block_tables, max_blocks_per_seq,
                  page_size, max_seqlen_k, window_size, num_splits, scale, workspace, workspace_bytes, out, lse, stream,
                  true);
}

}  // extern "C"
