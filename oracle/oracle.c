/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.  A plain, slow fp64 CPU attention
 * used to check the HIP kernels.  Only the tests, the smoke check and the
 * bench's CPU-baseline leg may load it; the product path never does.  It
 * shares no code, header, table or helper with the HIP library.
 *
 * What it computes (one definition, written out):
 *
 *   MSLK - complete kernel reference for LLM agents, "Attention - Core fMHA",
 *   memory_efficient_attention: scaled Q K^T, the mask as an additive 0/-inf
 *   bias, softmax over keys, product with V; the output keeps the query layout
 *   with the last axis taken from V.
 *   memory_efficient_attention_forward_requires_grad: also returns the
 *   per-row log-sum-exp (LSE).
 *   memory_efficient_attention_partial: the same over one disjoint K/V shard.
 *   memory_efficient_attention_backward: the exact gradients dq, dk, dv for an
 *   upstream gradient, given the forward's out and lse (oracle_attention_backward).
 *   merge_attentions: the exact LSE-weighted combination of shard results.
 *
 * For batch b, head h, query row i and allowed key set A(i):
 *   s_ij   = scale * sum_d q[b,i,h,d] k[b,j,h,d]          (j in A(i))
 *   m_i    = max_j s_ij
 *   l_i    = sum_j exp(s_ij - m_i)
 *   out_i  = sum_j exp(s_ij - m_i) / l_i * v[b,j,h,:]
 *   lse_i  = m_i + ln l_i                                   (natural log)
 * An empty A(i) gives out_i = 0 and lse_i = -inf.
 *
 * Mask kinds (A(i)):
 *   0 none:            all keys                      (no attn_bias)
 *   1 causal top-left: j <= i                        ("Attention - Biases &
 *                      masks", LowerTriangularMask: zeros on and below the
 *                      diagonal, -inf above)
 *   2 block-diagonal:  the keys of the query's own packed sequence
 *                      (BlockDiagonalMask)
 *   3 block-diagonal causal: same sequence and j - ks <= i - qs, the
 *                      top-left causal mask inside every block
 *                      (BlockDiagonalCausalMask)
 *   The windowed / bottom-right kinds use, per sequence with Lq query rows and
 *   Lk keys (the whole tensor when not packed), local row i and local key j:
 *   d = j - i - shift, visible iff -wl <= d <= wr, where shift = Lk - Lq for
 *   bottom-right alignment (the diagonal ends in the last key) and 0 otherwise.
 *   4 causal bottom-right        shift=Lk-Lq, wr=0          (LowerTriangularFromBottomRightMask)
 *   5 block-diag causal b-right  per block, as 4            (BlockDiagonalCausalFromBottomRightMask)
 *   6 local bottom-right(L, R)   shift=Lk-Lq, wl=L, wr=R    (LocalAttentionFromBottomRightMask)
 *   7 causal local b-right(W)    shift=Lk-Lq, wl=W-1, wr=0  (LowerTriangularFromBottomRightLocalAttentionMask)
 *   8 block-diag causal local(W) per block, shift=0, wl=W-1, wr=0 (BlockDiagonalCausalLocalAttentionMask)
 *   9 block-diag causal local b-right(W) per block, as 7    (BlockDiagonalCausalLocalAttentionFromBottomRightMask)
 *   A window of size W lets a row see the W keys ending at its diagonal.
 *
 * Merge of S chunks (merge_attentions; "MSLK Kernel Library -- Complete
 * Reference", Quick start, "Exact softmax merge"):
 *   M* = max_c lse_c,  L = M* + ln sum_c exp(lse_c - M*),
 *   out = sum_c exp(lse_c - L) out_c.   All chunks at -inf give 0 and -inf.
 *
 * Quantised K/V caches ("Attention - operator protocol", InputsFp8: row or group
 * quantised FP8 K/V with scale/shift metadata, read directly by the split-K decode
 * backends): every stored key or value row r of one head holds D FP8 E4M3 codes and
 * one (scale, shift) pair; its value is fp8(code) * scale + shift.  The attention is
 * then the definition above applied to those values.
 *
 * INT4 caches (triton_splitk.FwOp, "row/group INT4 ... stored through int32"): unsigned
 * 4-bit codes, two per byte, with one (scale, shift) pair per group of D/G consecutive
 * elements of a row: x = code * scale + shift (oracle_dequant_int4_groupwise).
 *
 * Layouts (all contiguous, fp64):
 *   q [B,Mq,H,K], k [B,Mkv,H,K], v [B,Mkv,H,Kv], out [B,Mq,H,Kv], lse [B,H,Mq].
 *   Packed sequences: B = 1, seqstart_q/seqstart_k are prefix sums [nseq+1].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_MASK_NONE = 0, OR_MASK_CAUSAL = 1, OR_MASK_BLOCKDIAG = 2, OR_MASK_BLOCKDIAG_CAUSAL = 3 };

/* Sequence index of packed row `r` given prefix sums `ss` of `nseq` sequences, or -1. */
static int seq_of_row(int64_t r, const int32_t *ss, int nseq) {
    for (int s = 0; s < nseq; ++s)
        if (r >= ss[s] && r < ss[s + 1]) return s;
    return -1;
}

static int is_packed(int mask) { return mask == 2 || mask == 3 || mask == 5 || mask == 8 || mask == 9; }

/* 1 when key j is in A(i).  Mq/Mkv are the whole extents (used when not packed). */
static int key_allowed(int mask, int64_t i, int64_t j, const int32_t *sq, const int32_t *sk, int nseq,
                       int64_t Mq, int64_t Mkv, int64_t win_l, int64_t win_r) {
    int64_t li = i, lj = j, Lq = Mq, Lk = Mkv;
    if (is_packed(mask)) {
        int s = seq_of_row(i, sq, nseq);
        if (s < 0) return 0;
        if (j < sk[s] || j >= sk[s + 1]) return 0;
        li = i - sq[s];
        lj = j - sk[s];
        Lq = sq[s + 1] - sq[s];
        Lk = sk[s + 1] - sk[s];
    }
    switch (mask) {
    case OR_MASK_NONE:
    case OR_MASK_BLOCKDIAG:
        return 1;
    case OR_MASK_CAUSAL:
    case OR_MASK_BLOCKDIAG_CAUSAL:
        return lj <= li;
    case 4:
    case 5:
        return lj - li - (Lk - Lq) <= 0;
    case 6: {
        const int64_t d = lj - li - (Lk - Lq);
        return d >= -win_l && d <= win_r;
    }
    case 7:
    case 9: {
        const int64_t d = lj - li - (Lk - Lq);
        return d <= 0 && d > -win_l;  /* win_l is the window size W */
    }
    case 8: {
        const int64_t d = lj - li;
        return d <= 0 && d > -win_l;
    }
    default:
        return 0;
    }
}

int oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Returns 0 on success, nonzero on a bad argument. */
/* win_l / win_r: window parameters of kinds 6 (left, right) and 7-9 (win_l = window size). */
int oracle_attention(int64_t B, int64_t Mq, int64_t Mkv, int64_t H, int64_t K, int64_t Kv,
                     const double *q, const double *k, const double *v, int mask, int nseq,
                     const int32_t *seqstart_q, const int32_t *seqstart_k, double scale,
                     int64_t win_l, int64_t win_r, double *out, double *lse) {
    if (B < 0 || Mq < 0 || Mkv < 0 || H < 0 || K < 1 || Kv < 1) return 1;
    if (mask < 0 || mask > 9) return 1;
    if (is_packed(mask) && (B != 1 || nseq < 1 || !seqstart_q || !seqstart_k)) return 1;
    if ((mask >= 7 && win_l < 1) || (mask == 6 && (win_l < 0 || win_r < 0))) return 1;

    const int64_t rows = B * H * Mq;
    int err = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(Mkv > 0 ? Mkv : 1));
        char *ok = (char *)malloc((size_t)(Mkv > 0 ? Mkv : 1));
        if (!s || !ok) {
#pragma omp atomic write
            err = 2;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < rows; ++r) {
                const int64_t b = r / (H * Mq);
                const int64_t h = (r / Mq) % H;
                const int64_t i = r % Mq;
                const double *qi = q + ((b * Mq + i) * H + h) * K;
                double *oi = out + ((b * Mq + i) * H + h) * Kv;

                /* scores over the allowed keys, and their maximum */
                double m = -INFINITY;
                int64_t n_allowed = 0;
                for (int64_t j = 0; j < Mkv; ++j) {
                    ok[j] = (char)key_allowed(mask, i, j, seqstart_q, seqstart_k, nseq, Mq, Mkv, win_l, win_r);
                    if (!ok[j]) continue;
                    const double *kj = k + ((b * Mkv + j) * H + h) * K;
                    double dot = 0.0;
                    for (int64_t d = 0; d < K; ++d) dot += qi[d] * kj[d];
                    s[j] = scale * dot;
                    if (s[j] > m) m = s[j];
                    ++n_allowed;
                }
                for (int64_t d = 0; d < Kv; ++d) oi[d] = 0.0;
                if (n_allowed == 0) {
                    lse[(b * H + h) * Mq + i] = -INFINITY;
                    continue;
                }
                /* normaliser */
                double l = 0.0;
                for (int64_t j = 0; j < Mkv; ++j)
                    if (ok[j]) l += exp(s[j] - m);
                /* weighted sum of value rows */
                for (int64_t j = 0; j < Mkv; ++j) {
                    if (!ok[j]) continue;
                    const double p = exp(s[j] - m) / l;
                    const double *vj = v + ((b * Mkv + j) * H + h) * Kv;
                    for (int64_t d = 0; d < Kv; ++d) oi[d] += p * vj[d];
                }
                lse[(b * H + h) * Mq + i] = m + log(l);
            }
        }
        free(s);
        free(ok);
    }
    return err;
}

/* Backward of the attention above ("Attention - Core fMHA", memory_efficient_attention_backward:
 * from the upstream gradient dout, the forward's out and lse and the original q, k, v, return
 * dq, dk, dv).  With P_ij = exp(s_ij - lse_i) on the visible keys (0 elsewhere), the gradient
 * of out_i = sum_j P_ij v_j is, written out:
 *   dv_j  = sum_i P_ij dout_i
 *   dP_ij = dout_i . v_j,   D_i = dout_i . out_i  (= sum_j P_ij dP_ij)
 *   dS_ij = P_ij (dP_ij - D_i)
 *   dq_i  = scale * sum_j dS_ij k_j,   dk_j = scale * sum_i dS_ij q_i.
 * Rows with lse = -inf (no visible key) contribute nothing.  Two passes, both parallel and
 * free of races: one over query rows for dq, one over key rows for dk and dv. */
static double dotn(const double *a, const double *b, int64_t n) {
    double acc = 0.0;
    for (int64_t d = 0; d < n; ++d) acc += a[d] * b[d];
    return acc;
}

int oracle_attention_backward(int64_t B, int64_t Mq, int64_t Mkv, int64_t H, int64_t K, int64_t Kv,
                              const double *q, const double *k, const double *v, const double *out,
                              const double *lse, const double *dout, int mask, int nseq,
                              const int32_t *seqstart_q, const int32_t *seqstart_k, double scale, int64_t win_l,
                              int64_t win_r, double *dq, double *dk, double *dv) {
    if (B < 0 || Mq < 0 || Mkv < 0 || H < 0 || K < 1 || Kv < 1) return 1;
    if (mask < 0 || mask > 9) return 1;
    if (is_packed(mask) && (B != 1 || nseq < 1 || !seqstart_q || !seqstart_k)) return 1;
    if ((mask >= 7 && win_l < 1) || (mask == 6 && (win_l < 0 || win_r < 0))) return 1;

    double *D = (double *)malloc(sizeof(double) * (size_t)(B * H * Mq > 0 ? B * H * Mq : 1));
    if (!D) return 2;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < B * H * Mq; ++r) {
        const int64_t b = r / (H * Mq), h = (r / Mq) % H, i = r % Mq;
        const int64_t o = ((b * Mq + i) * H + h) * Kv;
        D[r] = dotn(dout + o, out + o, Kv);
    }
    /* dq: one query row at a time */
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < B * H * Mq; ++r) {
        const int64_t b = r / (H * Mq), h = (r / Mq) % H, i = r % Mq;
        const double *qi = q + ((b * Mq + i) * H + h) * K;
        const double *gi = dout + ((b * Mq + i) * H + h) * Kv;
        double *dqi = dq + ((b * Mq + i) * H + h) * K;
        const double li = lse[(b * H + h) * Mq + i];
        for (int64_t d = 0; d < K; ++d) dqi[d] = 0.0;
        if (li == -INFINITY) continue;
        for (int64_t j = 0; j < Mkv; ++j) {
            if (!key_allowed(mask, i, j, seqstart_q, seqstart_k, nseq, Mq, Mkv, win_l, win_r)) continue;
            const double *kj = k + ((b * Mkv + j) * H + h) * K;
            const double *vj = v + ((b * Mkv + j) * H + h) * Kv;
            const double p = exp(scale * dotn(qi, kj, K) - li);
            const double ds = p * (dotn(gi, vj, Kv) - D[r]);
            for (int64_t d = 0; d < K; ++d) dqi[d] += scale * ds * kj[d];
        }
    }
    /* dk, dv: one key row at a time */
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t c = 0; c < B * H * Mkv; ++c) {
        const int64_t b = c / (H * Mkv), h = (c / Mkv) % H, j = c % Mkv;
        const double *kj = k + ((b * Mkv + j) * H + h) * K;
        const double *vj = v + ((b * Mkv + j) * H + h) * Kv;
        double *dkj = dk + ((b * Mkv + j) * H + h) * K;
        double *dvj = dv + ((b * Mkv + j) * H + h) * Kv;
        for (int64_t d = 0; d < K; ++d) dkj[d] = 0.0;
        for (int64_t d = 0; d < Kv; ++d) dvj[d] = 0.0;
        for (int64_t i = 0; i < Mq; ++i) {
            const int64_t r = (b * H + h) * Mq + i;
            if (lse[r] == -INFINITY) continue;
            if (!key_allowed(mask, i, j, seqstart_q, seqstart_k, nseq, Mq, Mkv, win_l, win_r)) continue;
            const double *qi = q + ((b * Mq + i) * H + h) * K;
            const double *gi = dout + ((b * Mq + i) * H + h) * Kv;
            const double p = exp(scale * dotn(qi, kj, K) - lse[r]);
            const double ds = p * (dotn(gi, vj, Kv) - D[r]);
            for (int64_t d = 0; d < Kv; ++d) dvj[d] += p * gi[d];
            for (int64_t d = 0; d < K; ++d) dkj[d] += scale * ds * qi[d];
        }
    }
    free(D);
    return 0;
}

/* FP8 E4M3 (OCP "FN" variant, the 8-bit float of MI355X): 1 sign bit, 4 exponent bits
 * with bias 7, 3 mantissa bits; exponent 0 holds subnormals m/8 * 2^-6; no infinities;
 * S.1111.111 is NaN.  Largest finite magnitude 1.75 * 2^8 = 448. */
double oracle_fp8_e4m3(uint8_t code) {
    const int sign = code >> 7, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    const double mag = e == 0 ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* Row-wise dequantisation of an FP8 K/V cache ("Attention - operator protocol" in the kernel
 * reference, InputsFp8: row/group quantised FP8 caches with scale/shift metadata):
 * x[r, d] = fp8(codes[r, d]) * ss[r, 0] + ss[r, 1] for `rows` rows of `D` values. */
void oracle_dequant_fp8_rowwise(int64_t rows, int64_t D, const uint8_t *codes, const double *ss, double *x) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t d = 0; d < D; ++d) x[r * D + d] = oracle_fp8_e4m3(codes[r * D + d]) * ss[2 * r] + ss[2 * r + 1];
}

/* Group-wise FP8 dequantisation (InputsFp8: "row/group quantised" FP8 caches): each of `rows`
 * rows holds D E4M3 codes and G (scale, shift) pairs, one per group of D/G consecutive elements:
 * x[r, d] = fp8(codes[r, d]) * ss[r, g, 0] + ss[r, g, 1],  g = d / (D/G).  G = 1 is the
 * row-wise form above. */
void oracle_dequant_fp8_groupwise(int64_t rows, int64_t D, int64_t G, const uint8_t *codes, const double *ss,
                                  double *x) {
    const int64_t gs = D / G;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t d = 0; d < D; ++d) {
            const int64_t g = d / gs;
            x[r * D + d] = oracle_fp8_e4m3(codes[r * D + d]) * ss[(r * G + g) * 2] + ss[(r * G + g) * 2 + 1];
        }
}

/* E8M0 block scale (the MX formats' shared scale): 2^(e - 127) for e = 0 .. 254; e = 255 is NaN. */
double oracle_e8m0(uint8_t e) { return e == 255 ? NAN : ldexp(1.0, (int)e - 127); }

/* MXFP8 dequantisation ("Attention - operator protocol": InputsMXFp8, FP8 K/V with E8M0 block
 * scales): each of `rows` rows holds D E4M3 codes and D/32 E8M0 scales, one per block of 32
 * consecutive elements (the MX standard's block size):  x[r, d] = fp8(codes[r, d]) * 2^(e[r, d/32] - 127). */
void oracle_dequant_mxfp8(int64_t rows, int64_t D, const uint8_t *codes, const uint8_t *e8m0, double *x) {
    const int64_t nb = D / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t d = 0; d < D; ++d)
            x[r * D + d] = oracle_fp8_e4m3(codes[r * D + d]) * oracle_e8m0(e8m0[r * nb + d / 32]);
}

/* Group-wise INT4 dequantisation (triton_splitk.FwOp: row/group INT4 caches stored through
 * int32 words): each of `rows` rows holds D unsigned 4-bit codes, two per byte, element 2i in
 * the low nibble of byte i (so eight per 32-bit word), and G (scale, shift) pairs, one per
 * group of D/G consecutive elements:  x[r, d] = code[r, d] * ss[r, g, 0] + ss[r, g, 1],
 * g = d / (D/G).  G = 1 is the row-wise form. */
void oracle_dequant_int4_groupwise(int64_t rows, int64_t D, int64_t G, const uint8_t *codes, const double *ss,
                                   double *x) {
    const int64_t gs = D / G;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t d = 0; d < D; ++d) {
            const uint8_t byte = codes[r * (D / 2) + d / 2];
            const int code = (d % 2 == 0) ? (byte & 15) : (byte >> 4);
            const int64_t g = d / gs;
            x[r * D + d] = code * ss[(r * G + g) * 2] + ss[(r * G + g) * 2 + 1];
        }
}

/* out_chunks [S,B,M,H,Kv], lse_chunks [S,B,H,M] -> out [B,M,H,Kv], lse [B,H,M]. */
int oracle_merge(int64_t S, int64_t B, int64_t M, int64_t H, int64_t Kv, const double *out_chunks,
                 const double *lse_chunks, double *out, double *lse) {
    if (S < 1 || B < 0 || M < 0 || H < 0 || Kv < 1) return 1;
    const int64_t rows = B * M * H;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t b = r / (M * H);
        const int64_t i = (r / H) % M;
        const int64_t h = r % H;
        const int64_t lse_off = (b * H + h) * M + i;
        double *o = out + r * Kv;
        for (int64_t d = 0; d < Kv; ++d) o[d] = 0.0;

        double mstar = -INFINITY;
        for (int64_t c = 0; c < S; ++c) {
            const double x = lse_chunks[c * B * H * M + lse_off];
            if (x > mstar) mstar = x;
        }
        if (mstar == -INFINITY) {
            lse[lse_off] = -INFINITY;
            continue;
        }
        double sum = 0.0;
        for (int64_t c = 0; c < S; ++c) sum += exp(lse_chunks[c * B * H * M + lse_off] - mstar);
        const double L = mstar + log(sum);
        for (int64_t c = 0; c < S; ++c) {
            const double w = exp(lse_chunks[c * B * H * M + lse_off] - L);
            const double *oc = out_chunks + c * B * M * H * Kv + r * Kv;
            for (int64_t d = 0; d < Kv; ++d) o[d] += w * oc[d];
        }
        lse[lse_off] = L;
    }
    return 0;
}
