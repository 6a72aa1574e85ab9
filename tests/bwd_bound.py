"""Per-element worst-case error bound for the bf16 attention backward -- TEST INFRASTRUCTURE.

The GPU backward ("MSLK - complete kernel reference for LLM agents", Attention - Core fMHA,
memory_efficient_attention_backward) computes, for every (batch, head):

    x_ij  = fl32(q_i . k_j) * c - L_i            (c = fp32(scale log2 e), L_i = fp32(lse_i log2 e))
    P_ij  = exp2(x_ij)                             fp32, from the forward's saved fp32 lse
    D_i   = fl32(dout_i . out_i)                   with out the forward's bf16 output
    dP_ij = fl32(dout_i . v_j)
    dS_ij = bf16(P_ij (dP_ij - D_i))
    dq_i  = bf16(scale * fl32(sum_j dS_ij k_j))
    dk_j  = bf16(scale * fl32(sum_i dS_ij q_i))
    dv_j  = bf16(fl32(sum_i bf16(P_ij) dout_i))

q, k, v and dout are exact bf16 values, so every product of two of them is exact in fp32.
With u = 2^-8 (bf16, 8 significant bits, round to nearest), e = 2^-24 (fp32) and
g(n) = n e (the classic bound for an n-term fp32 sum, any order), first-order error
propagation against the exact (fp64) gradients gives, with |.| taken elementwise:

    rel. error of P_ij      r_ij = g(K) A_ij + 2e (|s_ij| + |lse_i|) + 2^-22 + E_i
                            A_ij = |scale| |q_i|.|k_j|,  E_i the forward LSE error:
                            E_i  = max_j (g(K) A_ij + 2e |s_ij|) + g(Mkv) + 2^-16 + 2e |lse_i|
                            (2^-22 covers exp2/log2 to a few ulp, 2^-16 a chain of rescales)
    error of the forward out  |dO_id| <= (u + R_i) |O_id| + (u + R_i + g(Mkv)) (P |v|)_id,
                            R_i = max_j r_ij
    error of D_i            dD_i = sum_d |dout_id| dO_id + g(Kv) sum_d |dout_id||O_id|
    error of dS_ij          F_ij = (u + r_ij + 2e) |dS_ij| + P_ij (g(Kv) (|dout||v|^T)_ij + dD_i)
    dq_i:   u |dq_i| + |scale| (F |k| + g(Mkv) |dS| |k|)_i + e |dq_i|
    dk_j:   u |dk_j| + |scale| (F^T |q| + g(Mq) |dS|^T |q|)_j + e |dk_j|
    dv_j:   u |dv_j| + ((u + r + g(Mq)) o P)^T |dout| (row j)

Underflow: a result below the smallest normal fp32 (n = 2^-126; bf16 has the same range) may
be flushed to zero or kept denormal, an absolute error of at most n either way.  Each visible
P and dS element, each bf16 output, each product entering an fp32 sum and each forward
weight 2^(x - m) (at most 2^8 before its division by l >= 1) adds that much:
F_ij gains n (2 + |dP_ij - D_i|) on visible keys, the forward out's error 2^8 n (vis |v|),
dq and dk gain n (1 + Mkv) and n (1 + Mq) besides F's share, and dv gains
(2n vis)^T |dout| + n (1 + Mq).  These terms matter only where the gradients themselves
underflow (keys whose scores lie ~90 below the row maximum).

The D term is what makes keys with a large shared component sensitive: dq_i holds
scale D_i sum_j P_ij k_j, which cancels only for exact D.  Second-order terms (u^2 and
smaller) are covered by the factor 1 + 8u that the tests apply.  Nothing here comes from
the GPU path: the bound is evaluated in fp64 from the oracle's inputs and outputs.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from oracle import brute

U_BF16 = 2.0 ** -8
E_F32 = 2.0 ** -24
ETA = 2.0 ** -126  # smallest normal fp32 (and bf16): the most a flushed or denormal result is off
SECOND_ORDER = 1.0 + 8 * U_BF16


def _g(n: int) -> float:
    return n * E_F32


def bwd_error_bound(q, k, v, dout, out, lse, ref, mask=0, scale=None, seqstart_q=None, seqstart_k=None,
                    window=None, window_right=None, workers=16):
    """Bounds [B, M, H, D] for |dq|, |dk|, |dv| errors of the bf16 backward (first order; the
    caller multiplies by SECOND_ORDER).  q, k, v, dout: exact inputs; out, lse: the oracle's
    exact forward; ref: the oracle's (dq, dk, dv)."""
    q, k, v, dout, out = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout, out))
    lse = np.asarray(lse, dtype=np.float64)
    B, Mq, H, K = q.shape
    Mkv, Kv = k.shape[1], v.shape[-1]
    sc = 1.0 / math.sqrt(K) if scale is None else float(scale)
    vis = np.isfinite(brute.materialize(mask, Mq, Mkv, seqstart_q, seqstart_k, window, window_right))
    dq_r, dk_r, dv_r = (np.asarray(x, dtype=np.float64) for x in ref)
    bq, bk, bv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)

    def one(bh):
        b, h = divmod(bh, H)
        qi, ki, vi, gi, oi = q[b, :, h], k[b, :, h], v[b, :, h], dout[b, :, h], out[b, :, h]
        L = lse[b, h]
        has = np.isfinite(L)
        Lf = np.where(has, L, 0.0)
        S = sc * (qi @ ki.T)
        A = abs(sc) * (np.abs(qi) @ np.abs(ki).T)
        see = vis & has[:, None]
        P = np.exp(np.where(see, S - Lf[:, None], -np.inf))
        aS_ = np.where(see, np.abs(S), 0.0)
        aL = np.abs(Lf)[:, None]
        E = np.max(np.where(see, _g(K) * A + 2 * E_F32 * aS_, 0.0), axis=1) + _g(Mkv) + 2.0 ** -16 \
            + 2 * E_F32 * np.abs(Lf)
        r = np.where(see, _g(K) * A + 2 * E_F32 * (aS_ + aL) + 2.0 ** -22 + E[:, None], 0.0)
        R = r.max(axis=1)[:, None]
        ag, ao, av = np.abs(gi), np.abs(oi), np.abs(vi)
        vf = see.astype(np.float64)
        dO = (U_BF16 + R) * ao + (U_BF16 + R + _g(Mkv)) * (P @ av) + 2.0 ** 8 * ETA * (vf @ av)
        dD = np.sum(ag * dO, axis=1) + _g(Kv) * np.sum(ag * ao, axis=1)
        D = np.sum(gi * oi, axis=1)
        dPD = (gi @ vi.T) - D[:, None]
        dS = P * dPD
        adS = np.abs(dS)
        F = (U_BF16 + r + 2 * E_F32) * adS + P * (_g(Kv) * (ag @ av.T) + dD[:, None]) \
            + ETA * vf * (2.0 + np.abs(dPD))
        aq, ak = np.abs(qi), np.abs(ki)
        bq[b, :, h] = (U_BF16 + E_F32) * np.abs(dq_r[b, :, h]) + abs(sc) * (F @ ak + _g(Mkv) * (adS @ ak)) \
            + ETA * (1 + Mkv)
        bk[b, :, h] = (U_BF16 + E_F32) * np.abs(dk_r[b, :, h]) + abs(sc) * (F.T @ aq + _g(Mq) * (adS.T @ aq)) \
            + ETA * (1 + Mq)
        bv[b, :, h] = (U_BF16 + E_F32) * np.abs(dv_r[b, :, h]) + ((U_BF16 + r + _g(Mq)) * P + 2 * ETA * vf).T @ ag \
            + ETA * (1 + Mq)

    with ThreadPoolExecutor(max(1, min(workers, B * H))) as ex:
        list(ex.map(one, range(B * H)))
    return bq, bk, bv


def bound_ratio(got, ref, bound) -> float:
    """max over elements of |got - ref| / (SECOND_ORDER * bound); exact agreement where the bound is 0."""
    got, ref, bound = (np.asarray(x, dtype=np.float64) for x in (got, ref, bound))
    err = np.abs(got - ref)
    lim = SECOND_ORDER * bound
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(lim > 0, err / np.where(lim > 0, lim, 1.0), np.where(err > 0, np.inf, 0.0))
    return float(ratio.max()) if ratio.size else 0.0
