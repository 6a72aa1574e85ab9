"""Dense numpy fp64 attention with a materialised mask bias -- TEST INFRASTRUCTURE.

An independent second reading of the same definition as ``oracle.c``, written
the way the pages describe a reference check: build the full [Mq, Mkv] bias of
zeros and -inf ("Attention - Biases & masks", AttentionBias.materialize), add it
to the scaled scores, take the softmax over keys and multiply by V
("Attention - Core fMHA", memory_efficient_attention).  The LSE is the log of
the plain sum of exponentials, with no maximum subtracted, so it is only meant
for the small, moderate-valued inputs of the tests.
"""
from __future__ import annotations

import math

import numpy as np

MASK_NONE, MASK_CAUSAL, MASK_BLOCKDIAG, MASK_BLOCKDIAG_CAUSAL = 0, 1, 2, 3
PACKED = (2, 3, 5, 8, 9)


def _block(bias, mask, qs, qe, ks, ke, window, window_right):
    """Fill the visible region of one (query block, key block) pair, row by row with slices."""
    Lq, Lk = qe - qs, ke - ks
    for r in range(Lq):
        if mask in (0, 2):
            lo, hi = 0, Lk - 1                       # everything
        elif mask in (1, 3):
            lo, hi = 0, r                            # top-left causal: keys up to the row
        elif mask in (4, 5):
            lo, hi = 0, r + Lk - Lq                  # diagonal ends in the last key
        elif mask == 6:
            c = r + Lk - Lq
            lo, hi = c - window, c + window_right    # window around the bottom-right diagonal
        elif mask in (7, 9):
            c = r + Lk - Lq
            lo, hi = c - window + 1, c               # the `window` keys ending at the diagonal
        else:                                        # 8: top-left causal window
            lo, hi = r - window + 1, r
        lo, hi = max(lo, 0), min(hi, Lk - 1)
        if hi >= lo:
            bias[qs + r, ks + lo: ks + hi + 1] = 0.0


def materialize(mask: int, Mq: int, Mkv: int, seqstart_q=None, seqstart_k=None, window=None,
                window_right=None) -> np.ndarray:
    """Dense additive bias [Mq, Mkv]: 0 where the key is visible, -inf elsewhere."""
    bias = np.full((Mq, Mkv), -np.inf)
    if mask in PACKED:
        sq = list(seqstart_q)
        sk = list(seqstart_k if seqstart_k is not None else seqstart_q)
        for s in range(len(sq) - 1):
            _block(bias, mask, sq[s], sq[s + 1], sk[s], sk[s + 1], window, window_right)
    else:
        _block(bias, mask, 0, Mq, 0, Mkv, window, window_right)
    return bias


def attention(q, k, v, mask: int = MASK_NONE, scale=None, seqstart_q=None, seqstart_k=None, window=None,
              window_right=None):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Mq, H, K = q.shape
    Mkv, Kv = k.shape[1], v.shape[3]
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    bias = materialize(mask, Mq, Mkv, seqstart_q, seqstart_k, window, window_right)
    out = np.zeros((B, Mq, H, Kv))
    lse = np.full((B, H, Mq), -np.inf)
    for b in range(B):
        for h in range(H):
            s = scale * (q[b, :, h, :] @ k[b, :, h, :].T) + bias
            e = np.exp(s)
            tot = e.sum(axis=1)
            nz = tot > 0
            out[b, nz, h, :] = (e[nz] / tot[nz, None]) @ v[b, :, h, :]
            lse[b, h, nz] = np.log(tot[nz])
    return out, lse
