"""fp64 CPU oracle for the attention forward, backward, partial and merge -- TEST INFRASTRUCTURE.

Only ``tests/``, the smoke check and the bench's CPU-baseline leg use this
package.  The HIP product path never imports, links or calls it, and it shares
no code with that path.  ``oracle.c`` holds the definition (see its header for
the passages of the MSLK pages it follows); ``brute.py`` is an independent dense
numpy version with a materialised mask bias, used to cross-check it.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

MASK_NONE, MASK_CAUSAL, MASK_BLOCKDIAG, MASK_BLOCKDIAG_CAUSAL = 0, 1, 2, 3
MASK_CAUSAL_BR, MASK_BLOCKDIAG_CAUSAL_BR, MASK_LOCAL_BR, MASK_CAUSAL_LOCAL_BR = 4, 5, 6, 7
MASK_BLOCKDIAG_CAUSAL_LOCAL, MASK_BLOCKDIAG_CAUSAL_LOCAL_BR = 8, 9
PACKED = (MASK_BLOCKDIAG, MASK_BLOCKDIAG_CAUSAL, MASK_BLOCKDIAG_CAUSAL_BR, MASK_BLOCKDIAG_CAUSAL_LOCAL,
          MASK_BLOCKDIAG_CAUSAL_LOCAL_BR)

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, OpenMP, no fast-math) into liboracle.so."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", SRC, "-o", tmp, "-lm"],
                       check=True)
        os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build(force=True)
        lib = ctypes.CDLL(LIB)
        i64, dp, ip = ctypes.c_int64, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int32)
        lib.oracle_attention.argtypes = [i64, i64, i64, i64, i64, i64, dp, dp, dp, ctypes.c_int, ctypes.c_int,
                                         ip, ip, ctypes.c_double, i64, i64, dp, dp]
        lib.oracle_attention.restype = ctypes.c_int
        lib.oracle_attention_backward.argtypes = [i64, i64, i64, i64, i64, i64, dp, dp, dp, dp, dp, dp, ctypes.c_int,
                                                  ctypes.c_int, ip, ip, ctypes.c_double, i64, i64, dp, dp, dp]
        lib.oracle_attention_backward.restype = ctypes.c_int
        lib.oracle_merge.argtypes = [i64, i64, i64, i64, i64, dp, dp, dp, dp]
        lib.oracle_merge.restype = ctypes.c_int
        lib.oracle_threads.restype = ctypes.c_int
        lib.oracle_fp8_e4m3.argtypes = [ctypes.c_uint8]
        lib.oracle_fp8_e4m3.restype = ctypes.c_double
        lib.oracle_dequant_fp8_rowwise.argtypes = [i64, i64, ctypes.c_void_p, dp, dp]
        lib.oracle_dequant_fp8_rowwise.restype = None
        lib.oracle_dequant_fp8_groupwise.argtypes = [i64, i64, i64, ctypes.c_void_p, dp, dp]
        lib.oracle_dequant_fp8_groupwise.restype = None
        lib.oracle_e8m0.argtypes = [ctypes.c_uint8]
        lib.oracle_e8m0.restype = ctypes.c_double
        lib.oracle_dequant_mxfp8.argtypes = [i64, i64, ctypes.c_void_p, ctypes.c_void_p, dp]
        lib.oracle_dequant_mxfp8.restype = None
        lib.oracle_dequant_int4_groupwise.argtypes = [i64, i64, i64, ctypes.c_void_p, dp, dp]
        lib.oracle_dequant_int4_groupwise.restype = None
        _lib = lib
    return _lib


def _dp(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def threads() -> int:
    return int(_load().oracle_threads())


def attention(q, k, v, mask: int = MASK_NONE, scale=None, seqstart_q=None, seqstart_k=None, window=None,
              window_right=None):
    """Exact attention (fp64).

    q [B,Mq,H,K], k [B,Mkv,H,K], v [B,Mkv,H,Kv] -> (out [B,Mq,H,Kv], lse [B,H,Mq]).
    ``scale`` None means 1/sqrt(K).  Packed-sequence masks take int prefix sums
    (``seqstart_k`` defaults to ``seqstart_q``) and need B == 1.  ``window`` is the
    window size of the causal-local kinds, or the left window of MASK_LOCAL_BR
    (with ``window_right``).
    """
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    B, Mq, H, K = q.shape
    Mkv, Kv = k.shape[1], v.shape[3]
    assert k.shape == (B, Mkv, H, K) and v.shape == (B, Mkv, H, Kv)
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    out = np.empty((B, Mq, H, Kv), dtype=np.float64)
    lse = np.empty((B, H, Mq), dtype=np.float64)
    nseq = 0
    sq = sk = None
    if mask in PACKED:
        sq = np.ascontiguousarray(seqstart_q, dtype=np.int32)
        sk = np.ascontiguousarray(seqstart_k if seqstart_k is not None else seqstart_q, dtype=np.int32)
        nseq = len(sq) - 1
        assert len(sk) == len(sq)
    ip = ctypes.POINTER(ctypes.c_int32)
    rc = _load().oracle_attention(B, Mq, Mkv, H, K, Kv, _dp(q), _dp(k), _dp(v), int(mask), nseq,
                                  sq.ctypes.data_as(ip) if sq is not None else None,
                                  sk.ctypes.data_as(ip) if sk is not None else None,
                                  float(scale), int(window or 0), int(window_right or 0), _dp(out), _dp(lse))
    if rc != 0:
        raise ValueError(f"oracle_attention rejected its arguments (code {rc})")
    return out, lse


def attention_backward(dout, out, lse, q, k, v, mask: int = MASK_NONE, scale=None, seqstart_q=None,
                       seqstart_k=None, window=None, window_right=None):
    """Exact gradients (dq, dk, dv) of the attention for upstream gradient ``dout`` (fp64).

    ``out`` and ``lse`` are the forward's results for the same arguments; the mask
    arguments are those of ``attention``.
    """
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.ascontiguousarray(out, dtype=np.float64)
    lse = np.ascontiguousarray(lse, dtype=np.float64)
    dout = np.ascontiguousarray(dout, dtype=np.float64)
    B, Mq, H, K = q.shape
    Mkv, Kv = k.shape[1], v.shape[3]
    assert k.shape == (B, Mkv, H, K) and v.shape == (B, Mkv, H, Kv)
    assert out.shape == dout.shape == (B, Mq, H, Kv) and lse.shape == (B, H, Mq)
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    nseq = 0
    sq = sk = None
    if mask in PACKED:
        sq = np.ascontiguousarray(seqstart_q, dtype=np.int32)
        sk = np.ascontiguousarray(seqstart_k if seqstart_k is not None else seqstart_q, dtype=np.int32)
        nseq = len(sq) - 1
    ip = ctypes.POINTER(ctypes.c_int32)
    rc = _load().oracle_attention_backward(B, Mq, Mkv, H, K, Kv, _dp(q), _dp(k), _dp(v), _dp(out), _dp(lse),
                                           _dp(dout), int(mask), nseq,
                                           sq.ctypes.data_as(ip) if sq is not None else None,
                                           sk.ctypes.data_as(ip) if sk is not None else None, float(scale),
                                           int(window or 0), int(window_right or 0), _dp(dq), _dp(dk), _dp(dv))
    if rc != 0:
        raise ValueError(f"oracle_attention_backward rejected its arguments (code {rc})")
    return dq, dk, dv


def merge(out_chunks, lse_chunks):
    """Exact LSE-weighted merge of S chunks.

    out_chunks [S,B,M,H,Kv] (or a list of [B,M,H,Kv]), lse_chunks [S,B,H,M]
    -> (out [B,M,H,Kv], lse [B,H,M]).
    """
    oc = np.ascontiguousarray(np.stack(out_chunks) if isinstance(out_chunks, (list, tuple)) else out_chunks,
                              dtype=np.float64)
    lc = np.ascontiguousarray(np.stack(lse_chunks) if isinstance(lse_chunks, (list, tuple)) else lse_chunks,
                              dtype=np.float64)
    S, B, M, H, Kv = oc.shape
    assert lc.shape == (S, B, H, M)
    out = np.empty((B, M, H, Kv), dtype=np.float64)
    lse = np.empty((B, H, M), dtype=np.float64)
    rc = _load().oracle_merge(S, B, M, H, Kv, _dp(oc), _dp(lc), _dp(out), _dp(lse))
    if rc != 0:
        raise ValueError(f"oracle_merge rejected its arguments (code {rc})")
    return out, lse


def partial(q, k, v, j0: int, j1: int, mask: int = MASK_NONE, scale=None):
    """Attention over the key shard [j0, j1) alone (the shard is its own key sequence)."""
    return attention(q, k[:, j0:j1], v[:, j0:j1], mask=mask,
                     scale=(1.0 / math.sqrt(q.shape[3])) if scale is None else scale)


def fp8_e4m3(code: int) -> float:
    """Value of one FP8 E4M3 code (OCP FN variant)."""
    return float(_load().oracle_fp8_e4m3(int(code) & 0xFF))


def dequant_fp8_rowwise(codes, scale_shift):
    """codes uint8 [..., D], scale_shift [..., 2] -> fp64 [..., D] = fp8(code) * scale + shift."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    ss = np.ascontiguousarray(scale_shift, dtype=np.float64)
    assert ss.shape == codes.shape[:-1] + (2,)
    D = codes.shape[-1]
    rows = codes.size // D if D else 0
    x = np.empty(codes.shape, dtype=np.float64)
    _load().oracle_dequant_fp8_rowwise(rows, D, codes.ctypes.data, _dp(ss), _dp(x))
    return x


def dequant_fp8_groupwise(codes, scale_shift):
    """codes uint8 [..., D] (E4M3), scale_shift [..., G, 2] -> fp64 [..., D] = fp8(code) * scale +
    shift of the element's group (D/G consecutive elements per group)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    ss = np.ascontiguousarray(scale_shift, dtype=np.float64)
    G = ss.shape[-2]
    D = codes.shape[-1]
    assert ss.shape == codes.shape[:-1] + (G, 2) and D % G == 0
    rows = codes.size // D if D else 0
    x = np.empty(codes.shape, dtype=np.float64)
    _load().oracle_dequant_fp8_groupwise(rows, D, G, codes.ctypes.data, _dp(ss), _dp(x))
    return x


def e8m0(e: int) -> float:
    """Value of one E8M0 block scale: 2^(e - 127), NaN for 255."""
    return float(_load().oracle_e8m0(int(e) & 0xFF))


def dequant_mxfp8(codes, scales):
    """codes uint8 [..., D] (E4M3), scales uint8 [..., D/32] (E8M0, one per block of 32 elements)
    -> fp64 [..., D] = fp8(code) * 2^(e - 127)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    sc = np.ascontiguousarray(scales, dtype=np.uint8)
    D = codes.shape[-1]
    assert D % 32 == 0 and sc.shape == codes.shape[:-1] + (D // 32,)
    rows = codes.size // D if D else 0
    x = np.empty(codes.shape, dtype=np.float64)
    _load().oracle_dequant_mxfp8(rows, D, codes.ctypes.data, sc.ctypes.data, _dp(x))
    return x


def dequant_int4_groupwise(codes, scale_shift):
    """codes uint8 [..., D/2] (two 4-bit codes per byte, even element low), scale_shift [..., G, 2]
    -> fp64 [..., D] = code * scale + shift of the element's group."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    ss = np.ascontiguousarray(scale_shift, dtype=np.float64)
    G = ss.shape[-2]
    D = 2 * codes.shape[-1]
    assert ss.shape == codes.shape[:-1] + (G, 2) and D % G == 0
    rows = codes.size // (D // 2) if D else 0
    x = np.empty(codes.shape[:-1] + (D,), dtype=np.float64)
    _load().oracle_dequant_int4_groupwise(rows, D, G, codes.ctypes.data, _dp(ss), _dp(x))
    return x


def chunk_bounds(Mkv: int, S: int):
    """Equal contiguous chunks: chunk s covers [s*c, min(Mkv, (s+1)*c)) with c = ceil(Mkv/S)."""
    c = -(-Mkv // S)
    return [(min(Mkv, s * c), min(Mkv, (s + 1) * c)) for s in range(S)]
