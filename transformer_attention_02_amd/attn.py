"""ctypes binding of libattn.so: argument marshalling only.

Each function has the name of the C entry point it calls (include/attn.h) and
turns torch tensors into the C descriptors (pointer, dtype, shape, strides in
elements) plus the current HIP stream.  Torch is used for device memory and
streams only; every step of the computation runs in the library's HIP kernels.
Outputs that the caller does not pass are allocated with ``torch.empty``.

Importing this module loads the library and raises ImportError if it is
missing: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn.so")

ATTN_OK, ATTN_ERR_INVALID_ARGUMENT, ATTN_ERR_UNSUPPORTED, ATTN_ERR_WORKSPACE_TOO_SMALL, ATTN_ERR_LAUNCH = range(5)
ATTN_DTYPE_F32, ATTN_DTYPE_BF16, ATTN_DTYPE_FP8_E4M3, ATTN_DTYPE_F16, ATTN_DTYPE_INT4X2, ATTN_DTYPE_E8M0 = range(6)
MASK_NONE, MASK_CAUSAL, MASK_BLOCKDIAG, MASK_BLOCKDIAG_CAUSAL = 0, 1, 2, 3
MASK_CAUSAL_BR, MASK_BLOCKDIAG_CAUSAL_BR, MASK_LOCAL_BR, MASK_CAUSAL_LOCAL_BR = 4, 5, 6, 7
MASK_BLOCKDIAG_CAUSAL_LOCAL, MASK_BLOCKDIAG_CAUSAL_LOCAL_BR = 8, 9
WINDOWED = (MASK_LOCAL_BR, MASK_CAUSAL_LOCAL_BR, MASK_BLOCKDIAG_CAUSAL_LOCAL, MASK_BLOCKDIAG_CAUSAL_LOCAL_BR)
MAX_CHUNKS = 128

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m transformer_attention_02_amd.build`")
_lib = ctypes.CDLL(LIB_PATH)


class AttnTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 5), ("stride", ctypes.c_int64 * 5)]


class AttnMask(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("window_size", ctypes.c_int32), ("window_left", ctypes.c_int32),
                ("window_right", ctypes.c_int32)]


class AttnVarlen(ctypes.Structure):
    _fields_ = [("seqstart_q", ctypes.c_void_p), ("seqstart_k", ctypes.c_void_p), ("nseq", ctypes.c_int32),
                ("max_seqlen_q", ctypes.c_int32), ("max_seqlen_k", ctypes.c_int32)]


_P = ctypes.POINTER
_T = _P(AttnTensor)
_lib.attn_fwd.argtypes = [_T, _T, _T, ctypes.c_int32, _P(AttnVarlen), ctypes.c_float, _T, ctypes.c_void_p,
                          ctypes.c_void_p]
_lib.attn_fwd.restype = ctypes.c_int
_lib.attn_partial.argtypes = _lib.attn_fwd.argtypes
_lib.attn_partial.restype = ctypes.c_int
_lib.attn_fwd_ex.argtypes = [_T, _T, _T, _P(AttnMask), _P(AttnVarlen), ctypes.c_float, _T, ctypes.c_void_p,
                             ctypes.c_void_p]
_lib.attn_fwd_ex.restype = ctypes.c_int
_lib.attn_partial_ex.argtypes = _lib.attn_fwd_ex.argtypes
_lib.attn_partial_ex.restype = ctypes.c_int
_lib.attn_merge.argtypes = [ctypes.c_int32, _T, _P(ctypes.c_void_p), _T, ctypes.c_void_p, ctypes.c_void_p]
_lib.attn_merge.restype = ctypes.c_int
_lib.attn_fwd_kvcache.argtypes = [_T, _T, _T, _P(AttnMask), ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t, _T,
                                   ctypes.c_void_p, ctypes.c_void_p]
_lib.attn_fwd_kvcache.restype = ctypes.c_int
_lib.attn_fwd_kvcache_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32]
_lib.attn_fwd_kvcache_workspace_bytes.restype = ctypes.c_size_t
_lib.attn_decode_num_splits.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]
_lib.attn_decode_num_splits.restype = ctypes.c_int32
_lib.attn_decode_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32]
_lib.attn_decode_workspace_bytes.restype = ctypes.c_size_t
_lib.attn_decode_splitkv.argtypes = [_T, _T, _T, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t,
                                     _T, ctypes.c_void_p, ctypes.c_void_p]
_lib.attn_decode_splitkv.restype = ctypes.c_int
_lib.attn_decode_splitkv_noalloc.argtypes = [_T, _T, _T, ctypes.c_int32, ctypes.c_float, _T, ctypes.c_void_p,
                                              ctypes.c_void_p]
_lib.attn_decode_splitkv_noalloc.restype = ctypes.c_int
_lib.attn_decode_splitkv_paged.argtypes = [_T, _T, _T, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t, _T, ctypes.c_void_p,
                                           ctypes.c_void_p]
_lib.attn_decode_splitkv_paged.restype = ctypes.c_int
_lib.attn_decode_splitkv_fp8.argtypes = [_T, _T, _T, _T, _T, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t, _T, ctypes.c_void_p,
                                         ctypes.c_void_p]
_lib.attn_decode_splitkv_fp8.restype = ctypes.c_int
_lib.attn_decode_splitkv_int4.argtypes = _lib.attn_decode_splitkv_fp8.argtypes
_lib.attn_decode_splitkv_int4.restype = ctypes.c_int
_lib.attn_decode_splitkv_mxfp8.argtypes = _lib.attn_decode_splitkv_fp8.argtypes
_lib.attn_decode_splitkv_mxfp8.restype = ctypes.c_int
_lib.attn_bwd_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]
_lib.attn_bwd_workspace_bytes.restype = ctypes.c_size_t
_lib.attn_bwd_ds_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]
_lib.attn_bwd_ds_workspace_bytes.restype = ctypes.c_size_t
_lib.attn_bwd.argtypes = [_T, _T, _T, _T, _T, ctypes.c_void_p, _P(AttnMask), _P(AttnVarlen), ctypes.c_float,
                          ctypes.c_void_p, ctypes.c_size_t, _T, _T, _T, ctypes.c_void_p]
_lib.attn_bwd.restype = ctypes.c_int
_lib.attn_last_error.argtypes = []
_lib.attn_last_error.restype = ctypes.c_char_p


class AttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"status {status}: {msg}")
        self.status = status


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return ATTN_DTYPE_F32
    if dt == torch.bfloat16:
        return ATTN_DTYPE_BF16
    if dt == torch.float8_e4m3fn:
        return ATTN_DTYPE_FP8_E4M3
    if dt == torch.float16:
        return ATTN_DTYPE_F16
    if dt == torch.float8_e8m0fnu:
        return ATTN_DTYPE_E8M0
    raise TypeError(f"unsupported dtype {dt}")


def _dev(t, name: str):
    """The kernels dereference every pointer on the GPU: host tensors are refused here."""
    if t is not None and t.numel() and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor, got one on {t.device}")
    return t


def _index(t, name: str):
    """Sequence offsets, lengths and block tables: int32 and contiguous (the device check comes
    with the other tensors')."""
    if t is None:
        return None
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _lse_buf(lse, rows: int, name: str = "lse"):
    """A caller's LSE array ([B, H_total, M] fp32, contiguous) with room for the `rows` values a call
    reads or writes."""
    if lse is None:
        return None
    if lse.dtype != torch.float32:
        raise TypeError(f"{name} must be float32, got {lse.dtype}")
    if not lse.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if lse.numel() < rows:
        raise ValueError(f"{name} holds {lse.numel()} values; the call needs {rows}")
    return lse


def _on_device(**tensors) -> None:
    for name, t in tensors.items():
        _dev(t, name)


def _ws_bytes(workspace) -> int:
    _dev(workspace, "workspace")
    return workspace.numel() * workspace.element_size()


def desc(t: torch.Tensor, dtype_code=None, name: str = "tensor") -> AttnTensor:
    """C descriptor of a 4-D [B,M,H,D] or 5-D [B,M,G,H,D] tensor (strides in elements); `dtype_code`
    overrides the code derived from the torch dtype (uint8 INT4 caches are ATTN_DTYPE_INT4X2)."""
    _dev(t, name)
    d = AttnTensor()
    d.data = t.data_ptr() if t.numel() else None
    d.dtype = _dtype_code(t.dtype) if dtype_code is None else dtype_code
    d.ndim = t.dim()
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def _stream(stream, device=None) -> ctypes.c_void_p:
    """The caller's stream, else the current stream of the tensors' device."""
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(rc: int) -> None:
    if rc != ATTN_OK:
        raise AttnError(rc, attn_last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _scale(scale) -> float:
    return float("nan") if scale is None else float(scale)


def _htot(t: torch.Tensor) -> int:
    return t.shape[2] * t.shape[3] if t.dim() == 5 else t.shape[2]


def _varlen(seqstart_q, seqstart_k, max_seqlen_q, max_seqlen_k=None):
    if seqstart_q is None:
        return None, None
    _index(seqstart_q, "seqstart_q")
    _index(seqstart_k, "seqstart_k")
    if seqstart_k is not None and seqstart_k.numel() != seqstart_q.numel():
        # the kernels read seqstart_k[s + 1] for every sequence s of seqstart_q
        raise ValueError(f"seqstart_k has {seqstart_k.numel()} entries; seqstart_q has {seqstart_q.numel()}")
    vl = AttnVarlen()
    vl.seqstart_q = seqstart_q.data_ptr()
    vl.seqstart_k = seqstart_k.data_ptr() if seqstart_k is not None else None
    vl.nseq = seqstart_q.numel() - 1
    vl.max_seqlen_q = int(max_seqlen_q)
    vl.max_seqlen_k = int(max_seqlen_k or 0)
    return ctypes.byref(vl), vl


def attn_last_error() -> str:
    return _lib.attn_last_error().decode()


def _mask_arg(mask, window_size, window_left, window_right, partial):
    """(C function, mask argument): the plain entry point for kinds without windows, _ex otherwise."""
    if mask in WINDOWED or window_size is not None or window_left is not None or window_right is not None:
        m = AttnMask(int(mask), int(window_size or 0), int(window_left or 0), int(window_right or 0))
        return (_lib.attn_partial_ex if partial else _lib.attn_fwd_ex), m, ctypes.byref(m)
    return (_lib.attn_partial if partial else _lib.attn_fwd), None, int(mask)


def _forward(fn, q, k, v, mask, scale, seqstart_q, seqstart_k, max_seqlen_q, out, lse, stream, out_dtype):
    if out is None:
        out = torch.empty((*q.shape[:-1], v.shape[-1]), dtype=out_dtype, device=q.device)
    if lse is True:
        lse = torch.empty((q.shape[0], _htot(q), q.shape[1]), dtype=torch.float32, device=q.device)
    elif lse is False:
        lse = None
    vref, _keep = _varlen(seqstart_q, seqstart_k, max_seqlen_q)
    _lse_buf(lse, q.shape[0] * _htot(q) * q.shape[1])
    _on_device(seqstart_q=seqstart_q, seqstart_k=seqstart_k, lse=lse)
    dq, dk, dv, do = desc(q, name="q"), desc(k, name="k"), desc(v, name="v"), desc(out, name="out")
    cfn, _m, marg = _mask_arg(mask[0], *mask[1:], partial=fn == "partial")
    _check(cfn(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), marg, vref, _scale(scale),
               ctypes.byref(do), _ptr(lse), _stream(stream, q.device)))
    return out, lse


class Prepared:
    """A call of one C entry point with its arguments marshalled once.

    Calling the object re-issues the same C call (same tensors, same stream) with
    no per-call Python work beyond the ctypes call itself; the tensors it was
    built from are kept alive by the object.
    """

    def __init__(self, fn, args, keep):
        self._fn, self._args, self._keep = fn, args, keep

    def __call__(self):
        _check(self._fn(*self._args))


def prepare_fwd(q, k, v, out, lse, mask=MASK_NONE, scale=None, seqstart_q=None, seqstart_k=None,
                max_seqlen_q=None, partial=False, stream=None, window_size=None, window_left=None,
                window_right=None) -> Prepared:
    """attn_fwd (or attn_partial, or their _ex forms for windowed masks) marshalled up front."""
    vref, vl = _varlen(seqstart_q, seqstart_k, max_seqlen_q)
    _lse_buf(lse, q.shape[0] * _htot(q) * q.shape[1])
    _on_device(seqstart_q=seqstart_q, seqstart_k=seqstart_k, lse=lse)
    ds = [desc(q, name="q"), desc(k, name="k"), desc(v, name="v"), desc(out, name="out")]
    cfn, m, marg = _mask_arg(mask, window_size, window_left, window_right, partial)
    args = (ctypes.byref(ds[0]), ctypes.byref(ds[1]), ctypes.byref(ds[2]), marg, vref, _scale(scale),
            ctypes.byref(ds[3]), _ptr(lse), _stream(stream, q.device))
    return Prepared(cfn, args, (ds, vl, m, q, k, v, out, lse))


def prepare_decode(q, k, v, num_splits, workspace, out, lse, scale=None, stream=None) -> Prepared:
    """attn_decode_splitkv with every argument marshalled up front."""
    _on_device(lse=_lse_buf(lse, q.shape[0] * _htot(q)))
    ds = [desc(q, name="q"), desc(k, name="k"), desc(v, name="v"), desc(out, name="out")]
    args = (ctypes.byref(ds[0]), ctypes.byref(ds[1]), ctypes.byref(ds[2]), int(num_splits), _scale(scale),
            _ptr(workspace), _ws_bytes(workspace), ctypes.byref(ds[3]), _ptr(lse), _stream(stream, q.device))
    return Prepared(_lib.attn_decode_splitkv, args, (ds, q, k, v, workspace, out, lse))


def _merge_lses(chunks, lses, lse_out, out):
    if len(chunks) != len(lses):
        raise ValueError("out_chunks and lse_chunks differ in length")
    if not chunks:
        return
    rows = chunks[0].shape[0] * _htot(chunks[0]) * chunks[0].shape[1]
    for i, x in enumerate(lses):
        _lse_buf(x, rows, f"lse_chunks[{i}]")
    _lse_buf(lse_out, rows, "lse")
    _on_device(lse=lse_out, **{f"lse_chunks[{i}]": x for i, x in enumerate(lses)})


def prepare_merge(out_chunks, lse_chunks, out, lse=None, stream=None) -> Prepared:
    """attn_merge with every argument marshalled up front."""
    chunks = list(out_chunks.unbind(0)) if isinstance(out_chunks, torch.Tensor) else list(out_chunks)
    lses = list(lse_chunks.unbind(0)) if isinstance(lse_chunks, torch.Tensor) else list(lse_chunks)
    n = len(chunks)
    _merge_lses(chunks, lses, lse, out)
    descs = (AttnTensor * max(1, n))(*[desc(c, name=f"out_chunks[{i}]") for i, c in enumerate(chunks)])
    lptrs = (ctypes.c_void_p * max(1, n))(*[x.data_ptr() for x in lses])
    do = desc(out, name="out")
    args = (n, descs, lptrs, ctypes.byref(do), _ptr(lse), _stream(stream, out.device))
    return Prepared(_lib.attn_merge, args, (descs, lptrs, do, chunks, lses, out, lse))


def attn_fwd(q, k, v, mask=MASK_NONE, scale=None, seqstart_q=None, seqstart_k=None, max_seqlen_q=None,
             out=None, lse=True, stream=None, window_size=None, window_left=None, window_right=None):
    """memory_efficient_attention_forward_requires_grad: returns (out, lse); lse=False skips the LSE.

    Windowed masks take window_size (kinds 7-9) or window_left/window_right (kind 6) and go
    through attn_fwd_ex."""
    return _forward("fwd", q, k, v, (mask, window_size, window_left, window_right), scale, seqstart_q, seqstart_k,
                    max_seqlen_q, out, lse, stream, q.dtype)


def attn_partial(q, k, v, mask=MASK_NONE, scale=None, seqstart_q=None, seqstart_k=None, max_seqlen_q=None,
                 out=None, lse=True, stream=None, out_dtype=torch.float32, window_size=None, window_left=None,
                 window_right=None):
    """memory_efficient_attention_partial over the shard (k, v): returns (out fp32 by default, lse)."""
    return _forward("partial", q, k, v, (mask, window_size, window_left, window_right), scale, seqstart_q,
                    seqstart_k, max_seqlen_q, out, lse, stream, out_dtype)


def attn_merge(out_chunks, lse_chunks, out=None, write_lse=True, out_dtype=None, stream=None):
    """merge_attentions over a list of chunks (or a stacked [S, ...] tensor): returns (out, lse or None)."""
    chunks = list(out_chunks.unbind(0)) if isinstance(out_chunks, torch.Tensor) else list(out_chunks)
    lses = list(lse_chunks.unbind(0)) if isinstance(lse_chunks, torch.Tensor) else list(lse_chunks)
    n = len(chunks)
    c0 = chunks[0] if n else None
    if out is None and c0 is not None:
        out = torch.empty(c0.shape, dtype=out_dtype or c0.dtype, device=c0.device)
    lse = None
    if write_lse and c0 is not None:
        lse = torch.empty((c0.shape[0], _htot(c0), c0.shape[1]), dtype=torch.float32, device=c0.device)
    _merge_lses(chunks, lses, lse, out)
    descs = (AttnTensor * max(1, n))(*[desc(c, name=f"out_chunks[{i}]") for i, c in enumerate(chunks)])
    lptrs = (ctypes.c_void_p * max(1, n))(*[x.data_ptr() for x in lses])
    _check(_lib.attn_merge(n, descs, lptrs, ctypes.byref(desc(out, name="out")) if out is not None else None,
                           _ptr(lse), _stream(stream, out.device if out is not None else None)))
    return out, lse


def attn_decode_workspace_bytes(B: int, H_total: int, Kv: int, num_splits: int) -> int:
    return int(_lib.attn_decode_workspace_bytes(B, H_total, Kv, num_splits))


def attn_decode_num_splits(B: int, H_total: int, Mkv: int) -> int:
    """The library's split count for a decode of B x H_total rows over Mkv keys."""
    return int(_lib.attn_decode_num_splits(int(B), int(H_total), int(Mkv)))


def attn_decode_splitkv(q, k, v, num_splits, scale=None, workspace=None, out=None, lse=True, stream=None):
    """Split-KV decode for q [B,1,(G,)H,K]: returns (out, lse or None).  num_splits None: the
    library's choice (attn_decode_num_splits)."""
    if num_splits is None:
        num_splits = attn_decode_num_splits(q.shape[0], _htot(q), k.shape[1])
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    if lse is True:
        lse = torch.empty((q.shape[0], _htot(q), 1), dtype=torch.float32, device=q.device)
    elif lse is False:
        lse = None
    need = attn_decode_workspace_bytes(q.shape[0], _htot(q), q.shape[-1], num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _on_device(lse=_lse_buf(lse, q.shape[0] * _htot(q)))
    _check(_lib.attn_decode_splitkv(ctypes.byref(desc(q, name="q")), ctypes.byref(desc(k, name="k")),
                                    ctypes.byref(desc(v, name="v")), int(num_splits), _scale(scale),
                                    _ptr(workspace), _ws_bytes(workspace), ctypes.byref(desc(out, name="out")),
                                    _ptr(lse), _stream(stream, q.device)))
    return out, lse


def attn_fwd_kvcache_workspace_bytes(Mq: int, H_total: int, Kv: int, num_splits: int) -> int:
    return int(_lib.attn_fwd_kvcache_workspace_bytes(int(Mq), int(H_total), int(Kv), int(num_splits)))


def _kvcache_args(q, k, v, seqstart_q, seqlens_k, max_seqlen_q, max_seqlen_k, mask, window_size, window_left,
                  window_right, block_tables, page_size, num_splits, scale, workspace, out, lse, stream, seqstart_k=None):
    _index(seqstart_q, "seqstart_q")
    if seqlens_k is None:
        raise ValueError("seqlens_k is required")
    _cache_index(q, seqlens_k, block_tables, "sequences", B=seqstart_q.numel() - 1)
    _index(seqstart_k, "seqstart_k")
    if seqstart_k is not None and seqstart_k.numel() < seqstart_q.numel() - 1:
        raise ValueError(f"seqstart_k holds {seqstart_k.numel()} values; there are {seqstart_q.numel() - 1} sequences")
    _lse_buf(lse, _htot(q) * q.shape[1])
    _on_device(seqstart_q=seqstart_q, seqlens_k=seqlens_k, block_tables=block_tables, lse=lse, workspace=workspace,
               seqstart_k=seqstart_k)
    m = AttnMask(int(mask), int(window_size or 0), int(window_left or 0), int(window_right or 0))
    ds = [desc(q, name="q"), desc(k, name="k"), desc(v, name="v"), desc(out, name="out")]
    mb = block_tables.shape[1] if block_tables is not None else 0
    args = (ctypes.byref(ds[0]), ctypes.byref(ds[1]), ctypes.byref(ds[2]), ctypes.byref(m), _ptr(seqstart_q),
            int(seqstart_q.numel() - 1), int(max_seqlen_q), _ptr(seqstart_k), _ptr(seqlens_k), _ptr(block_tables), int(mb),
            int(page_size or 0), int(max_seqlen_k), int(num_splits), _scale(scale), _ptr(workspace),
            _ws_bytes(workspace) if workspace is not None else 0, ctypes.byref(ds[3]), _ptr(lse),
            _stream(stream, q.device))
    return args, (ds, m)


def attn_fwd_kvcache(q, k, v, seqstart_q, seqlens_k, max_seqlen_q, max_seqlen_k, mask=MASK_NONE, window_size=None,
                     window_left=None, window_right=None, block_tables=None, page_size=None, num_splits=1,
                     scale=None, workspace=None, out=None, lse=True, stream=None, seqstart_k=None):
    """Packed query blocks [1, Mq, (G,) H, K] against padded KV lanes (block_tables None), a paged
    cache, or gappy lanes (seqstart_k: each sequence's first row of one k/v tensor), with the
    padded-keys masks aligned from the bottom right of each sequence (MASK_NONE, MASK_CAUSAL_BR,
    MASK_LOCAL_BR, MASK_CAUSAL_LOCAL_BR).  Returns (out, lse or None)."""
    if out is None:
        out = torch.empty((*q.shape[:-1], v.shape[-1]), dtype=q.dtype, device=q.device)
    if lse is True:
        lse = torch.empty((1, _htot(q), q.shape[1]), dtype=torch.float32, device=q.device)
    elif lse is False:
        lse = None
    if workspace is None and num_splits > 1:
        need = attn_fwd_kvcache_workspace_bytes(q.shape[1], _htot(q), v.shape[-1], num_splits)
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    args, _keep = _kvcache_args(q, k, v, seqstart_q, seqlens_k, max_seqlen_q, max_seqlen_k, mask, window_size,
                                window_left, window_right, block_tables, page_size, num_splits, scale, workspace, out,
                                lse, stream, seqstart_k)
    _check(_lib.attn_fwd_kvcache(*args))
    return out, lse


def prepare_fwd_kvcache(q, k, v, seqstart_q, seqlens_k, max_seqlen_q, max_seqlen_k, out, lse, mask=MASK_NONE,
                        window_size=None, window_left=None, window_right=None, block_tables=None, page_size=None,
                        num_splits=1, scale=None, workspace=None, stream=None, seqstart_k=None) -> Prepared:
    """attn_fwd_kvcache with every argument marshalled up front."""
    args, keep = _kvcache_args(q, k, v, seqstart_q, seqlens_k, max_seqlen_q, max_seqlen_k, mask, window_size,
                               window_left, window_right, block_tables, page_size, num_splits, scale, workspace, out,
                               lse, stream, seqstart_k)
    return Prepared(_lib.attn_fwd_kvcache, args, (keep, q, k, v, seqstart_q, seqlens_k, block_tables, workspace, out,
                                                   lse, seqstart_k))


NOALLOC_SCRATCH_BYTES = 32 << 20  # ATTN_NOALLOC_SCRATCH_BYTES


def attn_decode_splitkv_noalloc(q, k, v, num_splits, out, lse=None, scale=None, stream=None):
    """attn_decode_splitkv without a workspace: the partials live in the library's static per-GPU
    scratch.  The caller passes `out` (and `lse` [B, H_total, 1] fp32, or None), so that nothing is
    allocated here either.  Calls that may overlap on one GPU share that scratch and race."""
    _on_device(lse=_lse_buf(lse, q.shape[0] * _htot(q)))
    _check(_lib.attn_decode_splitkv_noalloc(ctypes.byref(desc(q, name="q")), ctypes.byref(desc(k, name="k")),
                                            ctypes.byref(desc(v, name="v")), int(num_splits), _scale(scale),
                                            ctypes.byref(desc(out, name="out")), _ptr(lse),
                                            _stream(stream, q.device)))
    return out, lse


def _cache_index(q, seqlens, block_tables, what="batch elements", B=None):
    """seqlens [>= B] and block_tables [>= B, n] int32: the kernels read seqlens[b] and row b of the
    table for every batch element b of q (or every sequence b of B)."""
    _index(seqlens, "seqlens")
    _index(block_tables, "block_tables")
    B = q.shape[0] if B is None else B
    if seqlens is not None and seqlens.numel() < B:
        raise ValueError(f"seqlens holds {seqlens.numel()} values; q has {B} {what}")
    if block_tables is not None and (block_tables.dim() != 2 or block_tables.shape[0] < B):
        raise ValueError(f"block_tables must be 2-D with at least {B} rows, got shape {tuple(block_tables.shape)}")


def _paged_args(q, k, v, seqlens, block_tables, page_size, max_seqlen_k, num_splits, scale, workspace, out, lse,
                stream, window_size=None):
    _cache_index(q, seqlens, block_tables)
    _lse_buf(lse, q.shape[0] * _htot(q))
    _on_device(seqlens=seqlens, block_tables=block_tables, lse=lse)
    ds = [desc(q, name="q"), desc(k, name="k"), desc(v, name="v"), desc(out, name="out")]
    mb = block_tables.shape[1] if block_tables is not None else 0
    args = (ctypes.byref(ds[0]), ctypes.byref(ds[1]), ctypes.byref(ds[2]), _ptr(seqlens), _ptr(block_tables),
            int(mb), int(page_size or 0), int(max_seqlen_k), int(window_size or 0), int(num_splits), _scale(scale),
            _ptr(workspace), _ws_bytes(workspace), ctypes.byref(ds[3]), _ptr(lse), _stream(stream, q.device))
    return args, ds


def attn_decode_splitkv_paged(q, k, v, seqlens, num_splits, max_seqlen_k, block_tables=None, page_size=None,
                              scale=None, workspace=None, out=None, lse=True, stream=None, window_size=None):
    """Split-KV decode against padded lanes (block_tables None) or a paged cache: returns (out, lse or None).
    num_splits None: the library's choice for max_seqlen_k keys (or the window's).  window_size W: the
    query sees only its sequence's last W keys."""
    if num_splits is None:
        num_splits = attn_decode_num_splits(q.shape[0], _htot(q), min(max_seqlen_k, window_size or max_seqlen_k))
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    if lse is True:
        lse = torch.empty((q.shape[0], _htot(q), 1), dtype=torch.float32, device=q.device)
    elif lse is False:
        lse = None
    need = attn_decode_workspace_bytes(q.shape[0], _htot(q), q.shape[-1], num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    args, _keep = _paged_args(q, k, v, seqlens, block_tables, page_size, max_seqlen_k, num_splits, scale, workspace,
                              out, lse, stream, window_size)
    _check(_lib.attn_decode_splitkv_paged(*args))
    return out, lse


def prepare_decode_paged(q, k, v, seqlens, num_splits, max_seqlen_k, workspace, out, lse, block_tables=None,
                         page_size=None, scale=None, stream=None, window_size=None) -> Prepared:
    """attn_decode_splitkv_paged with every argument marshalled up front."""
    args, ds = _paged_args(q, k, v, seqlens, block_tables, page_size, max_seqlen_k, num_splits, scale, workspace,
                           out, lse, stream, window_size)
    return Prepared(_lib.attn_decode_splitkv_paged, args, (ds, q, k, v, seqlens, block_tables, workspace, out, lse))


def _fp8_args(q, k, v, k_scale_shift, v_scale_shift, seqlens, block_tables, page_size, max_seqlen_k, num_splits,
              scale, workspace, out, lse, stream, kv_code=None, window_size=None):
    _cache_index(q, seqlens, block_tables)
    _lse_buf(lse, q.shape[0] * _htot(q))
    _on_device(seqlens=seqlens, block_tables=block_tables, lse=lse)
    ds = [desc(q, name="q"), desc(k, kv_code, "k"), desc(v, kv_code, "v"), desc(k_scale_shift, name="k_scale_shift"),
          desc(v_scale_shift, name="v_scale_shift"), desc(out, name="out")]
    mb = block_tables.shape[1] if block_tables is not None else 0
    args = (ctypes.byref(ds[0]), ctypes.byref(ds[1]), ctypes.byref(ds[2]), ctypes.byref(ds[3]), ctypes.byref(ds[4]),
            _ptr(seqlens), _ptr(block_tables), int(mb), int(page_size or 0), int(max_seqlen_k or 0),
            int(window_size or 0), int(num_splits), _scale(scale), _ptr(workspace), _ws_bytes(workspace),
            ctypes.byref(ds[5]), _ptr(lse), _stream(stream, q.device))
    return args, ds


def attn_decode_splitkv_fp8(q, k, v, k_scale_shift, v_scale_shift, num_splits, seqlens=None, max_seqlen_k=None,
                            block_tables=None, page_size=None, scale=None, workspace=None, out=None, lse=True,
                            out_dtype=None, stream=None, window_size=None):
    """Split-KV decode over FP8 E4M3 K/V caches (torch.float8_e4m3fn) with float16 (or float32:
    use_fp32_scales) (scale, shift) pairs [..., 2G] per cache row, head and group; lanes, padded
    lanes (seqlens) or pages (block_tables).  Returns (out, lse or None)."""
    if num_splits is None:  # the library's choice for the keys a sequence may hold
        num_splits = attn_decode_num_splits(q.shape[0], _htot(q), max_seqlen_k or k.shape[1])
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    if lse is True:
        lse = torch.empty((q.shape[0], _htot(q), 1), dtype=torch.float32, device=q.device)
    elif lse is False:
        lse = None
    need = attn_decode_workspace_bytes(q.shape[0], _htot(q), q.shape[-1], num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    args, _keep = _fp8_args(q, k, v, k_scale_shift, v_scale_shift, seqlens, block_tables, page_size, max_seqlen_k,
                            num_splits, scale, workspace, out, lse, stream, window_size=window_size)
    _check(_lib.attn_decode_splitkv_fp8(*args))
    return out, lse


def prepare_decode_fp8(q, k, v, k_scale_shift, v_scale_shift, num_splits, workspace, out, lse, seqlens=None,
                       max_seqlen_k=None, block_tables=None, page_size=None, scale=None, stream=None,
                       window_size=None) -> Prepared:
    """attn_decode_splitkv_fp8 with every argument marshalled up front."""
    args, ds = _fp8_args(q, k, v, k_scale_shift, v_scale_shift, seqlens, block_tables, page_size, max_seqlen_k,
                         num_splits, scale, workspace, out, lse, stream, window_size=window_size)
    return Prepared(_lib.attn_decode_splitkv_fp8, args,
                    (ds, q, k, v, k_scale_shift, v_scale_shift, seqlens, block_tables, workspace, out, lse))


def attn_bwd_workspace_bytes(B: int, H_total: int, Mq: int) -> int:
    return int(_lib.attn_bwd_workspace_bytes(B, H_total, Mq))


def attn_bwd_ds_workspace_bytes(B: int, H_total: int, Mq: int, Mkv: int) -> int:
    return int(_lib.attn_bwd_ds_workspace_bytes(B, H_total, Mq, Mkv))


# largest kept-dS workspace the binding allocates by itself
KEEP_DS_MAX_BYTES = 8 << 30


def _bwd_args(dout, q, k, v, out, lse, mask, scale, seqstart_q, seqstart_k, max_seqlen_q, max_seqlen_k,
              window_size, window_left, window_right, workspace, dq, dk, dv, stream):
    _lse_buf(lse, q.shape[0] * _htot(q) * q.shape[1])
    vref, vl = _varlen(seqstart_q, seqstart_k, max_seqlen_q, max_seqlen_k)
    _on_device(lse=lse, seqstart_q=seqstart_q, seqstart_k=seqstart_k)
    m = AttnMask(int(mask), int(window_size or 0), int(window_left or 0), int(window_right or 0))
    ds = [desc(x, name=n) for x, n in ((dout, "dout"), (q, "q"), (k, "k"), (v, "v"), (out, "out"), (dq, "dq"),
                                        (dk, "dk"), (dv, "dv"))]
    args = (ctypes.byref(ds[0]), ctypes.byref(ds[1]), ctypes.byref(ds[2]), ctypes.byref(ds[3]), ctypes.byref(ds[4]),
            _ptr(lse), ctypes.byref(m), vref, _scale(scale), _ptr(workspace), _ws_bytes(workspace),
            ctypes.byref(ds[5]), ctypes.byref(ds[6]), ctypes.byref(ds[7]), _stream(stream, q.device))
    return args, (ds, vl, m)


def attn_bwd(dout, q, k, v, out, lse, mask=MASK_NONE, scale=None, seqstart_q=None, seqstart_k=None,
             max_seqlen_q=None, max_seqlen_k=None, window_size=None, window_left=None, window_right=None,
             dq=None, dk=None, dv=None, workspace=None, stream=None, keep_ds=None):
    """memory_efficient_attention_backward: returns (dq, dk, dv) for the forward of the same arguments.
    keep_ds (bf16 at head dim 128 without a block-diagonal mask, workspace allocated here): True
    sizes the workspace so that dS is kept instead of recomputed (when that workspace is at most
    KEEP_DS_MAX_BYTES); False or None leaves it at the minimum.  The two forms measured within a
    few percent of each other, either way round depending on what ran before."""
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if workspace is None:
        need = attn_bwd_workspace_bytes(q.shape[0], _htot(q), q.shape[1])
        if keep_ds and q.dtype == torch.bfloat16 and q.shape[-1] == 128 and seqstart_q is None:
            big = attn_bwd_ds_workspace_bytes(q.shape[0], _htot(q), q.shape[1], k.shape[1])
            if big <= KEEP_DS_MAX_BYTES:
                need = big
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    args, _keep = _bwd_args(dout, q, k, v, out, lse, mask, scale, seqstart_q, seqstart_k, max_seqlen_q,
                            max_seqlen_k, window_size, window_left, window_right, workspace, dq, dk, dv, stream)
    _check(_lib.attn_bwd(*args))
    return dq, dk, dv


def prepare_bwd(dout, q, k, v, out, lse, dq, dk, dv, workspace, mask=MASK_NONE, scale=None, seqstart_q=None,
                seqstart_k=None, max_seqlen_q=None, max_seqlen_k=None, window_size=None, window_left=None,
                window_right=None, stream=None) -> Prepared:
    """attn_bwd with every argument marshalled up front.  A workspace of at least
    attn_bwd_ds_workspace_bytes(...) selects the kept-dS form (bf16, head dim 128, no block-diagonal
    mask); attn_bwd_workspace_bytes(...) the two-kernel form."""
    args, keep = _bwd_args(dout, q, k, v, out, lse, mask, scale, seqstart_q, seqstart_k, max_seqlen_q,
                           max_seqlen_k, window_size, window_left, window_right, workspace, dq, dk, dv, stream)
    return Prepared(_lib.attn_bwd, args, (keep, dout, q, k, v, out, lse, dq, dk, dv, workspace))


def attn_decode_splitkv_int4(q, k, v, k_scale_shift, v_scale_shift, num_splits, seqlens=None, max_seqlen_k=None,
                             block_tables=None, page_size=None, scale=None, workspace=None, out=None, lse=True,
                             out_dtype=None, stream=None, window_size=None):
    """Split-KV decode over INT4 K/V caches: uint8 tensors [..., D/2] (two 4-bit codes per byte,
    even element low) with float16 (or float32) (scale, shift) pairs [..., 2G] per cache row, head and
    group.
    Lanes, padded lanes (seqlens) or pages (block_tables).  Returns (out, lse or None)."""
    if num_splits is None:  # the library's choice for the keys a sequence may hold
        num_splits = attn_decode_num_splits(q.shape[0], _htot(q), max_seqlen_k or k.shape[1])
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    if lse is True:
        lse = torch.empty((q.shape[0], _htot(q), 1), dtype=torch.float32, device=q.device)
    elif lse is False:
        lse = None
    need = attn_decode_workspace_bytes(q.shape[0], _htot(q), q.shape[-1], num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    args, _keep = _fp8_args(q, k, v, k_scale_shift, v_scale_shift, seqlens, block_tables, page_size, max_seqlen_k,
                            num_splits, scale, workspace, out, lse, stream, kv_code=ATTN_DTYPE_INT4X2,
                            window_size=window_size)
    _check(_lib.attn_decode_splitkv_int4(*args))
    return out, lse


def prepare_decode_int4(q, k, v, k_scale_shift, v_scale_shift, num_splits, workspace, out, lse, seqlens=None,
                        max_seqlen_k=None, block_tables=None, page_size=None, scale=None, stream=None,
                        window_size=None) -> Prepared:
    """attn_decode_splitkv_int4 with every argument marshalled up front."""
    args, ds = _fp8_args(q, k, v, k_scale_shift, v_scale_shift, seqlens, block_tables, page_size, max_seqlen_k,
                         num_splits, scale, workspace, out, lse, stream, kv_code=ATTN_DTYPE_INT4X2,
                         window_size=window_size)
    return Prepared(_lib.attn_decode_splitkv_int4, args,
                    (ds, q, k, v, k_scale_shift, v_scale_shift, seqlens, block_tables, workspace, out, lse))


def attn_decode_splitkv_mxfp8(q, k, v, k_scale, v_scale, num_splits, seqlens=None, max_seqlen_k=None,
                              block_tables=None, page_size=None, scale=None, workspace=None, out=None, lse=True,
                              out_dtype=None, stream=None, window_size=None):
    """Split-KV decode over MXFP8 K/V caches: E4M3 codes (torch.float8_e4m3fn) with one E8M0 block
    scale per 32 elements (torch.float8_e8m0fnu [..., D/32]).  Lanes, padded lanes (seqlens) or
    pages (block_tables).  Returns (out, lse or None)."""
    if num_splits is None:  # the library's choice for the keys a sequence may hold
        n = max_seqlen_k or k.shape[1]
        num_splits = attn_decode_num_splits(q.shape[0], _htot(q), min(n, window_size or n))
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    if lse is True:
        lse = torch.empty((q.shape[0], _htot(q), 1), dtype=torch.float32, device=q.device)
    elif lse is False:
        lse = None
    need = attn_decode_workspace_bytes(q.shape[0], _htot(q), q.shape[-1], num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    args, _keep = _fp8_args(q, k, v, k_scale, v_scale, seqlens, block_tables, page_size, max_seqlen_k, num_splits,
                            scale, workspace, out, lse, stream, window_size=window_size)
    _check(_lib.attn_decode_splitkv_mxfp8(*args))
    return out, lse


def prepare_decode_mxfp8(q, k, v, k_scale, v_scale, num_splits, workspace, out, lse, seqlens=None,
                         max_seqlen_k=None, block_tables=None, page_size=None, scale=None, stream=None,
                         window_size=None) -> Prepared:
    """attn_decode_splitkv_mxfp8 with every argument marshalled up front."""
    args, ds = _fp8_args(q, k, v, k_scale, v_scale, seqlens, block_tables, page_size, max_seqlen_k, num_splits,
                         scale, workspace, out, lse, stream, window_size=window_size)
    return Prepared(_lib.attn_decode_splitkv_mxfp8, args,
                    (ds, q, k, v, k_scale, v_scale, seqlens, block_tables, workspace, out, lse))
