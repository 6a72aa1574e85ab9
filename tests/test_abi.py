"""Host-only tests of the C ABI: the library loads, exports what include/attn.h
declares, and rejects invalid requests before any launch (no GPU needed: the
descriptors point at fake addresses that the validation never dereferences)."""
import ctypes
import os
import re
import subprocess

import pytest

from transformer_attention_02_amd import attn as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")
FAKE = 0x10000  # 16-byte aligned, never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z0-9_]+\s*\*?\s*(attn_[a-z0-9_]+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(["attn_fwd", "attn_partial", "attn_fwd_ex", "attn_partial_ex", "attn_merge",
                                           "attn_fwd_kvcache", "attn_fwd_kvcache_workspace_bytes",
                                           "attn_decode_workspace_bytes", "attn_decode_num_splits", "attn_decode_splitkv",
                                           "attn_decode_splitkv_noalloc",
                                           "attn_decode_splitkv_paged",
                                           "attn_decode_splitkv_fp8", "attn_decode_splitkv_int4",
                                           "attn_decode_splitkv_mxfp8", "attn_bwd_workspace_bytes", "attn_bwd_ds_workspace_bytes",
                                           "attn_bwd",
                                           "attn_last_error"])


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", A.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(A._lib, name)


def tensor(shape, dtype=A.ATTN_DTYPE_BF16, stride=None, data=FAKE):
    d = A.AttnTensor()
    d.data = data
    d.dtype = dtype
    d.ndim = len(shape)
    if stride is None:
        stride, acc = [], 1
        for s in reversed(shape):
            stride.insert(0, acc)
            acc *= s
    for i, (s, st) in enumerate(zip(shape, stride)):
        d.shape[i] = s
        d.stride[i] = st
    return d


def fwd(q, k, v, o, mask=0, varlen=None, scale=float("nan"), lse=FAKE, fn=None):
    fn = fn or A._lib.attn_fwd
    return fn(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), mask, varlen, scale, ctypes.byref(o),
              ctypes.c_void_p(lse) if lse else None, None)


def std4(M=128, D=128, dt=A.ATTN_DTYPE_BF16):
    return tensor([2, M, 4, D], dt)


@pytest.mark.parametrize("case,status,needle", [
    ("stride", A.ATTN_ERR_INVALID_ARGUMENT, "stride 1"),
    ("dtype_mix", A.ATTN_ERR_INVALID_ARGUMENT, "one dtype"),
    ("k_dim", A.ATTN_ERR_INVALID_ARGUMENT, "head dims differ"),
    ("kv_rows", A.ATTN_ERR_INVALID_ARGUMENT, "key counts"),
    ("out_dim", A.ATTN_ERR_INVALID_ARGUMENT, "out head dim"),
    ("batch", A.ATTN_ERR_INVALID_ARGUMENT, "batch"),
    ("mask", A.ATTN_ERR_INVALID_ARGUMENT, "mask kind"),
    ("align", A.ATTN_ERR_INVALID_ARGUMENT, "16-byte"),
    ("ndim", A.ATTN_ERR_INVALID_ARGUMENT, "ndim"),
    ("hd96", A.ATTN_ERR_UNSUPPORTED, "K and Kv in {64, 128, 256}"),
    ("f32_big", A.ATTN_ERR_UNSUPPORTED, "<= 128"),
    ("varlen_missing", A.ATTN_ERR_INVALID_ARGUMENT, "varlen"),
    ("out_dtype", A.ATTN_ERR_INVALID_ARGUMENT, "q's dtype"),
    ("scale_inf", A.ATTN_ERR_INVALID_ARGUMENT, "scale"),
    ("null", A.ATTN_ERR_INVALID_ARGUMENT, "NULL"),
    ("out_broadcast", A.ATTN_ERR_INVALID_ARGUMENT, "stride-0"),
])
def test_fwd_rejects(case, status, needle):
    q, k, v, o = std4(), std4(256), std4(256), std4()
    kw = {}
    if case == "stride":
        q = tensor([2, 128, 4, 128], stride=[65536, 512, 128, 2])
    elif case == "dtype_mix":
        k = std4(256, dt=A.ATTN_DTYPE_F32)
    elif case == "k_dim":
        k = std4(256, 64)
    elif case == "kv_rows":
        v = std4(255)
    elif case == "out_dim":
        o = std4(128, 64)
    elif case == "batch":
        k = tensor([3, 256, 4, 128])
    elif case == "mask":
        kw["mask"] = 7
    elif case == "align":
        q = tensor([2, 128, 4, 128], data=FAKE + 8)
    elif case == "ndim":
        q = tensor([2, 128, 128])
    elif case == "hd96":
        q, k, v, o = std4(128, 96), std4(256, 96), std4(256, 96), std4(128, 96)
    elif case == "f32_big":
        f = A.ATTN_DTYPE_F32
        q, k, v, o = std4(128, 256, f), std4(256, 256, f), std4(256, 256, f), std4(128, 256, f)
    elif case == "varlen_missing":
        kw["mask"] = A.MASK_BLOCKDIAG_CAUSAL
    elif case == "out_dtype":
        o = std4(dt=A.ATTN_DTYPE_F32)
    elif case == "scale_inf":
        kw["scale"] = float("inf")
    elif case == "null":
        q = tensor([2, 128, 4, 128], data=0)
    elif case == "out_broadcast":  # both batch elements would store to the same rows
        o = tensor([2, 128, 4, 128], stride=[0, 512, 128, 1])
    rc = fwd(q, k, v, o, **kw)
    assert rc == status
    assert needle in A.attn_last_error()


def test_partial_allows_fp32_out_but_needs_lse():
    q, k, v = std4(), std4(256), std4(256)
    o32 = std4(dt=A.ATTN_DTYPE_F32)
    rc = fwd(q, k, v, o32, lse=0, fn=A._lib.attn_partial)
    assert rc == A.ATTN_ERR_INVALID_ARGUMENT and "lse is required" in A.attn_last_error()


def test_varlen_checks():
    q, k, v, o = (tensor([1, 300, 4, 128]) for _ in range(4))
    vl = A.AttnVarlen()
    vl.seqstart_q = FAKE
    vl.nseq = 0
    vl.max_seqlen_q = 100
    assert fwd(q, k, v, o, mask=A.MASK_BLOCKDIAG, varlen=ctypes.byref(vl)) == A.ATTN_ERR_INVALID_ARGUMENT
    vl.nseq = 3
    vl.max_seqlen_q = 301
    assert fwd(q, k, v, o, mask=A.MASK_BLOCKDIAG, varlen=ctypes.byref(vl)) == A.ATTN_ERR_INVALID_ARGUMENT
    assert "max_seqlen_q" in A.attn_last_error()
    q2, k2, v2, o2 = (tensor([2, 300, 4, 128]) for _ in range(4))
    vl.max_seqlen_q = 100
    assert fwd(q2, k2, v2, o2, mask=A.MASK_BLOCKDIAG, varlen=ctypes.byref(vl)) == A.ATTN_ERR_INVALID_ARGUMENT
    assert "B == 1" in A.attn_last_error()


def test_empty_problem_is_a_no_op():
    q, k, v, o = tensor([0, 128, 4, 128]), tensor([0, 256, 4, 128]), tensor([0, 256, 4, 128]), tensor([0, 128, 4, 128])
    assert fwd(q, k, v, o) == A.ATTN_OK


def merge_call(n, chunks, lses, out, lse_out=FAKE):
    arr = (A.AttnTensor * max(1, n))(*chunks)
    lp = (ctypes.c_void_p * max(1, n))(*lses)
    return A._lib.attn_merge(n, arr, lp, ctypes.byref(out), ctypes.c_void_p(lse_out), None)


def test_merge_rejects():
    c = tensor([1, 128, 16, 128], A.ATTN_DTYPE_F32)
    o = tensor([1, 128, 16, 128])
    assert merge_call(0, [], [], o) == A.ATTN_ERR_INVALID_ARGUMENT
    assert "at least one chunk" in A.attn_last_error()
    assert merge_call(129, [c] * 129, [FAKE] * 129, o) == A.ATTN_ERR_UNSUPPORTED
    c2 = tensor([1, 64, 16, 128], A.ATTN_DTYPE_F32)
    assert merge_call(2, [c, c2], [FAKE, FAKE], o) == A.ATTN_ERR_INVALID_ARGUMENT
    c3 = tensor([1, 128, 16, 128], A.ATTN_DTYPE_F32, stride=[16 * 128 * 256, 16 * 256, 256, 1])
    assert merge_call(2, [c, c3], [FAKE, FAKE], o) == A.ATTN_ERR_UNSUPPORTED
    assert merge_call(2, [c, c], [FAKE, 0], o) == A.ATTN_ERR_INVALID_ARGUMENT
    assert "lse_chunks[1]" in A.attn_last_error()
    assert merge_call(1, [c], [FAKE], tensor([1, 128, 8, 128])) == A.ATTN_ERR_INVALID_ARGUMENT
    o_heads0 = tensor([1, 128, 16, 128], stride=[128 * 128, 128, 0, 1])
    assert merge_call(2, [c, c], [FAKE, FAKE], o_heads0) == A.ATTN_ERR_INVALID_ARGUMENT
    assert "stride-0" in A.attn_last_error()


def test_decode_workspace_and_rejects():
    B, H, D, S = 16, 32, 128, 64
    need = A.attn_decode_workspace_bytes(B, H, D, S)
    assert need == (S * B * H * D * 4 + 255) // 256 * 256 + (S * B * H * 4 + 255) // 256 * 256
    assert A.attn_decode_workspace_bytes(B, H, D, 0) == 0
    q, o = tensor([B, 1, H, D]), tensor([B, 1, H, D])
    k, v = tensor([B, 1024, H, D]), tensor([B, 1024, H, D])

    def call(num_splits=S, ws=FAKE * 256, wsb=need, qq=q):
        return A._lib.attn_decode_splitkv(ctypes.byref(qq), ctypes.byref(k), ctypes.byref(v), num_splits,
                                          float("nan"), ctypes.c_void_p(ws), wsb, ctypes.byref(o), None, None)
    assert call(wsb=need - 1) == A.ATTN_ERR_WORKSPACE_TOO_SMALL
    assert call(num_splits=0) == A.ATTN_ERR_INVALID_ARGUMENT
    assert call(num_splits=129) == A.ATTN_ERR_UNSUPPORTED
    assert call(ws=FAKE * 256 + 16) == A.ATTN_ERR_INVALID_ARGUMENT
    assert call(qq=tensor([B, 2, H, D])) == A.ATTN_ERR_INVALID_ARGUMENT
    o_b0 = tensor([B, 1, H, D], stride=[0, H * D, D, 1])
    assert A._lib.attn_decode_splitkv(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), S, float("nan"),
                                      ctypes.c_void_p(FAKE * 256), need, ctypes.byref(o_b0), None,
                                      None) == A.ATTN_ERR_INVALID_ARGUMENT
    assert "stride-0" in A.attn_last_error()


def fwd_ex(q, k, v, o, mask, varlen=None, fn=None):
    fn = fn or A._lib.attn_fwd_ex
    return fn(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), ctypes.byref(mask) if mask is not None else None,
              varlen, float("nan"), ctypes.byref(o), ctypes.c_void_p(FAKE), None)


def test_windowed_masks_need_the_ex_entry_point_and_valid_windows():
    q, k, v, o = std4(), std4(256), std4(256), std4()
    for kind in (6, 7, 8, 9):
        assert fwd(q, k, v, o, mask=kind) == A.ATTN_ERR_INVALID_ARGUMENT
        assert "_ex" in A.attn_last_error()
    assert fwd_ex(q, k, v, o, None) == A.ATTN_ERR_INVALID_ARGUMENT
    assert fwd_ex(q, k, v, o, A.AttnMask(7, 0, 0, 0)) == A.ATTN_ERR_INVALID_ARGUMENT
    assert "window_size" in A.attn_last_error()
    assert fwd_ex(q, k, v, o, A.AttnMask(6, 0, -1, 3)) == A.ATTN_ERR_INVALID_ARGUMENT
    assert "window_left" in A.attn_last_error()
    assert fwd_ex(q, k, v, o, A.AttnMask(10, 1, 0, 0)) == A.ATTN_ERR_INVALID_ARGUMENT
    assert fwd_ex(q, k, v, o, A.AttnMask(8, 4, 0, 0)) == A.ATTN_ERR_INVALID_ARGUMENT  # packed kind, no varlen
    assert "varlen" in A.attn_last_error()
    assert fwd_ex(q, k, v, o, A.AttnMask(5, 0, 0, 0), fn=A._lib.attn_partial_ex) == A.ATTN_ERR_INVALID_ARGUMENT


def test_paged_decode_rejects():
    B, H, D, S = 4, 8, 128, 4
    need = A.attn_decode_workspace_bytes(B, H, D, S)
    q, o = tensor([B, 1, H, D]), tensor([B, 1, H, D])
    cache = tensor([1, 64 * 16, H, D])

    def call(k=cache, seqlens=FAKE, bt=FAKE, mb=8, page=16, mx=128, wsb=need, W=0):
        return A._lib.attn_decode_splitkv_paged(ctypes.byref(q), ctypes.byref(k), ctypes.byref(k), ctypes.c_void_p(seqlens),
                                                ctypes.c_void_p(bt) if bt else None, mb, page, mx, W, S, float("nan"),
                                                ctypes.c_void_p(FAKE * 256), wsb, ctypes.byref(o), None, None)
    assert call(seqlens=0) == A.ATTN_ERR_INVALID_ARGUMENT and "seqlens" in A.attn_last_error()
    assert call(page=0) == A.ATTN_ERR_INVALID_ARGUMENT
    assert call(page=48) == A.ATTN_ERR_INVALID_ARGUMENT and "whole number of pages" in A.attn_last_error()
    assert call(mx=8 * 16 + 1) == A.ATTN_ERR_INVALID_ARGUMENT and "max_seqlen_k" in A.attn_last_error()
    assert call(k=tensor([2, 64 * 16, H, D])) == A.ATTN_ERR_INVALID_ARGUMENT and "batch 1" in A.attn_last_error()
    assert call(wsb=need - 1) == A.ATTN_ERR_WORKSPACE_TOO_SMALL
    lanes = tensor([B, 300, H, D])
    assert call(k=lanes, bt=0, mx=301) == A.ATTN_ERR_INVALID_ARGUMENT   # padded lanes: max_seqlen_k <= lane capacity
    assert call(W=-1) == A.ATTN_ERR_INVALID_ARGUMENT and "window_size" in A.attn_last_error()


def test_fp8_decode_rejects():
    B, H, D, S, M = 4, 8, 128, 4, 256
    need = A.attn_decode_workspace_bytes(B, H, D, S)
    q, o = tensor([B, 1, H, D]), tensor([B, 1, H, D])
    k8 = tensor([B, M, H, D], A.ATTN_DTYPE_FP8_E4M3)
    ss = tensor([B, M, H, 2], A.ATTN_DTYPE_F16, data=FAKE + 4)  # 4-byte alignment suffices for metadata

    def call(qq=q, k=k8, kss=ss, vss=ss, oo=o, seqlens=0, bt=0, mx=0):
        return A._lib.attn_decode_splitkv_fp8(ctypes.byref(qq), ctypes.byref(k), ctypes.byref(k), ctypes.byref(kss),
                                              ctypes.byref(vss), ctypes.c_void_p(seqlens) if seqlens else None,
                                              ctypes.c_void_p(bt) if bt else None, 8, 32, mx, 0, S, float("nan"),
                                              ctypes.c_void_p(FAKE * 256), need, ctypes.byref(oo), None, None)
    assert call(k=tensor([B, M, H, D])) == A.ATTN_ERR_INVALID_ARGUMENT and "dtype" in A.attn_last_error()
    assert call(kss=tensor([B, M, H, 2], A.ATTN_DTYPE_F32)) == A.ATTN_ERR_INVALID_ARGUMENT
    assert call(vss=tensor([B, M, H, 4], A.ATTN_DTYPE_F16)) == A.ATTN_ERR_INVALID_ARGUMENT
    assert "scale/shift" in A.attn_last_error()
    assert call(kss=tensor([B, M - 1, H, 2], A.ATTN_DTYPE_F16)) == A.ATTN_ERR_INVALID_ARGUMENT
    assert call(kss=tensor([B, M, H, 2], A.ATTN_DTYPE_F16, data=FAKE + 2)) == A.ATTN_ERR_INVALID_ARGUMENT
    assert call(qq=tensor([B, 1, H, D], A.ATTN_DTYPE_F32)) == A.ATTN_ERR_INVALID_ARGUMENT and "bf16" in A.attn_last_error()
    assert call(bt=FAKE) == A.ATTN_ERR_INVALID_ARGUMENT and "seqlens" in A.attn_last_error()
    assert call(k=tensor([B, M, H, 96], A.ATTN_DTYPE_FP8_E4M3)) == A.ATTN_ERR_INVALID_ARGUMENT
    assert call(k=tensor([B, M, H, D], A.ATTN_DTYPE_FP8_E4M3, data=FAKE + 8)) == A.ATTN_ERR_INVALID_ARGUMENT
    # fp32 (scale, shift) pairs (use_fp32_scales): both tensors fp32, rows 8-byte aligned
    ss32 = tensor([B, M, H, 2], A.ATTN_DTYPE_F32)
    assert call(kss=ss32, vss=ss) == A.ATTN_ERR_INVALID_ARGUMENT and "share one dtype" in A.attn_last_error()
    assert call(kss=ss32, vss=tensor([B, M, H, 2], A.ATTN_DTYPE_F32, data=FAKE + 4)) == A.ATTN_ERR_INVALID_ARGUMENT
    assert "8-byte aligned" in A.attn_last_error()
    odd = tensor([B, M, H, 2], A.ATTN_DTYPE_F32)
    odd.stride[1] = H * 2 + 1  # rows of an odd number of fp32: not 8-byte aligned
    odd.stride[0] = M * odd.stride[1]
    assert call(kss=odd, vss=odd) == A.ATTN_ERR_INVALID_ARGUMENT and "multiple of 8 bytes" in A.attn_last_error()


def test_mxfp8_decode_rejects():
    B, H, D, S, M = 4, 8, 128, 4, 256
    need = A.attn_decode_workspace_bytes(B, H, D, S)
    q, o = tensor([B, 1, H, D]), tensor([B, 1, H, D])
    k8 = tensor([B, M, H, D], A.ATTN_DTYPE_FP8_E4M3)
    sc = lambda n, dt=A.ATTN_DTYPE_E8M0: tensor([B, M, H, n], dt, data=FAKE + 1)  # byte scales: any alignment

    def call(k=k8, ks=None, vs=None):
        ks = ks or sc(D // 32)
        vs = vs or ks
        return A._lib.attn_decode_splitkv_mxfp8(ctypes.byref(q), ctypes.byref(k), ctypes.byref(k), ctypes.byref(ks),
                                                ctypes.byref(vs), None, None, 0, 0, 0, 0, S, float("nan"),
                                                ctypes.c_void_p(FAKE * 256), need, ctypes.byref(o), None, None)
    assert call(ks=sc(D // 32, A.ATTN_DTYPE_F16)) == A.ATTN_ERR_INVALID_ARGUMENT and "dtype" in A.attn_last_error()
    assert call(ks=sc(D // 16)) == A.ATTN_ERR_INVALID_ARGUMENT and "D/32" in A.attn_last_error()
    assert call(vs=tensor([B, M - 1, H, D // 32], A.ATTN_DTYPE_E8M0)) == A.ATTN_ERR_INVALID_ARGUMENT
    assert call(k=tensor([B, M, H, D // 2], A.ATTN_DTYPE_INT4X2)) == A.ATTN_ERR_INVALID_ARGUMENT
    assert call(k=tensor([B, M, H, 48], A.ATTN_DTYPE_FP8_E4M3), ks=sc(1)) == A.ATTN_ERR_INVALID_ARGUMENT


def test_fp8_and_f16_tensors_are_rejected_outside_the_fp8_decode():
    q8 = tensor([2, 128, 4, 128], A.ATTN_DTYPE_FP8_E4M3)
    h = tensor([2, 128, 4, 128], A.ATTN_DTYPE_F16)
    assert fwd(q8, q8, q8, q8) == A.ATTN_ERR_INVALID_ARGUMENT and "dtype" in A.attn_last_error()
    assert fwd(h, h, h, h) == A.ATTN_ERR_INVALID_ARGUMENT
    assert fwd(std4(), q8, q8, std4()) == A.ATTN_ERR_INVALID_ARGUMENT


def test_bwd_kept_ds_workspace_size():
    """The kept-dS workspace: the two row arrays, then round_up(Mkv, 128) x round_up(Mq, 256) bf16
    per (batch, head), 256-byte rounded; SIZE_MAX once Mq passes 2^24; 0 for negative sizes."""
    for B, H, Mq, Mkv in [(2, 32, 2048, 2048), (1, 3, 300, 333), (2, 1, 1, 1), (1, 1, 0, 5), (3, 2, 257, 0)]:
        rows = A.attn_bwd_workspace_bytes(B, H, Mq)
        ds = B * H * ((Mkv + 127) // 128 * 128) * ((Mq + 255) // 256 * 256) * 2
        assert A.attn_bwd_ds_workspace_bytes(B, H, Mq, Mkv) == rows + (ds + 255) // 256 * 256
    assert A.attn_bwd_ds_workspace_bytes(2, 32, 2048, 2048) == 1048576 + 2 * 32 * 2048 * 2048 * 2
    assert A.attn_bwd_ds_workspace_bytes(1, 1, (1 << 24) + 1, 1) == 2 ** 64 - 1
    assert A.attn_bwd_ds_workspace_bytes(1, 1, 1 << 24, 1) < 2 ** 40
    assert A.attn_bwd_ds_workspace_bytes(-1, 1, 1, 1) == 0


def test_bwd_workspace_and_rejects():
    B, M, H, D = 2, 256, 4, 128
    need = A.attn_bwd_workspace_bytes(B, H, M)
    assert need == 2 * ((B * H * M * 4 + 255) // 256 * 256)
    t = lambda shape=(B, M, H, D), dt=A.ATTN_DTYPE_BF16, stride=None: tensor(list(shape), dt, stride)
    m = A.AttnMask(1, 0, 0, 0)

    def call(g=None, q=None, k=None, v=None, o=None, dq=None, dk=None, dv=None, mask=m, ws=FAKE * 256, wsb=need,
             lse=FAKE, varlen=None):
        ds = [x if x is not None else t() for x in (g, q, k, v, o, dq, dk, dv)]
        return A._lib.attn_bwd(*[ctypes.byref(x) for x in ds[:5]], ctypes.c_void_p(lse) if lse else None,
                               ctypes.byref(mask) if mask is not None else None, varlen, float("nan"),
                               ctypes.c_void_p(ws), wsb, *[ctypes.byref(x) for x in ds[5:]], None)
    assert call(wsb=need - 1) == A.ATTN_ERR_WORKSPACE_TOO_SMALL
    assert call(ws=FAKE * 256 + 16) == A.ATTN_ERR_INVALID_ARGUMENT
    assert call(lse=0) == A.ATTN_ERR_INVALID_ARGUMENT and "lse" in A.attn_last_error()
    assert call(mask=None) == A.ATTN_ERR_INVALID_ARGUMENT
    assert call(q=t(dt=A.ATTN_DTYPE_F32)) == A.ATTN_ERR_INVALID_ARGUMENT and "dtype" in A.attn_last_error()
    f32 = t((B, M, H, 160), dt=A.ATTN_DTYPE_F32)  # fp32 head dims above 128 are not built
    assert call(f32, f32, f32, f32, f32, f32, f32, f32) == A.ATTN_ERR_UNSUPPORTED
    assert call(dq=t((B, M + 1, H, D))) == A.ATTN_ERR_INVALID_ARGUMENT and "q's shape" in A.attn_last_error()
    assert call(g=t((B, M, H, 64))) == A.ATTN_ERR_INVALID_ARGUMENT and "dout" in A.attn_last_error()
    assert call(dv=t((B, M, H, 64))) == A.ATTN_ERR_INVALID_ARGUMENT
    expanded = t(stride=[M * H * D, H * D, 0, 1])
    assert call(dk=expanded) == A.ATTN_ERR_INVALID_ARGUMENT and "stride-0" in A.attn_last_error()
    assert call(mask=A.AttnMask(3, 0, 0, 0)) == A.ATTN_ERR_INVALID_ARGUMENT and "varlen" in A.attn_last_error()
    assert call(mask=A.AttnMask(7, 0, 0, 0)) == A.ATTN_ERR_INVALID_ARGUMENT and "window_size" in A.attn_last_error()
    d96 = t((B, M, H, 96))
    assert call(d96, d96, d96, d96, d96, d96, d96, d96) == A.ATTN_ERR_UNSUPPORTED


def test_int4_decode_rejects():
    B, H, D, S, M = 4, 8, 128, 4, 256
    need = A.attn_decode_workspace_bytes(B, H, D, S)
    q, o = tensor([B, 1, H, D]), tensor([B, 1, H, D])
    k4 = tensor([B, M, H, D // 2], A.ATTN_DTYPE_INT4X2)
    ss = lambda G: tensor([B, M, H, 2 * G], A.ATTN_DTYPE_F16, data=FAKE + 4)

    def call(k=k4, kss=None, vss=None, fn=A._lib.attn_decode_splitkv_int4):
        kss = kss or ss(1)
        vss = vss or kss
        return fn(ctypes.byref(q), ctypes.byref(k), ctypes.byref(k), ctypes.byref(kss), ctypes.byref(vss), None, None,
                  0, 0, 0, 0, S, float("nan"), ctypes.c_void_p(FAKE * 256), need, ctypes.byref(o), None, None)
    assert call(kss=ss(8)) == A.ATTN_ERR_UNSUPPORTED and "multiple of 32" in A.attn_last_error()   # groups of 16
    assert call(kss=ss(3)) == A.ATTN_ERR_UNSUPPORTED
    assert call(kss=ss(2), vss=ss(4)) == A.ATTN_ERR_INVALID_ARGUMENT
    assert call(k=tensor([B, M, H, D], A.ATTN_DTYPE_INT4X2)) == A.ATTN_ERR_INVALID_ARGUMENT  # D codes = D/2 bytes
    assert call(k=tensor([B, M, H, D // 2], A.ATTN_DTYPE_FP8_E4M3)) == A.ATTN_ERR_INVALID_ARGUMENT
    k8 = tensor([B, M, H, D], A.ATTN_DTYPE_FP8_E4M3)
    # FP8 groups: a lane's 16 codes share one group, so D/G must be a multiple of 16
    assert call(k=k8, kss=ss(16), fn=A._lib.attn_decode_splitkv_fp8) == A.ATTN_ERR_UNSUPPORTED
    assert "multiple of 16" in A.attn_last_error()
    assert call(k=tensor([B, M, H, D // 2], A.ATTN_DTYPE_INT4X2, data=FAKE + 8)) == A.ATTN_ERR_INVALID_ARGUMENT


def test_noalloc_decode_refuses_more_than_its_scratch():
    # 64 x 64 x 128 rows of 128 floats need 268 MB of partials: refused before any launch
    q = tensor([64, 1, 64, 128])
    k = tensor([64, 256, 64, 128])
    o = tensor([64, 1, 64, 128])
    assert A.attn_decode_workspace_bytes(64, 64, 128, 128) > A.NOALLOC_SCRATCH_BYTES
    rc = A._lib.attn_decode_splitkv_noalloc(ctypes.byref(q), ctypes.byref(k), ctypes.byref(k), 128, float("nan"),
                                            ctypes.byref(o), None, None)
    assert rc == A.ATTN_ERR_UNSUPPORTED
    assert "bytes of scratch" in A.attn_last_error()


def test_noalloc_scratch_size_matches_the_header():
    text = open(HEADER).read()
    m = re.search(r"#define ATTN_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == A.NOALLOC_SCRATCH_BYTES


def test_decode_num_splits_fills_the_device_with_chunks_of_256_keys_or_more():
    # host-only: with no GPU the library assumes MI355X's 256 compute units; B * H * S reaches 8 per
    # unit unless chunks would fall below 256 keys, and S stays a power of two <= 128
    cus = 256
    for B, H, M in [(16, 32, 32768), (1, 32, 32768), (1, 8, 131072), (64, 32, 4096), (128, 8, 1024),
                    (4, 32, 8192), (16, 16, 16384), (32, 8, 2048), (1, 1, 100), (3, 5, 1 << 20)]:
        S = A.attn_decode_num_splits(B, H, M)
        assert 1 <= S <= 128 and S & (S - 1) == 0
        enough = B * H * S >= 8 * cus or S == 128 or M // (2 * S) < 256
        assert enough, (B, H, M, S)
        assert S == 1 or M // S >= 256, (B, H, M, S)
        assert S == 1 or B * H * (S // 2) < 8 * cus, (B, H, M, S)  # the smallest such power of two
    assert A.attn_decode_num_splits(16, 32, 32768) == 4
    assert A.attn_decode_num_splits(1, 32, 32768) == 64
    assert A.attn_decode_num_splits(0, 32, 32768) == 1


def test_fwd_kvcache_rejects():
    # packed queries [1, 300, 8, 128] against 4 lanes of 1024 keys or a paged cache of 64 pages of 256
    q, o = tensor([1, 300, 8, 128]), tensor([1, 300, 8, 128])
    lanes = tensor([4, 1024, 8, 128])
    cache = tensor([1, 64 * 256, 8, 128])
    ss, lens, tab = ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE + 64), ctypes.c_void_p(FAKE + 128)

    def call(k=lanes, kind=A.MASK_CAUSAL_BR, nseq=4, mq=100, tables=None, mb=0, page=0, mk=1024, S=1, ws=None,
             wsb=0, qq=q, oo=o, W=0, starts=None):
        m = A.AttnMask(kind, W, 0, 0)
        return A._lib.attn_fwd_kvcache(ctypes.byref(qq), ctypes.byref(k), ctypes.byref(k), ctypes.byref(m), ss, nseq,
                                       mq, starts, lens, tables, mb, page, mk, S, float("nan"), ws, wsb,
                                       ctypes.byref(oo), None, None)

    assert call(kind=A.MASK_CAUSAL) == A.ATTN_ERR_INVALID_ARGUMENT and "mask kind" in A.attn_last_error()
    assert call(kind=A.MASK_BLOCKDIAG) == A.ATTN_ERR_INVALID_ARGUMENT
    assert call(nseq=5) == A.ATTN_ERR_INVALID_ARGUMENT and "lane per sequence" in A.attn_last_error()
    assert call(mq=301) == A.ATTN_ERR_INVALID_ARGUMENT
    assert call(mk=1025) == A.ATTN_ERR_INVALID_ARGUMENT
    assert call(S=0) == A.ATTN_ERR_INVALID_ARGUMENT and call(S=129) == A.ATTN_ERR_INVALID_ARGUMENT
    assert call(S=4) == A.ATTN_ERR_INVALID_ARGUMENT  # no workspace
    need = A.attn_fwd_kvcache_workspace_bytes(300, 8, 128, 4)
    assert need == (4 * 300 * 8 * 128 * 4 + 255) // 256 * 256 + (4 * 300 * 8 * 4 + 255) // 256 * 256
    assert call(S=4, ws=ctypes.c_void_p(FAKE * 256), wsb=need - 1) == A.ATTN_ERR_WORKSPACE_TOO_SMALL
    assert call(k=cache, tables=tab, mb=64, page=96) == A.ATTN_ERR_UNSUPPORTED and "multiple of 64" in A.attn_last_error()
    assert call(k=cache, tables=tab, mb=8193, page=256, mk=256) == A.ATTN_ERR_UNSUPPORTED
    assert call(k=tensor([2, 64 * 256, 8, 128]), tables=tab, mb=64, page=256) == A.ATTN_ERR_INVALID_ARGUMENT
    assert call(k=tensor([1, 64 * 256 + 64, 8, 128]), tables=tab, mb=64, page=256) == A.ATTN_ERR_INVALID_ARGUMENT
    assert call(qq=tensor([2, 150, 8, 128]), oo=tensor([2, 150, 8, 128])) == A.ATTN_ERR_INVALID_ARGUMENT
    assert call(qq=tensor([1, 300, 8, 128], A.ATTN_DTYPE_F32)) == A.ATTN_ERR_UNSUPPORTED
    assert call(kind=A.MASK_CAUSAL_LOCAL_BR, W=0) == A.ATTN_ERR_INVALID_ARGUMENT
    assert A.attn_fwd_kvcache_workspace_bytes(300, 8, 128, 1) == 0
    # gappy lanes: key starts into one k/v tensor (B == 1), not over a paged cache
    gappy = ctypes.c_void_p(FAKE + 192)
    assert call(starts=gappy) == A.ATTN_ERR_INVALID_ARGUMENT and "B == 1" in A.attn_last_error()
    assert call(k=cache, tables=tab, mb=64, page=256, starts=gappy) == A.ATTN_ERR_UNSUPPORTED
    assert call(k=tensor([1, 4096, 8, 128]), starts=gappy, mk=4097) == A.ATTN_ERR_INVALID_ARGUMENT
    assert call(k=tensor([1, 4096, 8, 128]), starts=ctypes.c_void_p(FAKE + 194)) == A.ATTN_ERR_INVALID_ARGUMENT
