"""MI355X-native exact attention, FlashAttention-2 style (gfx950 HIP kernels).

Thin Python binding of ``libfa.so`` (declared in ``include/fa.h``). Every
step of the computation runs in the HIP kernels; this module only turns
torch device tensors into pointers, sizes and the current HIP stream, and
turns negative status codes into exceptions. There is no fallback: if the
library is missing or the tensors are not on a gfx950 device the calls fail.

Names follow the C ABI: ``fa_fwd``, ``fa_fwd_strided``, ``fa_fwd_varlen``,
``fa_bwd``, ``fa_bwd_noalloc``, ``fa_fwd_fa1_order``. Convenience wrappers that allocate the
outputs: ``attention``, ``attention_bnhd``, ``attention_qkvpacked``,
``attention_varlen``, ``attention_backward``.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_F16, FA_BF16 = 0, 1
STATUS = {
    0: "FA_OK", -1: "FA_ERR_NULL", -2: "FA_ERR_DIM", -3: "FA_ERR_UNSUPPORTED",
    -4: "FA_ERR_SCALE", -5: "FA_ERR_ALIGN", -6: "FA_ERR_LAUNCH", -7: "FA_ERR_ALIAS",
    -8: "FA_ERR_DEVICE", -9: "FA_ERR_TOO_LARGE",
}
BWD_NOALLOC_MAX_ROWS = 4194304  # FA_BWD_NOALLOC_MAX_ROWS of fa.h

_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int
_L = ctypes.c_int64
_F = ctypes.c_float

_SIGS = {
    "fa_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _P]),
    "fa_fwd_strided": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I] + [_L] * 12 + [_P]),
    "fa_fwd_varlen": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _P]),
    "fa_bwd": (_I, [_P] * 10 + [_I, _I, _I, _I, _F, _I, _I, _P]),
    "fa_bwd_workspace_bytes": (_L, [_I, _I, _I, _I]),
    "fa_bwd_noalloc": (_I, [_P] * 9 + [_I, _I, _I, _I, _F, _I, _I, _P]),
    "fa_fwd_fa1_order": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _P]),
    "fa_fwd_fa1_workspace_bytes": (_L, [_I, _I, _I, _I]),
    "fa_strerror": (ctypes.c_char_p, [_I]),
    "fa_version": (_I, []),
}


class FAError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {STATUS.get(code, code)} ({lib().fa_strerror(code).decode()})")


def lib() -> ctypes.CDLL:
    """The loaded libfa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m exact_attention_fa2_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(code: int, where: str) -> None:
    if code != 0:
        raise FAError(code, where)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float16:
        return FA_F16
    if t.dtype == torch.bfloat16:
        return FA_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (fp16 or bf16)")


def _stream(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _dev(*ts) -> None:
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on the GPU")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _contiguous(**ts) -> None:
    for name, t in ts.items():
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous (the kernels read it as a dense row-major tensor)")


def _need(t, name: str, numel: int, dtype=None) -> None:
    """A dense tensor holding at least `numel` elements (of `dtype`), so that the
    kernel's reads and writes stay inside it."""
    if t is None:
        return
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements; the call needs {numel}")


def _check_lse(lse, B: int, H: int, N: int, q) -> None:
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (B, H, N):
        raise ValueError(f"lse must be a contiguous float32 tensor of shape {(B, H, N)}, got "
                         f"{lse.dtype} {tuple(lse.shape)} (contiguous={lse.is_contiguous()})")
    if lse.device != q.device:
        raise ValueError("lse must live on q's device")


# ---------------------------------------------------------------------------
# raw entry points (same names and argument order as the C ABI)
# ---------------------------------------------------------------------------
def fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, stream=None):
    n = B * H * N * d
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _need(t, name, n)
    _need(lse, "lse", B * H * N, torch.float32)
    _dev(q, k, v, o, lse)
    _check(lib().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                        float(scale), int(bool(causal)), _dtype_code(q), _stream(stream)), "fa_fwd")


def fa_fwd_strided(q, k, v, o, lse, B, H, N, d, scale, causal, q_strides, k_strides, v_strides,
                   o_strides, stream=None):
    _need(lse, "lse", B * H * N, torch.float32)
    _dev(q, k, v, o, lse)
    _check(lib().fa_fwd_strided(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                                float(scale), int(bool(causal)), _dtype_code(q),
                                *q_strides, *k_strides, *v_strides, *o_strides, _stream(stream)),
           "fa_fwd_strided")


def fa_fwd_varlen(q, k, v, o, lse, cu_seqlens, B, T, max_seqlen, H, d, scale, causal, stream=None):
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _need(t, name, T * H * d)
    _need(lse, "lse", H * T, torch.float32)
    _need(cu_seqlens, "cu_seqlens", B + 1, torch.int32)
    _dev(q, k, v, o, lse, cu_seqlens)
    _check(lib().fa_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_seqlens), B, T,
                               max_seqlen, H, d, float(scale), int(bool(causal)), _dtype_code(q),
                               _stream(stream)), "fa_fwd_varlen")


def fa_bwd(q, k, v, o, do, lse, dq, dk, dv, workspace, B, H, N, d, scale, causal, stream=None):
    n = B * H * N * d
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do), ("dq", dq), ("dk", dk), ("dv", dv)):
        _need(t, name, n)
    _need(lse, "lse", B * H * N, torch.float32)
    _dev(q, k, v, o, do, lse, dq, dk, dv, workspace)
    _check(lib().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk),
                        _ptr(dv), _ptr(workspace), B, H, N, d, float(scale), int(bool(causal)),
                        _dtype_code(q), _stream(stream)), "fa_bwd")


def fa_bwd_noalloc(q, k, v, o, do, lse, dq, dk, dv, B, H, N, d, scale, causal, stream=None):
    n = B * H * N * d
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do), ("dq", dq), ("dk", dk), ("dv", dv)):
        _need(t, name, n)
    _need(lse, "lse", B * H * N, torch.float32)
    _dev(q, k, v, o, do, lse, dq, dk, dv)
    _check(lib().fa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk),
                                _ptr(dv), B, H, N, d, float(scale), int(bool(causal)), _dtype_code(q),
                                _stream(stream)), "fa_bwd_noalloc")


def fa_bwd_workspace_bytes(B, H, N, d) -> int:
    return int(lib().fa_bwd_workspace_bytes(B, H, N, d))


def fa_fwd_fa1_order(q, k, v, o, lse, workspace, B, H, N, d, scale, causal, stream=None):
    n = B * H * N * d
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _need(t, name, n)
    _need(lse, "lse", B * H * N, torch.float32)
    _dev(q, k, v, o, lse, workspace)
    _check(lib().fa_fwd_fa1_order(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(workspace), B, H,
                                  N, d, float(scale), int(bool(causal)), _dtype_code(q),
                                  _stream(stream)), "fa_fwd_fa1_order")


def fa_fwd_fa1_workspace_bytes(B, H, N, d) -> int:
    return int(lib().fa_fwd_fa1_workspace_bytes(B, H, N, d))


# ---------------------------------------------------------------------------
# convenience wrappers (allocate outputs with torch, then call the ABI)
# ---------------------------------------------------------------------------
def _default_scale(d, scale):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def _same(q, *others):
    for t in others:
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q, k and v must share shape, dtype and device")


def attention(q, k, v, causal=False, scale=None, stream=None):
    """O, LSE for contiguous q, k, v of shape [B, H, N, d]."""
    _same(q, k, v)
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous [B, H, N, d]")
    B, H, N, d = q.shape
    o = torch.empty_like(q, memory_format=torch.contiguous_format)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    fa_fwd(q, k, v, o, lse, B, H, N, d, _default_scale(d, scale), causal, stream)
    return o, lse


def _strides_bnhd(t):
    # [B, N, H, d] view -> (batch, head, row) strides; last dim must be unit-stride
    if t.stride(-1) != 1:
        raise ValueError("head-dim axis must be contiguous")
    return (t.stride(0), t.stride(2), t.stride(1))


def attention_bnhd(q, k, v, causal=False, scale=None, stream=None):
    """O [B, N, H, d] and LSE [B, H, N] for q, k, v of shape [B, N, H, d] (any strides
    with a unit-stride head dim)."""
    B, N, H, d = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k and v must share their shape")
    o = torch.empty((B, N, H, d), dtype=q.dtype, device=q.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    fa_fwd_strided(q, k, v, o, lse, B, H, N, d, _default_scale(d, scale), causal,
                   _strides_bnhd(q), _strides_bnhd(k), _strides_bnhd(v), _strides_bnhd(o), stream)
    return o, lse


def attention_qkvpacked(qkv, causal=False, scale=None, stream=None):
    """O [B, N, H, d] and LSE [B, H, N] for a packed qkv tensor of shape [B, N, 3, H, d]."""
    B, N, three, H, d = qkv.shape
    if three != 3:
        raise ValueError("qkv must be [B, N, 3, H, d]")
    return attention_bnhd(qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2], causal, scale, stream)


def attention_varlen(q, k, v, cu_seqlens, max_seqlen, causal=False, scale=None, stream=None):
    """O [T, H, d] and LSE [H, T] for packed sequences q, k, v of shape [T, H, d]."""
    _same(q, k, v)
    _contiguous(q=q, k=k, v=v)
    T, H, d = q.shape
    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int32 tensor")
    if cu_seqlens.device != q.device:
        raise ValueError("cu_seqlens must live on q's device")
    B = cu_seqlens.numel() - 1
    o = torch.empty_like(q, memory_format=torch.contiguous_format)
    lse = torch.empty((H, T), dtype=torch.float32, device=q.device)
    fa_fwd_varlen(q, k, v, o, lse, cu_seqlens, B, T, int(max_seqlen), H, d,
                  _default_scale(d, scale), causal, stream)
    return o, lse


def attention_backward(q, k, v, o, lse, do, causal=False, scale=None, stream=None):
    """dq, dk, dv for contiguous [B, H, N, d] tensors and the forward's LSE."""
    _same(q, k, v, o, do)
    _contiguous(q=q, k=k, v=v, o=o, do=do)
    B, H, N, d = q.shape
    _check_lse(lse, B, H, N, q)
    dq, dk, dv = (torch.empty_like(t, memory_format=torch.contiguous_format) for t in (q, k, v))
    ws = torch.empty(max(fa_bwd_workspace_bytes(B, H, N, d), 16), dtype=torch.uint8, device=q.device)
    fa_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, B, H, N, d, _default_scale(d, scale), causal, stream)
    return dq, dk, dv


def attention_fa1_order(q, k, v, causal=False, scale=None, stream=None):
    """The FlashAttention-1 loop order (ablation); same result as ``attention``."""
    _same(q, k, v)
    _contiguous(q=q, k=k, v=v)
    B, H, N, d = q.shape
    o = torch.empty_like(q, memory_format=torch.contiguous_format)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    ws = torch.empty(max(fa_fwd_fa1_workspace_bytes(B, H, N, d), 16), dtype=torch.uint8, device=q.device)
    fa_fwd_fa1_order(q, k, v, o, lse, ws, B, H, N, d, _default_scale(d, scale), causal, stream)
    return o, lse
