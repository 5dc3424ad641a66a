"""C-ABI checks that need no GPU: the library loads, exports every function
that include/fa.h declares, and rejects bad arguments on the host before any
HIP call (so the fake pointers below are never dereferenced or launched on).
"""
import ctypes
import os
import re

import pytest

import exact_attention_fa2_amd as fa
from exact_attention_fa2_amd import build as fabuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

OK, NULL, DIM, UNSUP, SCALE, ALIGN, LAUNCH, ALIAS, DEVICE, TOO_LARGE = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9
A = 0x7F0000000000  # fake, 16-byte aligned device addresses (never touched)
MB = 1 << 20


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fa.LIB_PATH):
        fabuild.build()
    return fa.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(fa_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_expected_entry_points():
    names = declared_functions()
    for n in ("fa_fwd", "fa_fwd_strided", "fa_fwd_varlen", "fa_bwd", "fa_bwd_workspace_bytes", "fa_bwd_noalloc",
              "fa_fwd_fa1_order", "fa_fwd_fa1_workspace_bytes", "fa_strerror", "fa_version"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    raw = ctypes.CDLL(fa.LIB_PATH)
    for n in declared_functions():
        assert hasattr(raw, n), n
    assert set(declared_functions()) == set(fa._SIGS), "binding signatures out of sync with fa.h"


def test_strerror_and_version(L):
    for code in (OK, NULL, DIM, UNSUP, SCALE, ALIGN, LAUNCH, ALIAS, DEVICE, TOO_LARGE):
        s = L.fa_strerror(code).decode()
        assert s and "unknown" not in s
    assert "unknown" in L.fa_strerror(12345).decode()
    assert L.fa_version() >> 16 == 1


def fwd(L, q=A, k=A + 64 * MB, v=A + 128 * MB, o=A + 192 * MB, lse=A + 256 * MB,
        B=1, H=2, N=64, d=64, scale=0.125, causal=0, dtype=0):
    return L.fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, None)


def test_fwd_argument_errors(L):
    assert fwd(L, q=None) == NULL
    assert fwd(L, lse=None) == NULL
    assert fwd(L, B=-1) == DIM
    assert fwd(L, N=-5) == DIM
    assert fwd(L, d=80) == UNSUP
    assert fwd(L, d=0, N=4) == UNSUP  # only B, H or N may be zero
    assert fwd(L, dtype=2) == UNSUP
    assert fwd(L, scale=float("nan")) == SCALE
    assert fwd(L, scale=float("inf")) == SCALE
    assert fwd(L, q=A + 8) == ALIGN
    assert fwd(L, lse=A + 256 * MB + 2) == ALIGN
    assert fwd(L, B=1 << 20, H=1 << 20, N=1 << 20, d=64) == DIM  # 2^66 elements
    assert fwd(L, o=A + 16) == ALIAS          # o overlaps q
    assert fwd(L, lse=A + 128 * MB + 64) == ALIAS  # lse overlaps v


def test_fwd_zero_sizes_are_noops(L):
    for kw in ({"B": 0}, {"H": 0}, {"N": 0}):
        assert fwd(L, q=None, k=None, v=None, o=None, lse=None, **kw) == OK


def test_fwd_error_precedence(L):
    # size errors are reported before pointer errors, so a bad call never launches
    assert fwd(L, q=None, B=-1) == DIM
    assert fwd(L, q=None, d=48) == UNSUP


def strided(L, strides=None, **kw):
    s = strides or [64 * 8 * 64, 64, 8 * 64] * 4
    args = dict(q=A, k=A + 64 * MB, v=A + 128 * MB, o=A + 192 * MB, lse=A + 256 * MB,
                B=2, H=8, N=64, d=64, scale=0.125, causal=0, dtype=1)
    args.update(kw)
    return L.fa_fwd_strided(args["q"], args["k"], args["v"], args["o"], args["lse"], args["B"], args["H"],
                            args["N"], args["d"], args["scale"], args["causal"], args["dtype"], *s, None)


def test_strided_argument_errors(L):
    s = [64 * 8 * 64, 64, 8 * 64] * 4
    bad = list(s)
    bad[2] = 8 * 64 + 4  # row stride not a multiple of 8 elements
    assert strided(L, bad) == ALIGN
    bad = list(s)
    bad[4] = -64
    assert strided(L, bad) == DIM
    bad = list(s)
    bad[0] = 1 << 62  # far element out of the addressable range
    assert strided(L, bad) == DIM
    for i in (2, 5, 8, 11):  # a row stride past 2^24 elements (32-bit tile offsets)
        bad = list(s)
        bad[i] = (1 << 24) + 8
        assert strided(L, bad) == DIM
    assert strided(L, o=A) == ALIAS
    assert strided(L, v=None) == NULL
    assert strided(L, d=32) == UNSUP


def test_strided_overlap_errors(L):
    s = [64 * 8 * 64, 64, 8 * 64] * 4  # [B, N, H, d] strides, B=2 H=8 N=64 d=64
    span = 2 * 64 * 8 * 64 * 2  # bytes of one such tensor
    assert strided(L) == OK or strided(L) == DEVICE  # a valid call (no GPU here)
    assert strided(L, o=A + span - 16) == ALIAS           # o starts inside q's range
    assert strided(L, lse=A + 64 * MB + 64) == ALIAS      # lse inside k
    assert strided(L, lse=A + 192 * MB + 4) == ALIAS      # lse inside o
    # packed QKV: q, k, v interleaved in one buffer are legal inputs
    pk = [64 * 3 * 8 * 64, 64, 3 * 8 * 64] * 3 + [64 * 8 * 64, 64, 8 * 64]
    assert strided(L, pk, k=A + 8 * 64 * 2, v=A + 2 * 8 * 64 * 2) in (OK, DEVICE)
    # output rows that collide
    for o_st in ([64 * 8 * 64, 64, 32],          # row stride below a row's 64 elements
                 [64 * 8 * 64, 0, 8 * 64],       # head stride 0 with 8 heads
                 [0, 64, 8 * 64],                # batch stride 0 with 2 batches
                 [64 * 8 * 64, 64, 8 * 8]):      # rows of consecutive heads interleave
        bad = s[:9] + o_st
        assert strided(L, bad) == ALIAS, o_st
    # rows that only touch (no shared element) are fine: o as [B, H, N, d]
    assert strided(L, s[:9] + [8 * 64 * 64, 64 * 64, 64]) in (OK, DEVICE)
    # an axis of extent 1 may have any stride
    assert strided(L, s[:9] + [0, 64, 8 * 64], B=1) in (OK, DEVICE)


def test_varlen_argument_errors(L):
    def call(**kw):
        a = dict(q=A, k=A + 64 * MB, v=A + 128 * MB, o=A + 192 * MB, lse=A + 256 * MB, cu=A + 300 * MB,
                 B=3, T=300, maxs=128, H=4, d=64, scale=0.1, causal=1, dtype=0)
        a.update(kw)
        return L.fa_fwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cu"], a["B"], a["T"], a["maxs"],
                               a["H"], a["d"], a["scale"], a["causal"], a["dtype"], None)
    assert call(cu=None) == NULL
    assert call(maxs=-1) == DIM
    assert call(maxs=301) == DIM
    assert call(T=-3) == DIM
    assert call(H=(1 << 24) // 64 + 1) == DIM  # row stride H*d past 2^24
    assert call(B=-1) == DIM
    assert call(B=0) == OK
    assert call(cu=A + 300 * MB + 2) == ALIGN
    assert call(d=40) == UNSUP


def test_python_binding_rejects_cpu_tensors(L):
    import torch
    q = torch.zeros(1, 1, 4, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        fa.attention(q, q, q)
    with pytest.raises(TypeError):
        fa._dtype_code(torch.zeros(1, dtype=torch.float32))


def test_fa1_order_argument_errors(L):
    def call(**kw):
        a = dict(q=A, k=A + 64 * MB, v=A + 128 * MB, o=A + 192 * MB, lse=A + 256 * MB, ws=A + 512 * MB,
                 B=1, H=2, N=64, d=64, scale=0.125, causal=0, dtype=0)
        a.update(kw)
        return L.fa_fwd_fa1_order(a["q"], a["k"], a["v"], a["o"], a["lse"], a["ws"], a["B"], a["H"], a["N"],
                                  a["d"], a["scale"], a["causal"], a["dtype"], None)
    assert call(ws=None) == NULL
    assert call(ws=A + 512 * MB + 4) == ALIGN
    assert call(ws=A + 192 * MB) == ALIAS  # workspace over o
    assert call(d=72) == UNSUP
    assert call(B=0, ws=None) == OK
    assert L.fa_fwd_fa1_workspace_bytes(1, 2, 64, 64) > 0
    assert L.fa_fwd_fa1_workspace_bytes(1, 2, 0, 64) == 0
    assert L.fa_fwd_fa1_workspace_bytes(1, -2, 64, 64) == -1
    assert L.fa_fwd_fa1_workspace_bytes(1, 2, 64, 80) == -1


def test_bwd_argument_errors(L):
    def call(**kw):
        a = dict(q=A, k=A + 64 * MB, v=A + 128 * MB, o=A + 192 * MB, do=A + 256 * MB, lse=A + 320 * MB,
                 dq=A + 384 * MB, dk=A + 448 * MB, dv=A + 512 * MB, ws=A + 576 * MB,
                 B=1, H=2, N=64, d=64, scale=0.125, causal=0, dtype=1)
        a.update(kw)
        return L.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"], a["ws"],
                        a["B"], a["H"], a["N"], a["d"], a["scale"], a["causal"], a["dtype"], None)
    assert call(do=None) == NULL
    assert call(ws=None) == NULL
    assert call(dq=A + 384 * MB + 2) == ALIGN
    assert call(dk=A) == ALIAS            # dk over q
    assert call(dv=A + 448 * MB) == ALIAS  # dv over dk
    assert call(ws=A + 320 * MB) == ALIAS  # workspace over lse
    assert call(d=32) == UNSUP
    assert call(d=256, q=None) == NULL  # d = 256 accepted
    assert call(scale=float("nan")) == SCALE
    assert call(N=0, q=None) == OK
    assert L.fa_bwd_workspace_bytes(2, 3, 100, 64) >= 2 * 3 * 100 * 4
    assert L.fa_bwd_workspace_bytes(2, 3, 0, 64) == 0
    assert L.fa_bwd_workspace_bytes(2, 3, 100, 70) == -1


def test_python_wrappers_check_layout_before_any_gpu_call(L):
    # every check below raises on CPU tensors before the device check, so it
    # would equally stop a bad call before any GPU work
    import torch
    B, H, N, d = 1, 2, 16, 64
    q = torch.zeros(B, H, N, d, dtype=torch.float16)
    bnhd = torch.zeros(B, N, H, d, dtype=torch.float16).transpose(1, 2)  # [B, H, N, d] view, not dense
    lse = torch.zeros(B, H, N, dtype=torch.float32)
    with pytest.raises(ValueError, match="contiguous"):
        fa.attention_backward(q, q, q, bnhd, lse, q)
    with pytest.raises(ValueError, match="contiguous"):
        fa.attention_backward(q, q, q, q, lse, bnhd)
    for bad in (lse.half(), lse.double(), torch.zeros(B, H, N - 1), torch.zeros(B, H, 2 * N)[..., ::2]):
        with pytest.raises(ValueError, match="lse"):
            fa.attention_backward(q, q, q, q, bad, q)
    with pytest.raises(ValueError, match="contiguous"):
        fa.attention_fa1_order(bnhd, bnhd, bnhd)
    T = 16
    qt = torch.zeros(T, H, d, dtype=torch.float16)
    cu = torch.tensor([0, T], dtype=torch.int32)
    with pytest.raises(ValueError, match="contiguous"):
        fa.attention_varlen(qt, torch.zeros(H, T, d, dtype=torch.float16).transpose(0, 1), qt, cu, T)
    # the raw entry points check element counts and the fp32 LSE
    o = torch.empty_like(q)
    with pytest.raises(ValueError, match="lse"):
        fa.fa_fwd(q, q, q, o, lse.half(), B, H, N, d, 0.125, False)
    with pytest.raises(ValueError, match="elements"):
        fa.fa_fwd(q, q, q, o, lse, B, H, 2 * N, d, 0.125, False)
    with pytest.raises(ValueError, match="contiguous"):
        fa.fa_fwd(q, q, q, bnhd, lse, B, H, N, d, 0.125, False)
    with pytest.raises(ValueError, match="elements"):
        fa.fa_bwd(q, q, q, q, q, lse, q, q, q, None, B, H, N + 1, d, 0.125, False)
    with pytest.raises(ValueError, match="cu_seqlens"):
        fa.fa_fwd_varlen(qt, qt, qt, qt, torch.zeros(H, T), cu.long(), 1, T, T, H, d, 0.125, False)
    # outputs of the wrappers are dense whatever the inputs' memory format
    x = torch.zeros(1, 2, 4, 64, dtype=torch.float16).to(memory_format=torch.channels_last)
    assert not x.is_contiguous() and torch.empty_like(x, memory_format=torch.contiguous_format).is_contiguous()


def test_bwd_noalloc_argument_errors(L):
    def call(**kw):
        a = dict(q=A, k=A + 64 * MB, v=A + 128 * MB, o=A + 192 * MB, do=A + 256 * MB, lse=A + 320 * MB,
                 dq=A + 384 * MB, dk=A + 448 * MB, dv=A + 512 * MB,
                 B=1, H=2, N=64, d=64, scale=0.125, causal=0, dtype=1)
        a.update(kw)
        return L.fa_bwd_noalloc(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"],
                                a["B"], a["H"], a["N"], a["d"], a["scale"], a["causal"], a["dtype"], None)
    assert fa.BWD_NOALLOC_MAX_ROWS == 4194304
    assert "#define FA_BWD_NOALLOC_MAX_ROWS 4194304" in open(HEADER).read()
    # B*H*N one past the static array is refused with the sizes, before any pointer
    n = fa.BWD_NOALLOC_MAX_ROWS // 64 + 1
    assert call(H=64, N=n, q=None) == TOO_LARGE
    assert call(H=64, N=fa.BWD_NOALLOC_MAX_ROWS // 64, q=None) == NULL  # at the limit: size accepted
    assert call(do=None) == NULL
    assert call(dq=A + 384 * MB + 2) == ALIGN
    assert call(dk=A) == ALIAS
    assert call(dv=A + 448 * MB) == ALIAS
    assert call(d=32) == UNSUP
    assert call(d=256, q=None) == NULL  # d = 256 accepted
    assert call(scale=float("inf")) == SCALE
    assert call(N=0, q=None) == OK
    assert call() == DEVICE  # valid arguments, no GPU in this process
