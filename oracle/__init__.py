"""Plain fp64 CPU oracle for exact attention (forward and backward).

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import this module:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` call it. It shares no code with the HIP library and imports
nothing from it.

Sources (web pages on FlashAttention; cited by title and section):

* "FlashAttention explainer" (aitangshan.cn), section 1: standard attention
  is three steps -- scores Q·Kᵀ, a row softmax scaled by 1/sqrt(d_k) whose
  weights sum to one, then the weighted sum of V rows.
* "YOLO11 attention swapped for a FlashAttention-2-style implementation"
  (discosf.com), section 1.2 (S = Q·Kᵀ, P = softmax(S), O = P·V) and
  section 3.2 (scores divided by sqrt(d); output shaped like q).
* "Why the official YOLOv12 image is fast" (pwwt.cn), section 5: scores are
  ``q @ kᵀ * scale``; the flash call takes ``softmax_scale`` and ``causal``.
* "FlashAttention explainer", section 7.1: the causal mask removes future
  positions.
* "YOLO models integrating Flash Attention" (rkmt.cn): the fused call also
  returns the per-row log-sum-exp.
* "FlashAttention explainer", section 6.2, and "YOLO11 ... FlashAttention-2"
  section 2.3: the backward pass recomputes S and P from Q, K, V and row
  statistics; its gradients are the plain derivatives of the forward map.

The method (tiling + online softmax) reaches exactly the result of the plain
definition up to floating-point order ("FlashAttention explainer" 4.3, 7.2;
"YOLO11 ... FlashAttention-2" 2.2), so this oracle is that definition written
out, one row at a time, in fp64:

    s_ij  = scale * sum_t q_it k_jt            for j in J_i
    m_i   = max_j s_ij
    l_i   = sum_j exp(s_ij - m_i)
    o_it  = sum_j exp(s_ij - m_i) v_jt / l_i
    lse_i = m_i + ln l_i

with J_i = {0..N-1}, or {0..i} when causal (top-left aligned, diagonal kept).
A matrix product from numpy is used as a library step; rows are processed in
chunks only to bound memory (rows are independent by definition).

Every function here is pinned by ``tests/test_oracle_pins.py`` against closed
forms, invariants, a library routine (torch's fp64 scaled-dot-product
attention on the CPU) and an independent blocked online-softmax derivation.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "decode_f16",
    "decode_bf16",
    "decode",
    "attention_fwd",
    "attention_fwd_rows",
    "attention_bwd",
]

_ROW_CHUNK = 1024


# ---------------------------------------------------------------------------
# Input decoding. The GPU consumes fp16 / bf16 bit patterns; the oracle reads
# the same bits and widens them exactly to fp64 (both formats embed exactly).
# ---------------------------------------------------------------------------
def decode_f16(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16)
    sign = np.where((b >> 15) & 1, -1.0, 1.0)
    exp = ((b >> 10) & 0x1F).astype(np.int64)
    man = (b & 0x3FF).astype(np.float64)
    normal = sign * np.ldexp(1.0 + man / 1024.0, exp - 15)
    subnormal = sign * np.ldexp(man, -24)
    special = np.where(man == 0, sign * np.inf, np.nan)
    return np.where(exp == 0, subnormal, np.where(exp == 31, special, normal))


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exact float64 values.

    bfloat16 is the upper half of an IEEE binary32, so the pattern shifted
    left by 16 bits is the binary32 of the same value.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):  # NaN payloads widen to NaN
        return b.view(np.float32).astype(np.float64)


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype in ("f16", "fp16", "float16"):
        return decode_f16(bits)
    if dtype in ("bf16", "bfloat16"):
        return decode_bf16(bits)
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------------------
# Forward
# ---------------------------------------------------------------------------
def _rows_fwd(q_rows, row_idx, k, v, scale, causal):
    """Three passes for a set of query rows of one (batch, head).

    q_rows: [R, d] fp64, row_idx: [R] query positions, k, v: [N, d] fp64.
    """
    n = k.shape[0]
    # pass 1: scores and row max ("FlashAttention explainer" 1, step one)
    s = scale * (q_rows @ k.T)  # [R, N]
    if causal:
        keep = np.arange(n)[None, :] <= np.asarray(row_idx)[:, None]
        s = np.where(keep, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    # pass 2: exponentials and their sum (step two: weights that sum to one)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    # pass 3: weighted sum of V rows (step three)
    o = (p @ v) / l
    lse = m[:, 0] + np.log(l[:, 0])
    return o, lse


def attention_fwd(q, k, v, scale: float, causal: bool):
    """O and LSE for q, k, v of shape [B, H, N, d] (any real dtype, used as fp64).

    Returns (o [B,H,N,d] fp64, lse [B,H,N] fp64, natural log).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = q.shape
    o = np.empty((B, H, N, d))
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            for r0 in range(0, N, _ROW_CHUNK):
                r1 = min(N, r0 + _ROW_CHUNK)
                idx = np.arange(r0, r1)
                o[b, h, r0:r1], lse[b, h, r0:r1] = _rows_fwd(
                    q[b, h, r0:r1], idx, k[b, h], v[b, h], scale, causal)
    return o, lse


def attention_fwd_rows(q, k, v, scale: float, causal: bool, rows):
    """O and LSE for selected rows only.

    rows: int array [R, 3] of (b, h, i). Returns (o [R, d], lse [R]).
    Used to check full-size outputs at sampled positions.
    """
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    d = q.shape[-1]
    o = np.empty((rows.shape[0], d))
    lse = np.empty(rows.shape[0])
    keys = rows[:, 0] * q.shape[1] + rows[:, 1]
    for key in np.unique(keys):
        sel = np.nonzero(keys == key)[0]
        b, h = int(rows[sel[0], 0]), int(rows[sel[0], 1])
        idx = rows[sel, 2]
        qr = np.asarray(q[b, h][idx], dtype=np.float64)
        o[sel], lse[sel] = _rows_fwd(qr, idx, np.asarray(k[b, h], np.float64),
                                     np.asarray(v[b, h], np.float64), scale, causal)
    return o, lse


# ---------------------------------------------------------------------------
# Backward: derivatives of the forward map, recomputing S and P from Q, K, V
# ("FlashAttention explainer" 6.2; "YOLO11 ... FlashAttention-2" 2.3).
#
# For one row, P_i = softmax(s_i). Its Jacobian-vector product is
#   dS_ij = P_ij * (dP_ij - sum_k P_ik dP_ik),  with dP = dO · Vᵀ,
# and with s = scale·Q·Kᵀ:  dQ = scale · dS · K,  dK = scale · dSᵀ · Q,
# while O = P·V gives dV = Pᵀ · dO.
# ---------------------------------------------------------------------------
def attention_bwd(q, k, v, do, scale: float, causal: bool):
    """Gradients (dq, dk, dv) of sum(O * do) for q, k, v, do of shape [B,H,N,d]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, H, N, d = q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, N, _ROW_CHUNK):
                r1 = min(N, r0 + _ROW_CHUNK)
                s = scale * (q[b, h, r0:r1] @ k[b, h].T)
                if causal:
                    keep = np.arange(N)[None, :] <= np.arange(r0, r1)[:, None]
                    s = np.where(keep, s, -np.inf)
                p = np.exp(s - s.max(axis=1, keepdims=True))
                p /= p.sum(axis=1, keepdims=True)
                dp = do[b, h, r0:r1] @ v[b, h].T
                ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                dv[b, h] += p.T @ do[b, h, r0:r1]
                dq[b, h, r0:r1] = scale * (ds @ k[b, h])
                dk[b, h] += scale * (ds.T @ q[b, h, r0:r1])
    return dq, dk, dv
