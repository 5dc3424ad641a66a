"""Work and traffic accounting for the attention forward (host-side, no GPU).

Algorithmic FLOP counts the two matrix products Q·Kᵀ and P·V: 2·N·N·d each
per (batch, head), i.e. 4·B·H·N²·d; under a causal mask only the kept pairs
j <= i are counted, 4·B·H·d·N(N+1)/2. Algorithmic bytes are the one read of
Q, K, V and the one write of O (storage dtype) plus the fp32 LSE: the N×N
score matrix never reaches HBM ("FlashAttention explainer" (aitangshan.cn),
sections 2.1 and 4.2).
"""
from __future__ import annotations

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, vendor figure
MFMA_PEAK_TFLOPS_16BIT = 2516.6  # 256 CU x 4096 flop/clk x 2.4 GHz, dense fp16/bf16


def pairs(N: int, causal: bool) -> int:
    """Number of (query, key) pairs scored per (batch, head)."""
    return N * (N + 1) // 2 if causal else N * N


def alg_flops(B: int, H: int, N: int, d: int, causal: bool) -> int:
    return 4 * B * H * d * pairs(N, causal)


def metric_flops(B: int, H: int, N: int, d: int) -> int:
    """The literal 4·B·H·N²·d of the headline metric (ignores the causal mask)."""
    return 4 * B * H * N * N * d


def alg_bytes(B: int, H: int, N: int, d: int, elem_bytes: int = 2) -> int:
    return 4 * B * H * N * d * elem_bytes + 4 * B * H * N


def alg_bytes_bwd(B: int, H: int, N: int, d: int, elem_bytes: int = 2) -> int:
    """Backward: read Q, K, V, O, dO and LSE once; write dQ, dK, dV once."""
    return 8 * B * H * N * d * elem_bytes + 4 * B * H * N


def num_tiles(n: int, block: int) -> int:
    """Blocks of ``block`` rows needed to cover ``n`` rows (last one ragged)."""
    return (n + block - 1) // block


def score_elems(N: int) -> int:
    """Elements of one N×N score matrix that the fused kernel never stores."""
    return N * N
