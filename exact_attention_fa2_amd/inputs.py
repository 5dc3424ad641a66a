"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module holds no attention arithmetic: it only draws Gaussian numbers
from a seeded CPU generator and rounds them to fp16 / bf16. Both the HIP
path and the fp64 oracle then consume the very same bit patterns.

Recipe: ``torch.Generator('cpu').manual_seed(seed)``; draw fp32 ``randn`` of
shape [B, H, N, d] for Q, then K, then V; multiply Q and K by ``sigma_qk`` and
V by ``sigma_v``; round to the storage dtype with round-to-nearest-even.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

_DT = {"f16": torch.float16, "bf16": torch.bfloat16}


def torch_dtype(dtype: str) -> torch.dtype:
    return _DT[dtype]


@dataclass(frozen=True)
class Workload:
    """One attention forward problem (shapes as in the pages' feature maps)."""

    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str
    causal: bool
    sigma_qk: float = 1.0
    sigma_v: float = 1.0

    @property
    def scale(self) -> float:
        return self.d ** -0.5

    def describe(self) -> str:
        return (f"B{self.B} H{self.H} N{self.N} d{self.d} {self.dtype} "
                f"{'causal' if self.causal else 'non-causal'} sigma_qk={self.sigma_qk}")


# The five workloads: a 20x20 map (N=400) small and batched, an 80x80 map
# (N=6400), 64x64 patch tokens (N=4096) and a long causal sequence (N=8192,
# d=128) whose Q and K have standard deviation 3 to stress the rescale.
WORKLOADS = {
    "n400_small": Workload("n400_small", 1, 4, 400, 64, "f16", False),
    "n400_batched": Workload("n400_batched", 16, 8, 400, 64, "bf16", False),
    "n6400": Workload("n6400", 4, 4, 6400, 64, "f16", False),
    "n4096": Workload("n4096", 4, 16, 4096, 64, "f16", False),
    "n8192_causal": Workload("n8192_causal", 1, 32, 8192, 128, "bf16", True, 3.0, 1.0),
}


# A packed batch of feature maps of four sizes (10x10, 20x20, 40x40, 80x80),
# four of each, for the variable-length entry point.
VARLEN_MIX = {"name": "varlen_mix", "seqlens": [100, 400, 1600, 6400] * 4, "H": 4, "d": 64,
              "dtype": "f16", "causal": False}


def make_qkv(B: int, H: int, N: int, d: int, dtype: str, seed: int,
             sigma_qk: float = 1.0, sigma_v: float = 1.0):
    """Seeded Q, K, V as contiguous CPU tensors [B, H, N, d] of ``dtype``."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    shape = (B, H, N, d)
    q = torch.randn(shape, generator=g, dtype=torch.float32) * sigma_qk
    k = torch.randn(shape, generator=g, dtype=torch.float32) * sigma_qk
    v = torch.randn(shape, generator=g, dtype=torch.float32) * sigma_v
    t = _DT[dtype]
    return q.to(t), k.to(t), v.to(t)


def make_workload(w: Workload, seed: int):
    return make_qkv(w.B, w.H, w.N, w.d, w.dtype, seed, w.sigma_qk, w.sigma_v)


def make_like(x: torch.Tensor, seed: int, sigma: float = 1.0) -> torch.Tensor:
    """A seeded Gaussian tensor with the shape and dtype of ``x`` (CPU)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    return (torch.randn(tuple(x.shape), generator=g, dtype=torch.float32) * sigma).to(x.dtype)


def make_varlen(seqlens, H: int, d: int, dtype: str, seed: int, sigma_qk: float = 1.0):
    """Packed variable-length batch: Q, K, V of shape [T, H, d] and cu_seqlens [B+1]."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    T = int(sum(seqlens))
    t = _DT[dtype]
    q = (torch.randn((T, H, d), generator=g) * sigma_qk).to(t)
    k = (torch.randn((T, H, d), generator=g) * sigma_qk).to(t)
    v = torch.randn((T, H, d), generator=g).to(t)
    cu = torch.zeros(len(seqlens) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(list(seqlens), dtype=torch.int64), 0).to(torch.int32)
    return q, k, v, cu


def bits(x: torch.Tensor):
    """The raw 16-bit patterns of a CPU fp16/bf16 tensor as a numpy uint16 array."""
    return x.contiguous().view(torch.int16).numpy().view("uint16")
