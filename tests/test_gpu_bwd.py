"""GPU parity of the backward pass (fa_bwd) against the fp64 oracle's
derivatives, on the same input bits.

Gate: |g - g_ref| <= 8 u S + ulp(g_ref)/2 per element, u being the unit
roundoff of the 16-bit type (2^-11 fp16, 2^-8 bf16): P and dS enter the
products rounded to 16 bits and each gradient element sums N such products,
so its error is a few units of u relative to the gradient's scale
S = max(max|g_ref|, F). F covers gradients that vanish by cancellation (one
key: dS = P (dP - D) with dP = D exactly): there the GPU keeps the fp32
rounding of the two equal terms, at most ~2^-20 d max|dO| max|V| each, times
d max(|Q|, |K|) |scale| through the last product.
"""
import numpy as np
import pytest
import torch

import oracle
import parity as P
import exact_attention_fa2_amd as fa
from exact_attention_fa2_amd import inputs

pytestmark = pytest.mark.gpu

U = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}


def gate_grad(g, ref, dtype, name, floor=0.0):
    err = np.abs(g - ref)
    scale = max(np.abs(ref).max(), floor)
    bound = 8 * U[dtype] * scale + 0.5 * P.ulp(ref, dtype)
    worst = float((err / np.maximum(scale, 1e-30)).max())
    assert (err <= bound).all(), f"{name}: max err {err.max():.3e} (rel {worst:.2e}), scale {scale:.3e}"
    return worst


def run(B, H, N, d, dtype, causal, seed, sigma_qk=1.0, scale=None):
    print(f"[fa_bwd] B{B} H{H} N{N} d{d} {dtype} causal={causal} seed={seed}", flush=True)
    q, k, v = inputs.make_qkv(B, H, N, d, dtype, seed, sigma_qk)
    do = inputs.make_like(q, seed + 1000)
    sc = d ** -0.5 if scale is None else scale
    qg, kg, vg, dog = (t.cuda() for t in (q, k, v, do))
    o, lse = fa.attention(qg, kg, vg, causal=causal, scale=sc)
    dq, dk, dv = fa.attention_backward(qg, kg, vg, o, lse, dog, causal=causal, scale=sc)
    torch.cuda.synchronize()
    qd, kd, vd, dod = (P.decode(x, dtype) for x in (q, k, v, do))
    rq, rk, rv = oracle.attention_bwd(qd, kd, vd, dod, sc, causal)
    amax = lambda x: float(np.abs(x).max())
    floor = 2.0 ** -20 * d * amax(dod) * amax(vd) * d * max(amax(qd), amax(kd)) * abs(sc)
    out = {}
    for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        out[name] = gate_grad(P.to64(g), r, dtype, name, floor)
    print("  rel errors", {k2: f"{v2:.2e}" for k2, v2 in out.items()}, flush=True)
    return out


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d,dtype", [(1, 64, "f16"), (64, 64, "bf16"), (200, 64, "f16"), (400, 64, "bf16"),
                                       (129, 128, "f16"), (300, 128, "bf16"), (97, 96, "f16"), (1000, 64, "f16"),
                                       (700, 128, "bf16"), (333, 96, "bf16"), (1030, 96, "f16"),
                                       (130, 256, "f16"), (300, 256, "bf16")])
def test_bwd_matches_oracle(N, d, dtype, causal):
    run(2, 2, N, d, dtype, causal, seed=N + d)


def test_bwd_scale_variants():
    run(1, 2, 150, 64, "f16", False, seed=7, scale=-0.1)
    run(1, 2, 150, 64, "bf16", True, seed=8, scale=0.3, sigma_qk=2.0)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_d128_negative_scale(causal):
    # d = 128 folds the sign of the scale into K and into dK's final multiply
    run(1, 2, 300, 128, "bf16", causal, seed=11, scale=-0.09)
    run(1, 1, 513, 128, "f16", causal, seed=12, scale=-0.2)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_d256(causal):
    # one wave per SIMD, accumulation registers as overflow; several key and
    # query blocks with a ragged tail, and a negative scale (K read
    # sign-flipped, dK multiplied by it at the end)
    run(1, 2, 517, 256, "bf16", causal, seed=13, scale=-0.0625)
    run(2, 1, 1100, 256, "f16", causal, seed=14, sigma_qk=2.0)


def test_bwd_deterministic():
    q, k, v = (t.cuda() for t in inputs.make_qkv(1, 4, 500, 64, "bf16", 9))
    do = inputs.make_like(q.cpu(), 10).cuda()
    o, lse = fa.attention(q, k, v, causal=True)
    g1 = fa.attention_backward(q, k, v, o, lse, do, causal=True)
    g2 = fa.attention_backward(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(g1, g2))


def run_sampled_heads(B, H, N, d, dtype, causal, seed, scale, sigma_qk=1.0, sigma_v=1.0):
    # all heads on the GPU, whole (batch, head) slices compared with the
    # oracle: the first, the last and one seeded head
    q, k, v = inputs.make_qkv(B, H, N, d, dtype, seed, sigma_qk, sigma_v)
    do = inputs.make_like(q, seed + 1000)
    qg, kg, vg, dog = (t.cuda() for t in (q, k, v, do))
    o, lse = fa.attention(qg, kg, vg, causal=causal, scale=scale)
    dq, dk, dv = fa.attention_backward(qg, kg, vg, o, lse, dog, causal=causal, scale=scale)
    torch.cuda.synchronize()
    grads = [P.to64(g) for g in (dq, dk, dv)]
    assert all(np.isfinite(g).all() for g in grads)
    rng = np.random.default_rng(7)
    heads = {(0, 0), (B - 1, H - 1), (int(rng.integers(B)), int(rng.integers(H)))}
    for b, h in sorted(heads):
        qd, kd, vd, dod = (P.decode(x[b:b + 1, h:h + 1], dtype) for x in (q, k, v, do))
        refs = oracle.attention_bwd(qd, kd, vd, dod, scale, causal)
        amax = lambda x: float(np.abs(x).max())
        floor = 2.0 ** -20 * d * amax(dod) * amax(vd) * d * max(amax(qd), amax(kd)) * abs(scale)
        rel = {}
        for gname, g, r in zip(("dq", "dk", "dv"), grads, refs):
            rel[gname] = gate_grad(g[b:b + 1, h:h + 1], r, dtype, f"{gname} head ({b},{h})", floor)
        print(f"  head ({b},{h}) rel errors", {k2: f"{v2:.2e}" for k2, v2 in rel.items()}, flush=True)


@pytest.mark.parametrize("name", ["n400_batched", "n4096", "n8192_causal"])
def test_bwd_workload_sampled_heads(name):
    # the backward at the benchmarked size, launched exactly as bench.py times it
    w = inputs.WORKLOADS[name]
    print(f"[fa_bwd] workload {name}: B{w.B} H{w.H} N{w.N} d{w.d} {w.dtype} causal={w.causal}", flush=True)
    run_sampled_heads(w.B, w.H, w.N, w.d, w.dtype, w.causal, 0, w.scale, w.sigma_qk, w.sigma_v)


# Both sides of the switch between the joint grid (at most one dQ block per
# CU, 256 on MI355X: dQ blocks are 128 query rows at d = 64, 96 and 256, 256
# rows at d = 128) and the separate kernels.
@pytest.mark.parametrize("B,H,N,d,dtype,causal", [
    (1, 64, 512, 64, "f16", True),     # 256 dQ blocks: joint
    (1, 65, 512, 64, "f16", True),     # 260: sequence
    (2, 64, 300, 64, "bf16", False),   # 384: sequence
    (1, 32, 2048, 128, "bf16", True),  # 256: joint
    (1, 33, 2048, 128, "f16", False),  # 264: sequence
    (1, 3, 4100, 64, "bf16", False),   # 99 (ragged last block): joint
    (1, 64, 512, 96, "bf16", False),   # 256: joint (three block kinds)
    (1, 64, 600, 96, "f16", True),     # 320: sequence
    (1, 32, 1000, 256, "f16", True),   # 256: joint
    (1, 33, 1000, 256, "bf16", False), # 264: sequence
])
def test_bwd_joint_and_sequence_paths(B, H, N, d, dtype, causal):
    print(f"[fa_bwd] paths B{B} H{H} N{N} d{d} {dtype} causal={causal}", flush=True)
    run_sampled_heads(B, H, N, d, dtype, causal, N + H, d ** -0.5)


def _random_bwd_shapes(n, seed=2027):
    # seeded shapes across the backward's regimes: every head dim it takes,
    # one or several key/query blocks, ragged lengths, both causal modes,
    # larger logits and scales of either sign
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        d = int(rng.choice([64, 96, 128]))
        N = int(rng.integers(1, 140)) if rng.random() < 0.3 else int(rng.integers(140, 1100))
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        sc = float(rng.choice([d ** -0.5, -(d ** -0.5), 0.2]))
        out.append((B, H, N, d, str(rng.choice(["f16", "bf16"])), bool(rng.integers(0, 2)),
                    float(rng.choice([1.0, 2.0])), round(sc, 6)))
    return out


@pytest.mark.parametrize("B,H,N,d,dtype,causal,sigma,scale", _random_bwd_shapes(16))
def test_bwd_random_shapes(B, H, N, d, dtype, causal, sigma, scale):
    run(B, H, N, d, dtype, causal, seed=300 + N, sigma_qk=sigma, scale=scale)
