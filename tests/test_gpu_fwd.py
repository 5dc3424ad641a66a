"""GPU parity of the forward kernels against the fp64 oracle (same input bits).

Runs through the C ABI (``fa_fwd`` / ``fa_fwd_strided`` / ``fa_fwd_varlen``
via the ctypes binding). Needs an MI355X and the built libfa.so.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import parity as P
import exact_attention_fa2_amd as fa
from exact_attention_fa2_amd import inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def run_case(B, H, N, d, dtype, causal, seed, scale=None, sigma_qk=1.0, sigma_v=1.0, rows=None):
    say(f"[fa_fwd] B{B} H{H} N{N} d{d} {dtype} causal={causal} seed={seed} scale={scale} sqk={sigma_qk}")
    q, k, v = inputs.make_qkv(B, H, N, d, dtype, seed, sigma_qk, sigma_v)
    sc = d ** -0.5 if scale is None else scale
    o, lse = fa.attention(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=sc)
    torch.cuda.synchronize()
    og, lg = P.to64(o), P.to64(lse)
    qd, kd, vd = (P.decode(x, dtype) for x in (q, k, v))
    if rows is None:
        ro, rl = oracle.attention_fwd(qd, kd, vd, sc, causal)
        eo = P.gate_o(og, ro, dtype)
        el = P.gate_lse(lg, rl)
    else:
        ro, rl = oracle.attention_fwd_rows(qd, kd, vd, sc, causal, rows)
        eo = P.gate_o(og[rows[:, 0], rows[:, 1], rows[:, 2]], ro, dtype)
        el = P.gate_lse(lg[rows[:, 0], rows[:, 1], rows[:, 2]], rl)
    assert np.isfinite(og).all() and np.isfinite(lg).all()
    return eo, el


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
def test_workload_parity(name, seed):
    # small workloads: every row against the oracle; large ones: ~400 sampled
    # rows touching every head, plus one whole (batch, head) slice per seed
    # (all of its rows, which at N=8192 causal is every tile shape of the
    # 8-wave d=128 kernel), from the same launch
    w = inputs.WORKLOADS[name]
    say(f"[fa_fwd] workload {name} seed {seed}: {w.describe()}")
    q, k, v = inputs.make_workload(w, seed)
    o, lse = fa.attention(q.to(DEV), k.to(DEV), v.to(DEV), causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    og, lg = P.to64(o), P.to64(lse)
    assert np.isfinite(og).all() and np.isfinite(lg).all()
    qd, kd, vd = (P.decode(x, w.dtype) for x in (q, k, v))
    if w.B * w.H * w.N * w.N <= 64 * 400 * 400 * 4:
        ro, rl = oracle.attention_fwd(qd, kd, vd, w.scale, w.causal)
        eo, el = P.gate_o(og, ro, w.dtype), P.gate_lse(lg, rl)
        strict = P.LAST_STRICT["held"]
        say(f"  {name} seed {seed}: all rows: max|dO| {eo:.3e} (plain max-abs {P.ATOL[w.dtype]:g} "
            f"{'held' if strict else 'exceeded: ulp allowance used'})  max|dLSE| {el:.3e}")
        return
    rows = P.sample_rows(w.B, w.H, w.N, 384, seed)
    ro, rl = oracle.attention_fwd_rows(qd, kd, vd, w.scale, w.causal, rows)
    eo = P.gate_o(og[rows[:, 0], rows[:, 1], rows[:, 2]], ro, w.dtype)
    strict = P.LAST_STRICT["held"]
    el = P.gate_lse(lg[rows[:, 0], rows[:, 1], rows[:, 2]], rl)
    say(f"  {name} seed {seed}: {len(rows)} sampled rows: max|dO| {eo:.3e} (plain max-abs "
        f"{P.ATOL[w.dtype]:g} {'held' if strict else 'exceeded: ulp allowance used'})  max|dLSE| {el:.3e}")
    b, h = seed % w.B, (5 * seed + 3) % w.H
    ro, rl = oracle.attention_fwd(qd[b:b + 1, h:h + 1], kd[b:b + 1, h:h + 1], vd[b:b + 1, h:h + 1], w.scale,
                                  w.causal)
    eo = P.gate_o(og[b:b + 1, h:h + 1], ro, w.dtype, what=f"O head ({b},{h})")
    strict = P.LAST_STRICT["held"]
    el = P.gate_lse(lg[b:b + 1, h:h + 1], rl)
    say(f"  {name} seed {seed}: whole head ({b},{h}), {w.N} rows: max|dO| {eo:.3e} (plain max-abs "
        f"{P.ATOL[w.dtype]:g} {'held' if strict else 'exceeded: ulp allowance used'})  max|dLSE| {el:.3e}")


# The dispatch runs the key-split kernel (one workgroup per 32-row unit, keys
# split over 4 waves) while B*H*ceil(N/32) is at most 512 (d=64) or 256
# (d=96 and 256, padded rows; d=128), and the main kernel past that; at d=64 it splits
# over 8 waves while that count is at most 256 and N >= 1024. Both sides of each boundary,
# against the oracle; long rows split over the waves with large logits
# (rescales in the merge), and short sequences that leave waves without keys.
@pytest.mark.parametrize("H,N,d,dtype,causal", [
    (32, 512, 64, "f16", False), (32, 513, 64, "bf16", True),
    (8, 1024, 128, "bf16", False), (8, 1025, 128, "f16", True),
    (2, 4096, 64, "bf16", False), (1, 3000, 64, "f16", True), (2, 4096, 128, "bf16", True),
    (3, 100, 64, "bf16", True), (4, 192, 128, "f16", False),
    (8, 1024, 64, "bf16", False), (8, 1025, 64, "f16", True), (8, 1023, 64, "f16", False),
    (1, 1024, 64, "bf16", True), (1, 8192, 64, "f16", False),
    (4, 400, 64, "f16", False), (2, 1000, 64, "bf16", True), (8, 1000, 64, "f16", False),
    (8, 1024, 96, "f16", False), (8, 1025, 96, "bf16", True), (1, 5000, 96, "bf16", False),
    (3, 100, 96, "f16", True), (2, 2100, 96, "f16", True),
    (4, 1024, 256, "bf16", False), (8, 1024, 256, "f16", True), (1, 6400, 256, "f16", False),
    (9, 1000, 256, "bf16", False), (2, 100, 256, "bf16", True)])
def test_key_split_path(H, N, d, dtype, causal):
    rows = P.sample_rows(1, H, N, 300, H + N) if H * N * N > 4 * 1024 * 1024 else None
    run_case(1, H, N, d, dtype, causal, 40 + H, None, 2.5, 1.0, rows)


@pytest.mark.parametrize("B,H,N,d,dtype", [(2, 8, 8192, 64, "f16"), (1, 16, 8200, 128, "bf16"),
                                           (1, 12, 4096, 128, "bf16"), (3, 8, 2000, 64, "bf16")])
def test_causal_block_orders(B, H, N, d, dtype):
    # causal launches order blocks by rank across heads; B*H a multiple of 16
    # with 32+ blocks a head takes the heads in pairs per XCD (the first two
    # shapes), other head counts the plain rank order (the last two)
    rows = P.sample_rows(B, H, N, 300, B * H + N)
    run_case(B, H, N, d, dtype, True, 70 + H, None, 2.0, 1.0, rows)


def test_long_causal_variance3_reading():
    # the other reading of the large-logit workload: variance 3 (sigma = sqrt 3)
    w = inputs.WORKLOADS["n8192_causal"]
    rows = P.sample_rows(w.B, w.H, w.N, 256, 5)
    run_case(w.B, w.H, w.N, w.d, w.dtype, True, 5, None, math.sqrt(3.0), 1.0, rows)


# ---------------------------------------------------------------------------
# ragged and degenerate shapes, every head dim, both dtypes
# ---------------------------------------------------------------------------
EDGE_N = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 257, 400, 401]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", EDGE_N)
def test_edge_lengths_d64(N, causal, dtype):
    run_case(2, 3, N, 64, dtype, causal, seed=N)


@pytest.mark.parametrize("d", [96, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 64, 129, 300])
def test_edge_lengths_other_dims(N, d, causal):
    run_case(1, 3, N, d, "bf16" if d != 96 else "f16", causal, seed=N + d)


@pytest.mark.parametrize("N", [1000, 1537])
def test_multi_block_causal_large_logits(N):
    run_case(1, 4, N, 128, "bf16", True, seed=11, sigma_qk=3.0)
    run_case(1, 4, N, 64, "f16", True, seed=12, sigma_qk=3.0)


def test_scale_variants():
    run_case(1, 2, 130, 64, "f16", False, seed=3, scale=0.0)
    run_case(1, 2, 130, 64, "f16", True, seed=3, scale=0.0)
    run_case(1, 2, 130, 64, "f16", False, seed=4, scale=-0.2)
    run_case(1, 2, 130, 128, "bf16", True, seed=4, scale=-0.05)
    run_case(1, 2, 97, 64, "bf16", False, seed=5, scale=1.0)


# ---------------------------------------------------------------------------
# identities on the GPU
# ---------------------------------------------------------------------------
def _gpu(q, k, v, causal, scale):
    o, lse = fa.attention(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_constant_v_is_returned(dtype, causal):
    say(f"[identity] constant V {dtype} causal={causal}")
    q, k, _ = inputs.make_qkv(1, 4, 1000, 128, dtype, 21, sigma_qk=3.0)
    c = inputs.make_like(torch.empty(128, dtype=q.dtype), 22)
    v = c.expand(1, 4, 1000, 128).contiguous()
    o, _ = _gpu(q, k, v, causal, 128 ** -0.5)
    ref = v.to(torch.float64).numpy()
    err = np.abs(P.to64(o) - ref)
    assert (err <= P.ulp(ref, dtype)).all(), err.max()


@pytest.mark.parametrize("causal", [False, True])
def test_q_zero_gives_mean(causal):
    say(f"[identity] Q=0 causal={causal}")
    _, k, v = inputs.make_qkv(2, 2, 400, 64, "f16", 31)
    q = torch.zeros_like(k)
    o, lse = _gpu(q, k, v, causal, 0.125)
    vv = v.to(torch.float64).numpy()
    if causal:
        mean = np.cumsum(vv, axis=2) / np.arange(1, 401)[None, None, :, None]
        lse_ref = np.log(np.arange(1, 401))[None, None]
    else:
        mean = np.broadcast_to(vv.mean(axis=2, keepdims=True), vv.shape)
        lse_ref = np.full((1, 1, 400), math.log(400))
    P.gate_o(P.to64(o), mean, "f16")
    P.gate_lse(P.to64(lse), np.broadcast_to(lse_ref, (2, 2, 400)))


def test_causal_row0_is_exact():
    say("[identity] causal row 0")
    q, k, v = inputs.make_qkv(1, 3, 777, 128, "bf16", 41, sigma_qk=3.0)
    o, lse = _gpu(q, k, v, True, 128 ** -0.5)
    assert torch.equal(o[:, :, 0], v[:, :, 0])
    s0 = (q[0, :, 0].double() * k[0, :, 0].double()).sum(-1) * 128 ** -0.5
    assert np.allclose(lse[0, :, 0].double().numpy(), s0.numpy(), atol=1e-4)


def test_dominant_score_selects_row():
    say("[identity] dominant score")
    N, d = 300, 64
    q = torch.zeros(1, 1, N, d)
    k = torch.randn(1, 1, N, d, generator=torch.Generator().manual_seed(3)) * 0.01
    q[..., 0] = 1.0
    k[0, 0, 123] = 0.0
    k[0, 0, 123, 0] = 30.0 / 0.125
    v = torch.randn(1, 1, N, d, generator=torch.Generator().manual_seed(4))
    q, k, v = q.half(), k.half(), v.half()
    o, _ = _gpu(q, k, v, False, 0.125)
    ref = np.broadcast_to(v[0, 0, 123].double().numpy(), (N, d))
    P.gate_o(P.to64(o[0, 0]), ref, "f16")


@pytest.mark.parametrize("H", [2, 64])
@pytest.mark.parametrize("jump", [18.0, 40.0])
def test_bf16_late_dominant_key(jump, H):
    # One late key scores `jump` (natural-log units) above every other key, so
    # its weight relative to the first tile's reference is about 2^(1.44 jump):
    # 2^26 at 18 (accepted under the 2^32 bf16 cap, no redo) and 2^58 at 40
    # (a redo and a rescale). Either way O and LSE must match the oracle.
    # H=2 runs the key-split kernel, H=64 the main kernel with the weight sums
    # by MFMA (its range check on the fp32 sums); the first and last heads are
    # compared.
    say(f"[bf16] late dominant key, jump {jump}, H {H}")
    N, d, sc = 1000, 64, 0.125
    g = torch.Generator().manual_seed(11)
    q = torch.zeros(1, H, N, d)
    q[..., 0] = 1.0
    k = torch.randn(1, H, N, d, generator=g) * 0.05
    k[0, :, 900] = 0.0
    k[0, :, 900, 0] = jump / sc
    v = torch.randn(1, H, N, d, generator=g)
    q, k, v = q.bfloat16(), k.bfloat16(), v.bfloat16()
    o, lse = _gpu(q, k, v, False, sc)
    og, lg = P.to64(o), P.to64(lse)
    for h in sorted({0, H - 1}):
        qd, kd, vd = (P.decode(x[:, h:h + 1], "bf16") for x in (q, k, v))
        ro, rl = oracle.attention_fwd(qd, kd, vd, sc, False)
        P.gate_o(og[:, h:h + 1], ro, "bf16")
        P.gate_lse(lg[:, h:h + 1], rl)


@pytest.mark.parametrize("B,H,N,sigma", [(16, 8, 400, 3.0), (8, 8, 1000, 1.0), (4, 32, 500, 2.5)])
def test_bf16_small_grid_mfma_weight_sums(B, H, N, sigma):
    # bf16 d=64 grids of at most 2048 units of 32 rows: the main kernel forms
    # the sums of the 16-bit weights by MFMA; large logits exercise the redo
    rows = P.sample_rows(B, H, N, 300, N)
    run_case(B, H, N, 64, "bf16", False, 60 + B, None, sigma, 1.0, rows)


@pytest.mark.parametrize("B,H,N,dtype,causal,sigma", [
    (3, 181, 100, "f16", False, 1.0), (2, 150, 128, "bf16", True, 3.0), (4, 70, 65, "bf16", False, 2.0),
    (5, 111, 64, "bf16", True, 3.0), (7, 80, 17, "f16", False, 1.0), (1, 601, 1, "bf16", False, 1.0),
    (3, 95, 33, "f16", True, 1.0), (9, 57, 32, "bf16", False, 2.5)])
def test_head_packed_short_maps(B, H, N, dtype, causal, sigma):
    # d=64 maps of at most 128 rows on grids past the key-split (more than 512
    # units of 32 rows) and 4-wave (256+ heads) limits: 2 heads per workgroup,
    # 4 up to 64 rows; head counts that leave the last workgroup partly empty
    units = B * H * ((N + 31) // 32)
    assert units > 512 and B * H >= 256, "shape must reach the head-packed kernel"
    run_case(B, H, N, 64, dtype, causal, 90 + N, None, sigma, 1.0)


@pytest.mark.parametrize("B,H,N,dtype,sigma", [
    (8, 16, 400, "bf16", 3.0), (32, 8, 256, "f16", 1.0), (2, 64, 333, "f16", 1.0), (4, 32, 500, "bf16", 2.5),
    (8, 8, 1000, "f16", 1.0), (4, 16, 1000, "bf16", 3.0), (1, 300, 129, "bf16", 1.0), (2, 70, 401, "f16", 2.0)])
def test_causal_16_row_units(B, H, N, dtype, sigma):
    # causal d=64 grids of 513..2048 units of 32 rows with 256+ workgroups of
    # 256 rows: 16-row units (16x16x32 MFMAs) in 4-wave workgroups; ragged
    # ends at 1, 15, 16 and 17 rows past a 64-key tile
    units = B * H * ((N + 31) // 32)
    assert 512 < units <= 2048 and B * H * ((N + 255) // 256) >= 256, "shape must reach the 16-row kernel"
    rows = P.sample_rows(B, H, N, 400, N) if B * H * N * N > 40_000_000 else None
    eo, el = run_case(B, H, N, 64, dtype, True, 110 + N, None, sigma, 1.0, rows)
    if rows is not None:
        # one whole head too, from a launch of the same grid
        q, k, v = inputs.make_qkv(B, H, N, 64, dtype, 110 + N, sigma, 1.0)
        o, lse = fa.attention(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, scale=64 ** -0.5)
        torch.cuda.synchronize()
        b, h = B - 1, H // 2
        qd, kd, vd = (P.decode(x[b:b + 1, h:h + 1], dtype) for x in (q, k, v))
        ro, rl = oracle.attention_fwd(qd, kd, vd, 64 ** -0.5, True)
        P.gate_o(P.to64(o)[b:b + 1, h:h + 1], ro, dtype)
        P.gate_lse(P.to64(lse)[b:b + 1, h:h + 1], rl)


@pytest.mark.parametrize("B,H,N,dtype,causal", [
    (1, 256, 128, "bf16", False),   # head-packed, 2 heads a workgroup, at its 128-row limit
    (1, 256, 129, "f16", False),    # one row past it: the 8-wave main kernel
    (1, 256, 129, "bf16", False),   # ... or, bf16, the kernel with MFMA weight sums
    (1, 257, 64, "f16", True),      # head-packed, 4 heads a workgroup, 513 units of 32 rows
    (1, 256, 64, "bf16", False),    # 512 units: still the key-split kernel
    (1, 157, 400, "bf16", True),    # causal, 2041 units: 16-row kernel
    (1, 158, 400, "f16", True),     # causal, 2054 units: the 8-wave main kernel
    (1, 255, 256, "f16", False),    # 255 workgroups of 256 rows: the 4-wave main kernel
    (1, 128, 512, "bf16", True)])   # causal, 2048 units, 256 workgroups of 256 rows: 16-row kernel
def test_dispatch_boundaries(B, H, N, dtype, causal):
    # shapes on either side of each d=64 dispatch bound, against the oracle
    # on 400 sampled rows (every head) plus one whole head
    rows = P.sample_rows(B, H, N, 400, B * H + N)
    run_case(B, H, N, 64, dtype, causal, 130 + H, None, 2.0, 1.0, rows)
    q, k, v = inputs.make_qkv(B, H, N, 64, dtype, 130 + H, 2.0, 1.0)
    o, lse = fa.attention(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=64 ** -0.5)
    torch.cuda.synchronize()
    h = H - 1
    qd, kd, vd = (P.decode(x[:, h:h + 1], dtype) for x in (q, k, v))
    ro, rl = oracle.attention_fwd(qd, kd, vd, 64 ** -0.5, causal)
    P.gate_o(P.to64(o)[:, h:h + 1], ro, dtype)
    P.gate_lse(P.to64(lse)[:, h:h + 1], rl)


def _random_shapes(n, seed=2026):
    # seeded shapes over the dispatch regimes: few or many heads, short or
    # long rows, ragged lengths, both head dims of the short-map kernels
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        d = int(rng.choice([64, 128]))
        N = int(rng.choice([int(rng.integers(1, 130)), int(rng.integers(130, 1100))]))
        BH = int(rng.choice([int(rng.integers(1, 40)), int(rng.integers(200, 700))]))
        if BH * N * d > 40_000_000:
            continue
        B = int(rng.integers(1, 4))
        H = max(1, BH // B)
        out.append((B, H, N, d, str(rng.choice(["f16", "bf16"])), bool(rng.integers(0, 2)),
                    float(rng.choice([1.0, 2.0, 3.0]))))
    return out


@pytest.mark.parametrize("B,H,N,d,dtype,causal,sigma", _random_shapes(24))
def test_random_shapes(B, H, N, d, dtype, causal, sigma):
    rows = P.sample_rows(B, H, N, 300, B * H + N) if B * H * N * N > 4_000_000 else None
    run_case(B, H, N, d, dtype, causal, 170 + N, None, sigma, 1.0, rows)


def test_deterministic():
    q, k, v = (t.to(DEV) for t in inputs.make_qkv(2, 4, 1000, 64, "f16", 51))
    o1, l1 = fa.attention(q, k, v, causal=True)
    o2, l2 = fa.attention(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_side_stream():
    q, k, v = (t.to(DEV) for t in inputs.make_qkv(1, 2, 200, 64, "bf16", 52))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o1, l1 = fa.attention(q, k, v)
    s.synchronize()
    o2, l2 = fa.attention(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ---------------------------------------------------------------------------
# properties that hold at any size, checked on the GPU result
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,causal,sqk", [("f16", False, 1.0), ("bf16", True, 3.0)])
def test_gpu_lse_normalises_rows(dtype, causal, sqk):
    # with the GPU's LSE, sum_j exp(s_ij - LSE_i) over the visible keys is 1
    # (s in fp64 from the same input bits); 1e-3 in LSE allows 1.1e-3 here
    say(f"[property] rows sum to 1 with the GPU LSE, {dtype} causal={causal}")
    B, H, N, d = 1, 4, 700, 64
    q, k, v = inputs.make_qkv(B, H, N, d, dtype, 71, sigma_qk=sqk)
    sc = d ** -0.5
    _, lse = _gpu(q, k, v, causal, sc)
    qd, kd = P.decode(q, dtype), P.decode(k, dtype)
    s = np.einsum("bhid,bhjd->bhij", qd, kd) * sc
    if causal:
        s = np.where(np.tril(np.ones((N, N), dtype=bool)), s, -np.inf)
    tot = np.exp(s - P.to64(lse)[..., None]).sum(-1)
    assert np.abs(tot - 1.0).max() <= 1.1e-3, np.abs(tot - 1.0).max()


def _grid(shape, seed, lo=-4.0, hi=4.0, step=1 / 64):
    # values on a coarse grid: sums and shifts of them stay exact in fp16
    g = torch.Generator().manual_seed(seed)
    n = int(round((hi - lo) / step))
    return (torch.randint(0, n + 1, shape, generator=g).double() * step + lo).half()


def test_gpu_invariants():
    say("[property] key/value permutation, key shift, linearity in V")
    B, H, N, d, sc = 1, 2, 333, 64, 0.125
    q, k, v = (_grid((B, H, N, d), s) for s in (81, 82, 83))
    o, lse = _gpu(q, k, v, False, sc)
    # permuting K and V rows jointly leaves O and LSE unchanged
    perm = torch.randperm(N, generator=torch.Generator().manual_seed(84))
    o_p, lse_p = _gpu(q, k[:, :, perm].contiguous(), v[:, :, perm].contiguous(), False, sc)
    P.gate_o(P.to64(o_p), P.to64(o), "f16")
    P.gate_lse(P.to64(lse_p), P.to64(lse))
    # K_j -> K_j + c for every j: O unchanged, LSE_i shifted by scale <q_i, c>
    cvec = _grid((d,), 85, -1.0, 1.0, 1 / 8)
    o_s, lse_s = _gpu(q, (k.double() + cvec.double()).half(), v, False, sc)
    assert torch.equal((k.double() + cvec.double()).half().double(), k.double() + cvec.double())
    P.gate_o(P.to64(o_s), P.to64(o), "f16")
    shift = (q.double() @ cvec.double()).numpy() * sc
    P.gate_lse(P.to64(lse_s), P.to64(lse) + shift)
    # O is linear in V: O(V1 + V2) = O(V1) + O(V2) (V1 + V2 exact in fp16)
    v2 = _grid((B, H, N, d), 86)
    o_2, _ = _gpu(q, k, v2, False, sc)
    o_12, _ = _gpu(q, k, (v.double() + v2.double()).half(), False, sc)
    ref = P.to64(o) + P.to64(o_2)
    err = np.abs(P.to64(o_12) - ref)
    bound = 3 * P.ATOL["f16"] + 1.5 * P.ulp(ref, "f16")
    assert (err <= bound).all(), float(err.max())


# ---------------------------------------------------------------------------
# layouts at the boundary: [B, N, H, d] and packed QKV [B, N, 3, H, d]
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_bnhd_and_packed_layouts(causal):
    say(f"[fa_fwd_strided] causal={causal}")
    B, N, H, d, dtype = 2, 400, 8, 64, "bf16"
    q, k, v = inputs.make_qkv(B, N, H, d, dtype, 61)  # drawn directly in [B, N, H, d]
    o, lse = fa.attention_bnhd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal)
    torch.cuda.synchronize()
    perm = lambda t: P.decode(t, dtype).transpose(0, 2, 1, 3)
    ro, rl = oracle.attention_fwd(perm(q), perm(k), perm(v), d ** -0.5, causal)
    P.gate_o(P.to64(o).transpose(0, 2, 1, 3), ro, dtype)
    P.gate_lse(P.to64(lse), rl)

    qkv = torch.stack([q, k, v], dim=2).contiguous()  # [B, N, 3, H, d]
    o2, lse2 = fa.attention_qkvpacked(qkv.to(DEV), causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o2.cpu(), o.cpu()) and torch.equal(lse2.cpu(), lse.cpu())


@pytest.mark.parametrize("B,N,H,dtype,causal", [
    (4, 100, 70, "bf16", False),   # head-packed kernel, 2 heads a workgroup
    (3, 60, 90, "f16", True),      # head-packed kernel, 4 heads a workgroup
    (2, 400, 70, "f16", True),     # causal 16-row kernel
    (1, 640, 300, "bf16", False)])  # the 8-wave main kernel
def test_strided_layouts_on_short_map_kernels(B, N, H, dtype, causal):
    # the short-map kernels address Q, K, V and O through the row, head and
    # batch strides: [B, N, H, d] views and packed QKV against the oracle
    say(f"[fa_fwd_strided] short maps B{B} N{N} H{H} {dtype} causal={causal}")
    d = 64
    q, k, v = inputs.make_qkv(B, N, H, d, dtype, 150 + N)  # drawn directly in [B, N, H, d]
    o, lse = fa.attention_bnhd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal)
    torch.cuda.synchronize()
    perm = lambda t: P.decode(t, dtype).transpose(0, 2, 1, 3)
    qd, kd, vd = perm(q), perm(k), perm(v)
    rows = P.sample_rows(B, H, N, 400, N)
    ro, rl = oracle.attention_fwd_rows(qd, kd, vd, d ** -0.5, causal, rows)
    og, lg = P.to64(o).transpose(0, 2, 1, 3), P.to64(lse)
    P.gate_o(og[rows[:, 0], rows[:, 1], rows[:, 2]], ro, dtype)
    P.gate_lse(lg[rows[:, 0], rows[:, 1], rows[:, 2]], rl)
    qkv = torch.stack([q, k, v], dim=2).contiguous()  # [B, N, 3, H, d]
    o2, lse2 = fa.attention_qkvpacked(qkv.to(DEV), causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o2.cpu(), o.cpu()) and torch.equal(lse2.cpu(), lse.cpu())


@pytest.mark.parametrize("d,dtype,causal", [(96, "f16", False), (96, "bf16", True), (256, "bf16", False),
                                            (256, "f16", True)])
def test_strided_layouts_on_padded_key_split(d, dtype, causal):
    # the key-split kernel's padded-row LDS-DMA at d = 96 and 256 reads K and
    # V through the row stride of [B, N, H, d] views and of packed QKV
    B, N, H = 1, 1000, 2
    say(f"[fa_fwd_strided] padded key split B{B} N{N} H{H} d{d} {dtype} causal={causal}")
    q, k, v = inputs.make_qkv(B, N, H, d, dtype, 170 + d)  # drawn directly in [B, N, H, d]
    o, lse = fa.attention_bnhd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal)
    torch.cuda.synchronize()
    perm = lambda t: P.decode(t, dtype).transpose(0, 2, 1, 3)
    qd, kd, vd = perm(q), perm(k), perm(v)
    ro, rl = oracle.attention_fwd(qd, kd, vd, d ** -0.5, causal)
    P.gate_o(P.to64(o).transpose(0, 2, 1, 3), ro, dtype)
    P.gate_lse(P.to64(lse), rl)
    qkv = torch.stack([q, k, v], dim=2).contiguous()  # [B, N, 3, H, d]
    o2, lse2 = fa.attention_qkvpacked(qkv.to(DEV), causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o2.cpu(), o.cpu()) and torch.equal(lse2.cpu(), lse.cpu())


@pytest.mark.parametrize("d", [64, 128])
def test_packed_qkv_pages_shape(d):
    # an 80x80 map with C = 256 channels split into heads of d
    say(f"[fa_fwd_strided] packed qkv N=6400 C=256 d={d}")
    B, N, H = 1, 6400, 256 // d
    g = torch.Generator().manual_seed(71)
    qkv = torch.randn(B, N, 3, H, d, generator=g).half()
    o, lse = fa.attention_qkvpacked(qkv.to(DEV))
    torch.cuda.synchronize()
    rows = P.sample_rows(B, H, N, 128, 71)
    dd = lambda i: P.decode(qkv[:, :, i].contiguous(), "f16").transpose(0, 2, 1, 3)
    ro, rl = oracle.attention_fwd_rows(dd(0), dd(1), dd(2), d ** -0.5, False, rows)
    og = P.to64(o).transpose(0, 2, 1, 3)
    P.gate_o(og[rows[:, 0], rows[:, 1], rows[:, 2]], ro, "f16")
    P.gate_lse(P.to64(lse)[rows[:, 0], rows[:, 1], rows[:, 2]], rl)


# ---------------------------------------------------------------------------
# variable-length packed batches
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("d,dtype", [(96, "f16"), (256, "bf16")])
def test_varlen_padded_key_split(d, dtype):
    # few sequences at d = 96 and 256: the key-split kernel's padded-row path
    # with the rows of each sequence found through cu_seqlens
    seqlens, H = [400, 1, 0, 100, 1000], 1
    say(f"[fa_fwd_varlen] {seqlens} H={H} d={d} {dtype} causal=False/True")
    q, k, v, cu = inputs.make_varlen(seqlens, H, d, dtype, 83)
    qd, kd, vd = (P.decode(x, dtype) for x in (q, k, v))
    for causal in (False, True):
        o, lse = fa.attention_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV), max(seqlens), causal=causal)
        torch.cuda.synchronize()
        og, lg = P.to64(o), P.to64(lse)
        for b, n in enumerate(seqlens):
            if n == 0:
                continue
            s0 = int(cu[b])
            sl = slice(s0, s0 + n)
            t = lambda x: x[sl].transpose(1, 0, 2)[None]
            ro, rl = oracle.attention_fwd(t(qd), t(kd), t(vd), d ** -0.5, causal)
            P.gate_o(og[sl].transpose(1, 0, 2)[None], ro, dtype, what=f"O seq {b}")
            P.gate_lse(lg[:, sl][None], rl)


@pytest.mark.parametrize("seqlens,H", [([400, 0, 37, 129], 2), ([1100, 0, 37, 2000], 1)])
def test_varlen_small_grid(seqlens, H):
    # few sequences: the key-split kernel's varlen path (4 waves per unit;
    # 8 for the second set, whose longest row has 32 tiles)
    say(f"[fa_fwd_varlen] {seqlens} H={H} d=64 bf16 causal=False/True")
    q, k, v, cu = inputs.make_varlen(seqlens, H, 64, "bf16", 82)
    qd, kd, vd = (P.decode(x, "bf16") for x in (q, k, v))
    for causal in (False, True):
        o, lse = fa.attention_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV), max(seqlens), causal=causal)
        torch.cuda.synchronize()
        og, lg = P.to64(o), P.to64(lse)
        for b, n in enumerate(seqlens):
            if n == 0:
                continue
            s0 = int(cu[b])
            sl = slice(s0, s0 + n)
            t = lambda x: x[sl].transpose(1, 0, 2)[None]
            ro, rl = oracle.attention_fwd(t(qd), t(kd), t(vd), 0.125, causal)
            P.gate_o(og[sl].transpose(1, 0, 2)[None], ro, "bf16", what=f"O seq {b}")
            P.gate_lse(lg[:, sl][None], rl)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d,dtype", [(64, "f16"), (128, "bf16")])
def test_varlen(causal, d, dtype):
    seqlens = [400, 1, 100, 129, 0, 64, 1600, 37]
    say(f"[fa_fwd_varlen] {seqlens} d={d} {dtype} causal={causal}")
    H = 4
    q, k, v, cu = inputs.make_varlen(seqlens, H, d, dtype, 81)
    o, lse = fa.attention_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV), max(seqlens), causal=causal)
    torch.cuda.synchronize()
    og, lg = P.to64(o), P.to64(lse)
    qd, kd, vd = (P.decode(x, dtype) for x in (q, k, v))
    for b, n in enumerate(seqlens):
        s0 = int(cu[b])
        if n == 0:
            continue
        sl = slice(s0, s0 + n)
        t = lambda x: x[sl].transpose(1, 0, 2)[None]  # [1, H, n, d]
        ro, rl = oracle.attention_fwd(t(qd), t(kd), t(vd), d ** -0.5, causal)
        P.gate_o(og[sl].transpose(1, 0, 2)[None], ro, dtype, what=f"O seq {b}")
        P.gate_lse(lg[:, sl][None], rl)


# ---------------------------------------------------------------------------
# beyond 2^31 elements per tensor: every offset must be 64-bit
# ---------------------------------------------------------------------------
def test_tensors_beyond_2pow31_elements():
    B, H, N, d = 256, 130, 1024, 64  # 2.18e9 elements, 4.4 GB per tensor
    assert B * H * N * d > 2 ** 31
    say(f"[fa_fwd + fa_bwd] B{B} H{H} N{N} d{d} f16 ({B * H * N * d} elements per tensor)")
    g = torch.Generator(device=DEV).manual_seed(123)
    q, k, v, do = (torch.randn((B, H, N, d), generator=g, device=DEV, dtype=torch.float16) for _ in range(4))
    o, lse = fa.attention(q, k, v)
    # heads at the start, middle and end; the last ones lie wholly past 2^31 elements
    heads = [(0, 0), (B // 2, 7), (B - 1, H - 2), (B - 1, H - 1)]
    for b, h in heads:
        qh, kh, vh = (P.decode(x[b, h][None, None].cpu(), "f16") for x in (q, k, v))
        ro, rl = oracle.attention_fwd(qh, kh, vh, d ** -0.5, False)
        P.gate_o(P.to64(o[b, h][None, None]), ro, "f16", what=f"O head ({b},{h})")
        P.gate_lse(P.to64(lse[b, h][None, None]), rl)
    dq, dk, dv = fa.attention_backward(q, k, v, o, lse, do)
    torch.cuda.synchronize()
    b, h = B - 1, H - 1
    qh, kh, vh, doh = (P.decode(x[b, h][None, None].cpu(), "f16") for x in (q, k, v, do))
    refs = oracle.attention_bwd(qh, kh, vh, doh, d ** -0.5, False)
    for name, gpu, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
        err = np.abs(P.to64(gpu[b, h][None, None]) - ref).max()
        assert err <= 8 * 2.0 ** -11 * np.abs(ref).max() + 2.0 ** -11, (name, err)
