"""Pins for the fp64 oracle: checks against things other than itself.

Each test fixes the oracle to a closed form, an invariant of the
mathematics, a library routine, or an independent derivation of the
online-softmax algebra. A final test plants plausible mistakes in a copy of
the oracle (on the CPU) and shows that every one of them fails a pin.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from exact_attention_fa2_amd import accounting, inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(1234)


def rand(*shape, scale=1.0):
    return rng.standard_normal(shape) * scale


# ---------------------------------------------------------------------------
# decoding of the 16-bit inputs
# ---------------------------------------------------------------------------
def test_decode_f16_all_patterns_match_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.decode_f16(bits)
    lib = bits.view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    ok = ~np.isnan(lib)
    assert np.array_equal(ours[ok], lib[ok])
    # signed zeros and infinities keep their sign
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(lib[ok]))


def test_decode_bf16_all_patterns_match_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.decode_bf16(bits)
    lib = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    ok = ~np.isnan(lib)
    assert np.array_equal(ours[ok], lib[ok])


def test_decode_known_values():
    assert oracle.decode_f16(np.array([0x3C00, 0xC000, 0x0001, 0x7BFF], np.uint16)).tolist() == [
        1.0, -2.0, 2.0 ** -24, 65504.0]
    assert oracle.decode_bf16(np.array([0x3F80, 0xC040, 0x0001], np.uint16)).tolist() == [
        1.0, -3.0, 2.0 ** -133]


def test_generator_bits_roundtrip():
    q, k, v = inputs.make_qkv(1, 2, 5, 8, "bf16", seed=3)
    assert np.array_equal(oracle.decode(inputs.bits(q), "bf16"), q.double().numpy())
    q, k, v = inputs.make_qkv(1, 2, 5, 8, "f16", seed=3)
    assert np.array_equal(oracle.decode(inputs.bits(v), "f16"), v.double().numpy())


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------
def test_two_key_closed_form():
    # Two queries, two orthogonal keys, identity values, scale 1/2.
    q = np.array([[[[1.0, 0.0], [0.0, 2.0]]]])
    k = np.array([[[[1.0, 0.0], [0.0, 1.0]]]])
    v = np.array([[[[1.0, 0.0], [0.0, 1.0]]]])
    o, lse = oracle.attention_fwd(q, k, v, 0.5, False)
    e5, e1 = math.exp(0.5), math.exp(1.0)
    np.testing.assert_allclose(o[0, 0, 0], [e5 / (e5 + 1), 1 / (e5 + 1)], rtol=0, atol=1e-15)
    np.testing.assert_allclose(o[0, 0, 1], [1 / (1 + e1), e1 / (1 + e1)], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[0, 0], [math.log(e5 + 1), math.log(1 + e1)], rtol=1e-15)
    o, lse = oracle.attention_fwd(q, k, v, 0.5, True)
    np.testing.assert_allclose(o[0, 0, 0], [1.0, 0.0], atol=0)
    assert lse[0, 0, 0] == 0.5
    np.testing.assert_allclose(o[0, 0, 1], [1 / (1 + e1), e1 / (1 + e1)], atol=1e-15)


@pytest.mark.parametrize("N", [1, 7, 400])
@pytest.mark.parametrize("causal", [False, True])
def test_q_zero_gives_mean_of_v(N, causal):
    v = rand(2, 3, N, 16)
    q = np.zeros_like(v)
    k = rand(2, 3, N, 16)
    o, lse = oracle.attention_fwd(q, k, v, 0.3, causal)
    if causal:
        mean = np.cumsum(v, axis=2) / np.arange(1, N + 1)[None, None, :, None]
        expect_lse = np.log(np.arange(1, N + 1, dtype=np.float64))[None, None, :]
    else:
        mean = np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
        expect_lse = np.full((2, 3, N), math.log(N))
    np.testing.assert_allclose(o, mean, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, np.broadcast_to(expect_lse, lse.shape), rtol=1e-14, atol=1e-14)


def test_scale_zero_gives_mean_of_v():
    q, k, v = rand(1, 2, 9, 8), rand(1, 2, 9, 8), rand(1, 2, 9, 8)
    o, lse = oracle.attention_fwd(q, k, v, 0.0, False)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape), atol=1e-14)
    np.testing.assert_allclose(lse, math.log(9), rtol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_constant_v_returns_constant(causal):
    q, k = rand(2, 2, 33, 8, scale=3.0), rand(2, 2, 33, 8, scale=3.0)
    c = rand(8)
    v = np.broadcast_to(c, (2, 2, 33, 8)).copy()
    o, _ = oracle.attention_fwd(q, k, v, 0.35, causal)
    np.testing.assert_allclose(o, v, rtol=1e-14, atol=1e-14)


def test_dominant_score_selects_its_value_row():
    N, d = 17, 8
    q = rand(1, 1, N, d)
    k = rand(1, 1, N, d) * 0.01
    v = rand(1, 1, N, d)
    jstar = 11
    # make key jstar align with every query strongly: s_i,j* exceeds the rest by >= 40
    k[0, 0, jstar] = 0.0
    q[0, 0, :, 0] = 1.0
    k[0, 0, jstar, 0] = 60.0
    o, lse = oracle.attention_fwd(q, k, v, 1.0, False)
    s = q[0, 0] @ k[0, 0].T
    assert (s[:, jstar][:, None] - np.delete(s, jstar, axis=1)).min() >= 40
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0, jstar], (N, d)), atol=N * math.exp(-40) * 10)


def test_causal_row0_and_n1():
    q, k, v = rand(1, 2, 6, 8), rand(1, 2, 6, 8), rand(1, 2, 6, 8)
    o, lse = oracle.attention_fwd(q, k, v, 0.7, True)
    assert np.array_equal(o[:, :, 0], v[:, :, 0])
    np.testing.assert_allclose(lse[:, :, 0], 0.7 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]), rtol=1e-15)
    o1, lse1 = oracle.attention_fwd(q[:, :, :1], k[:, :, :1], v[:, :, :1], 0.7, False)
    assert np.array_equal(o1, v[:, :, :1])
    np.testing.assert_allclose(lse1, lse[:, :, :1], rtol=1e-15)


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------
def test_joint_permutation_of_keys_and_values():
    q, k, v = rand(2, 2, 40, 16), rand(2, 2, 40, 16), rand(2, 2, 40, 16)
    perm = rng.permutation(40)
    o1, l1 = oracle.attention_fwd(q, k, v, 0.25, False)
    o2, l2 = oracle.attention_fwd(q, k[:, :, perm], v[:, :, perm], 0.25, False)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_shift_of_all_keys(causal):
    q, k, v = rand(1, 3, 21, 8), rand(1, 3, 21, 8), rand(1, 3, 21, 8)
    c = rand(8)
    o1, l1 = oracle.attention_fwd(q, k, v, 0.4, causal)
    o2, l2 = oracle.attention_fwd(q, k + c, v, 0.4, causal)
    np.testing.assert_allclose(o1, o2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(l2 - l1, 0.4 * (q @ c), rtol=1e-11, atol=1e-12)


def test_linear_in_v():
    q, k = rand(1, 2, 19, 8), rand(1, 2, 19, 8)
    v1, v2 = rand(1, 2, 19, 8), rand(1, 2, 19, 8)
    o1, _ = oracle.attention_fwd(q, k, v1, 0.5, True)
    o2, _ = oracle.attention_fwd(q, k, v2, 0.5, True)
    o3, _ = oracle.attention_fwd(q, k, 2.0 * v1 - 3.0 * v2, 0.5, True)
    np.testing.assert_allclose(o3, 2.0 * o1 - 3.0 * o2, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_rows_sum_to_one(causal):
    q, k, v = rand(1, 2, 50, 16, scale=2), rand(1, 2, 50, 16, scale=2), rand(1, 2, 50, 16)
    _, lse = oracle.attention_fwd(q, k, v, 0.3, causal)
    s = 0.3 * np.einsum("bhid,bhjd->bhij", q, k)
    if causal:
        s = np.where(np.tril(np.ones((50, 50), bool)), s, -np.inf)
    tot = np.exp(s - lse[..., None]).sum(-1)
    np.testing.assert_allclose(tot, 1.0, rtol=0, atol=1e-14)


# ---------------------------------------------------------------------------
# library routine: torch's fp64 scaled-dot-product attention on the CPU
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("shape", [(1, 4, 400, 64), (2, 3, 65, 128), (1, 2, 1, 64), (1, 1, 130, 96)])
@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa_fp64(shape, causal):
    q, k, v = rand(*shape, scale=2.0), rand(*shape, scale=2.0), rand(*shape)
    scale = 0.9 / math.sqrt(shape[-1])
    o, lse = oracle.attention_fwd(q, k, v, scale, causal)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale).numpy()
    s = scale * (tq @ tk.transpose(-1, -2))
    if causal:
        n = shape[2]
        s = s.masked_fill(~torch.ones(n, n, dtype=torch.bool).tril(), float("-inf"))
    ref_lse = torch.logsumexp(s, dim=-1).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# independent derivation: blocked online softmax (running max m, running sum
# l, rescale of earlier partial results by exp(m_old - m_new)) must reach the
# three-pass result ("FlashAttention explainer" 4.3; "YOLO11 ...
# FlashAttention-2" 2.2). Written here from the algebra, independently.
# ---------------------------------------------------------------------------
def blocked_online(q, k, v, scale, causal, bc):
    N, d = q.shape
    o = np.zeros((N, d))
    lse = np.zeros(N)
    for i in range(N):
        m, l, acc = -np.inf, 0.0, np.zeros(d)
        last = i + 1 if causal else N
        for j0 in range(0, last, bc):
            j1 = min(last, j0 + bc)
            s = scale * (k[j0:j1] @ q[i])
            m_new = max(m, s.max())
            alpha = math.exp(m - m_new) if m > -np.inf else 0.0
            p = np.exp(s - m_new)
            l = alpha * l + p.sum()
            acc = alpha * acc + p @ v[j0:j1]
            m = m_new
        o[i] = acc / l
        lse[i] = m + math.log(l)
    return o, lse


@pytest.mark.parametrize("N", [1, 2, 7, 17, 65])
@pytest.mark.parametrize("causal", [False, True])
def test_blocked_online_softmax_equals_three_pass(N, causal):
    q, k, v = rand(N, 8, scale=3), rand(N, 8, scale=3), rand(N, 8)
    o_ref, lse_ref = oracle.attention_fwd(q[None, None], k[None, None], v[None, None], 0.5, causal)
    for bc in sorted({1, 3, 16, 64, N}):
        o, lse = blocked_online(q, k, v, 0.5, causal, bc)
        np.testing.assert_allclose(o, o_ref[0, 0], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(lse, lse_ref[0, 0], rtol=1e-13, atol=1e-13)


def test_q_block_tiling_with_full_row_softmax():
    # A Q-block loop with a full-row softmax per block ("YOLO11 ...
    # FlashAttention-2" 3.2 sketch): rows are independent, so it must agree.
    q, k, v = (torch.from_numpy(rand(1, 2, 150, 16)) for _ in range(3))
    out = torch.empty_like(q)
    for s0 in range(0, 150, 64):
        sc = (q[:, :, s0:s0 + 64] @ k.transpose(-2, -1)) / 16 ** 0.5
        out[:, :, s0:s0 + 64] = torch.softmax(sc, dim=-1) @ v
    o, _ = oracle.attention_fwd(q.numpy(), k.numpy(), v.numpy(), 0.25, False)
    np.testing.assert_allclose(o, out.numpy(), rtol=1e-12, atol=1e-12)


def test_rows_variant_matches_full():
    q, k, v = rand(2, 3, 70, 16), rand(2, 3, 70, 16), rand(2, 3, 70, 16)
    o, lse = oracle.attention_fwd(q, k, v, 0.3, True)
    rows = np.array([[0, 0, 0], [1, 2, 69], [0, 1, 33], [1, 2, 5], [1, 0, 64]])
    o_r, lse_r = oracle.attention_fwd_rows(q, k, v, 0.3, True, rows)
    for n, (b, h, i) in enumerate(rows):
        np.testing.assert_allclose(o_r[n], o[b, h, i], rtol=1e-15, atol=1e-15)
        np.testing.assert_allclose(lse_r[n], lse[b, h, i], rtol=1e-15)


# ---------------------------------------------------------------------------
# backward: finite differences and torch autograd (fp64, CPU)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_backward_finite_differences(causal):
    q, k, v, do = rand(1, 1, 5, 4), rand(1, 1, 5, 4), rand(1, 1, 5, 4), rand(1, 1, 5, 4)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.6, causal)

    def f(q_, k_, v_):
        return float((oracle.attention_fwd(q_, k_, v_, 0.6, causal)[0] * do).sum())

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            num[idx] = (f(*args_p) - f(*args_m)) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8, err_msg=name)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_torch_autograd(causal):
    shape = (2, 2, 37, 16)
    q, k, v, do = rand(*shape), rand(*shape), rand(*shape), rand(*shape)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.25, causal)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=0.25)
    out.backward(torch.from_numpy(do))
    for ours, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(ours, ref.numpy(), rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------------------
# the pages' printed counts pin the accounting helpers
# ---------------------------------------------------------------------------
def test_page_counts():
    with open(os.path.join(GOLDEN, "page_counts.json")) as f:
        g = json.load(f)
    er = g["element_ratio"]
    assert er["N"] * er["d"] == er["qkv_elems"]
    assert accounting.score_elems(er["N"]) == er["score_elems"]
    assert accounting.score_elems(er["N"]) // (er["N"] * er["d"]) == er["ratio"]
    b = g["blocks_n400"]
    assert accounting.num_tiles(b["n"], b["block"]) == b["blocks"]
    mp = g["map_20x20"]
    assert mp["h"] * mp["w"] == mp["N"] and accounting.score_elems(mp["N"]) == mp["score_elems"]


def test_accounting_flops_bytes():
    assert accounting.alg_flops(1, 1, 4, 2, False) == 4 * 16 * 2
    assert accounting.alg_flops(1, 1, 4, 2, True) == 4 * 10 * 2
    assert accounting.metric_flops(1, 32, 8192, 128) == 2 * accounting.alg_flops(1, 32, 8192, 128, True) - 4 * 32 * 8192 * 128
    assert accounting.alg_bytes(16, 8, 400, 64) == 26_419_200


# ---------------------------------------------------------------------------
# planted mistakes: each mutated copy of the oracle's row routine must fail
# at least one of the pins above (run here as plain checks).
# ---------------------------------------------------------------------------
def _mutant(kind):
    def rows_fwd(q_rows, row_idx, k, v, scale, causal):
        n = k.shape[0]
        sc = 1.0 if kind == "drop_scale" else scale
        s = sc * (q_rows @ (v if kind == "k_is_v" else k).T)
        if causal:
            ri = np.asarray(row_idx)[:, None]
            keep = np.arange(n)[None, :] < ri if kind == "causal_strict" else np.arange(n)[None, :] <= ri
            keep = keep | (np.arange(n)[None, :] == 0) if kind == "causal_strict" else keep
            s = np.where(keep, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        p = np.exp(m - s) if kind == "sign" else np.exp(s - m)
        p = np.where(np.isfinite(p), p, 0.0)
        l = p.sum(axis=1, keepdims=True)
        o = (p @ v) if kind == "no_norm" else (p @ v) / l
        lse = m[:, 0] + (np.log2(l[:, 0]) if kind == "lse_base2" else np.log(l[:, 0]))
        return o, lse
    return rows_fwd


def _pins_pass():
    checks = []
    r = np.random.default_rng(7)
    q, k, v = (r.standard_normal((1, 2, 23, 8)) for _ in range(3))
    for causal in (False, True):
        o, lse = oracle.attention_fwd(q, k, v, 0.45, causal)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=0.45).numpy()
        checks.append(np.allclose(o, ref, rtol=1e-12, atol=1e-12))
        oz, lz = oracle.attention_fwd(np.zeros_like(q), k, v, 0.45, causal)
        n = np.arange(1, 24) if causal else np.full(23, 23)
        checks.append(np.allclose(lz, np.log(n)[None, None], atol=1e-13))
        checks.append(np.allclose(o[:, :, 0], v[:, :, 0]) if causal else True)
    return all(checks)


@pytest.mark.parametrize("kind", ["drop_scale", "k_is_v", "causal_strict", "sign", "no_norm", "lse_base2"])
def test_planted_mistakes_are_caught(kind, monkeypatch):
    assert _pins_pass()
    monkeypatch.setattr(oracle, "_rows_fwd", _mutant(kind))
    assert not _pins_pass(), f"mutant {kind} slipped through the pins"
