"""fa_bwd_noalloc (the backward for callers that cannot allocate: its row
terms live in a static device array of the library) against fa_bwd with a
caller-owned workspace, through the C ABI. Two calls in a row, the second on
a smaller problem, so the second runs on the array the first left behind."""
import numpy as np
import pytest
import torch

import oracle
import parity as P
import exact_attention_fa2_amd as fa
from exact_attention_fa2_amd import inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _case(B, H, N, d, dtype, causal, seed):
    print(f"[fa_bwd_noalloc] B{B} H{H} N{N} d{d} {dtype} causal={causal} seed={seed}", flush=True)
    q, k, v = inputs.make_qkv(B, H, N, d, dtype, seed, 2.0)
    do = inputs.make_like(q, seed + 500)
    qg, kg, vg, dog = (t.to(DEV) for t in (q, k, v, do))
    sc = d ** -0.5
    o, lse = fa.attention(qg, kg, vg, causal=causal, scale=sc)
    ref = fa.attention_backward(qg, kg, vg, o, lse, dog, causal=causal, scale=sc)
    got = [torch.empty_like(qg) for _ in range(3)]
    fa.fa_bwd_noalloc(qg, kg, vg, o, dog, lse, *got, B, H, N, d, sc, causal)
    torch.cuda.synchronize()
    return q, k, v, do, sc, ref, got


@pytest.mark.parametrize("first,second", [
    ((2, 8, 1000, 64, "bf16", True, 1), (1, 3, 300, 64, "bf16", True, 2)),
    ((1, 4, 2048, 128, "f16", False, 3), (1, 2, 130, 128, "f16", True, 4)),
    ((2, 4, 700, 96, "bf16", False, 5), (1, 1, 65, 96, "bf16", False, 6)),
])
def test_noalloc_matches_workspace_backward(first, second):
    for case in (first, second):
        B, H, N, d, dtype, causal, seed = case
        q, k, v, do, sc, ref, got = _case(*case)
        for name, r, g in zip(("dq", "dk", "dv"), ref, got):
            # the same kernels on the same inputs: bit-identical
            assert torch.equal(r, g), (name, float((r.float() - g.float()).abs().max()))
        # and within the backward's tolerance of the oracle on one head
        qd, kd, vd, dd = (P.decode(x[:1, :1], dtype) for x in (q, k, v, do))
        refs = oracle.attention_bwd(qd, kd, vd, dd, sc, causal)
        u = 2.0 ** -11 if dtype == "f16" else 2.0 ** -8
        for name, g, r in zip(("dq", "dk", "dv"), got, refs):
            err = np.abs(P.to64(g[:1, :1]) - r).max()
            assert err <= 8 * u * np.abs(r).max() + 0.5 * float(P.ulp(np.abs(r).max(), dtype)), (name, err)
