"""GPU parity of the FlashAttention-1 loop-order ablation (fa_fwd_fa1_order)
against the fp64 oracle, and its agreement with the FA2 kernels."""
import numpy as np
import pytest
import torch

import oracle
import parity as P
import exact_attention_fa2_amd as fa
from exact_attention_fa2_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d,dtype", [(1, 64, "f16"), (65, 64, "bf16"), (400, 64, "f16"), (333, 128, "bf16"),
                                       (130, 96, "f16"), (200, 256, "bf16"), (1100, 64, "f16")])
def test_fa1_order_matches_oracle(N, d, dtype, causal):
    print(f"[fa_fwd_fa1_order] N{N} d{d} {dtype} causal={causal}", flush=True)
    q, k, v = inputs.make_qkv(2, 3, N, d, dtype, seed=N + d, sigma_qk=2.0)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    o1, l1 = fa.attention_fa1_order(qg, kg, vg, causal=causal)
    o2, l2 = fa.attention(qg, kg, vg, causal=causal)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_fwd(*(P.decode(x, dtype) for x in (q, k, v)), d ** -0.5, causal)
    P.gate_o(P.to64(o1), ro, dtype)
    P.gate_lse(P.to64(l1), rl)
    # same online-softmax arithmetic as the FA2 kernels: at most a rounding step apart
    assert np.abs(P.to64(o1) - P.to64(o2)).max() <= 2 * P.ATOL[dtype]
