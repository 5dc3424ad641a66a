"""HIP graph capture of the entry points: replays must reproduce the eager
results bit for bit, with eager work and synchronisations between replays,
and a process whose very first call happens under capture must work (the
launchers query the device only through calls that capture allows)."""
import os
import subprocess
import sys
import textwrap

import pytest
import torch

import exact_attention_fa2_amd as fa
from exact_attention_fa2_amd import inputs

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _check_replays(fn, outs, eager, replays=3):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.synchronize()
    for i in range(replays):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, e in zip(outs, eager):
            assert torch.equal(t, e), f"replay {i} differs from the eager result"
        fn()  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("N,d,dtype,causal", [(400, 64, "bf16", False), (6400, 64, "f16", False),
                                              (1000, 128, "bf16", True), (300, 64, "f16", True)])
def test_forward_graph_replay(N, d, dtype, causal):
    print(f"[graph fwd] B2 H4 N{N} d{d} {dtype} causal={causal}", flush=True)
    q, k, v = (t.cuda() for t in inputs.make_qkv(2, 4, N, d, dtype, 3))
    o = torch.empty_like(q)
    lse = torch.empty(2, 4, N, dtype=torch.float32, device="cuda")
    call = lambda: fa.fa_fwd(q, k, v, o, lse, 2, 4, N, d, d ** -0.5, causal)
    call()
    torch.cuda.synchronize()
    eager = (o.clone(), lse.clone())
    _check_replays(call, (o, lse), eager)


@pytest.mark.parametrize("N,d,dtype,causal", [(400, 64, "bf16", False), (700, 128, "bf16", True)])
def test_backward_graph_replay(N, d, dtype, causal):
    print(f"[graph bwd] B1 H4 N{N} d{d} {dtype} causal={causal}", flush=True)
    q, k, v = (t.cuda() for t in inputs.make_qkv(1, 4, N, d, dtype, 4))
    do = inputs.make_like(q.cpu(), 5).cuda()
    o, lse = fa.attention(q, k, v, causal=causal)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = torch.empty(fa.fa_bwd_workspace_bytes(1, 4, N, d), dtype=torch.uint8, device="cuda")
    call = lambda: fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, 1, 4, N, d, d ** -0.5, causal)
    call()
    torch.cuda.synchronize()
    eager = (dq.clone(), dk.clone(), dv.clone())
    _check_replays(call, (dq, dk, dv), eager)


def test_first_call_under_capture():
    # a fresh process whose first forward and backward calls are captured
    code = textwrap.dedent("""
        import torch, exact_attention_fa2_amd as fa
        from exact_attention_fa2_amd import inputs
        B, H, N, d = 16, 8, 400, 64
        q, k, v = (t.cuda() for t in inputs.make_qkv(B, H, N, d, "bf16", 6))
        do = inputs.make_like(q.cpu(), 7).cuda()
        o = torch.empty_like(q); lse = torch.empty(B, H, N, dtype=torch.float32, device="cuda")
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
        ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
        g = torch.cuda.CUDAGraph(); s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                fa.fa_fwd(q, k, v, o, lse, B, H, N, d, 0.125, False)
                fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, B, H, N, d, 0.125, False)
        torch.cuda.synchronize()
        g.replay(); torch.cuda.synchronize()
        got = [t.clone() for t in (o, lse, dq, dk, dv)]
        fa.fa_fwd(q, k, v, o, lse, B, H, N, d, 0.125, False)
        fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, B, H, N, d, 0.125, False)
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(got, (o, lse, dq, dk, dv)))
        print("first call under capture: OK", flush=True)
    """)
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=240)
    print(r.stdout[-2000:], r.stderr[-2000:], flush=True)
    assert r.returncode == 0 and "OK" in r.stdout
