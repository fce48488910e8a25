"""HIP graph capture of the entry points (needs an MI355X).

The forward (one kernel) and the backward (three kernels) enqueue only kernel launches
on the caller's stream: no allocation, no memset, no host synchronisation. So both can
be captured into a HIP graph (torch.cuda.CUDAGraph) and replayed. Each test replays the
graph several times, writes new inputs into the captured buffers with eager torch work
between the replays, and checks every replay bitwise against an eager call on the same
inputs, and the first one against the fp64 oracle.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import default_scale, make_qkv

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
TOL = {"f32": (1e-5, 1e-4), "bf16": (2e-2, 1e-2)}


@pytest.fixture(scope="module")
def fa():
    import tiled_online_softmax_amd

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return tiled_online_softmax_amd


@pytest.mark.parametrize("dtype,d,causal", [("bf16", 128, True), ("bf16", 64, False), ("f32", 64, True),
                                            ("bf16", 128, False)])
def test_forward_graph_replays(fa, dtype, d, causal):
    B, H, N = 2, 4, 300
    scale = default_scale(d)
    q, k, v = (t.to(DEV) for t in make_qkv(B, H, N, d, dtype, seed=4000))
    O = torch.empty_like(q)
    L = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the capture
        fa.fa_fwd(q, k, v, O, L, B, H, N, d, causal, scale)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.fa_fwd(q, k, v, O, L, B, H, N, d, causal, scale)
    for r in range(3):
        qc, kc, vc = make_qkv(B, H, N, d, dtype, seed=4001 + r)
        q.copy_(qc)
        k.copy_(kc)
        v.copy_(vc)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        Oe, Le = fa.forward(q, k, v, causal=causal, scale=scale)
        torch.cuda.synchronize()
        assert torch.equal(O, Oe) and torch.equal(L, Le), f"replay {r} differs from the eager call"
        if r == 0:
            Oref, Lref = oracle.attention(qc.double().numpy(), kc.double().numpy(), vc.double().numpy(),
                                          causal, scale)
            eo = float(np.abs(O.double().cpu().numpy() - Oref).max())
            el = float(np.abs(L.double().cpu().numpy() - Lref).max())
            otol, ltol = TOL[dtype]
            print(f"[graph] {dtype} d={d} causal={causal} max|dO|={eo:.3e} max|dL|={el:.3e}", flush=True)
            assert eo <= otol and el <= ltol


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_forward_backward_graph_replays(fa, dtype):
    """One graph holding the forward and the backward (four kernels) over static buffers."""
    B, H, N, d, causal = 1, 3, 257, 64, True
    scale = default_scale(d)
    q, k, v = (t.to(DEV) for t in make_qkv(B, H, N, d, dtype, seed=4100))
    do = torch.zeros_like(q)
    O = torch.empty_like(q)
    L = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    work = torch.empty(2 * B * H * N, dtype=torch.float32, device=DEV)

    def body():
        fa.fa_fwd(q, k, v, O, L, B, H, N, d, causal, scale)
        fa.fa_bwd(q, k, v, O, L, do, dq, dk, dv, work, B, H, N, d, causal, scale)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        body()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    for r in range(3):
        qc, kc, vc = make_qkv(B, H, N, d, dtype, seed=4101 + r)
        gen = torch.Generator().manual_seed(4200 + r)
        q.copy_(qc)
        k.copy_(kc)
        v.copy_(vc)
        do.copy_(torch.randn((B, H, N, d), generator=gen).to(q.dtype))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        Oe, Le = fa.forward(q, k, v, causal=causal, scale=scale)
        dqe, dke, dve = fa.backward(q, k, v, Oe, Le, do, causal=causal, scale=scale)
        torch.cuda.synchronize()
        assert torch.equal(O, Oe) and torch.equal(L, Le), f"replay {r}: forward differs from eager"
        for name, a, b in (("dQ", dq, dqe), ("dK", dk, dke), ("dV", dv, dve)):
            assert torch.equal(a, b), f"replay {r}: {name} differs from eager"
