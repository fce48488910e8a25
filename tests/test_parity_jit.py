"""GPU parity of the shape-specialized forward (fa_fwd_specialized: kernels compiled at
run time with the sizes as constants) against the fp64 oracle and against fa_fwd.

Tolerances as for fa_fwd (max abs error): O 1e-5 / L 1e-4 for fp32, O 2e-2 / L 1e-2 for
bf16. The two entry points run the same kernel source; constant sizes may reorder the
integer work but not the floating-point arithmetic, which is checked bitwise here.
"""

import time

import numpy as np
import pytest
import torch

import oracle
from workloads import WORKLOADS, default_scale, make_qkv, sample_rows

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 1e-4), "bf16": (2e-2, 1e-2)}
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def fa():
    import tiled_online_softmax_amd

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return tiled_online_softmax_amd


CASES = [(1, 2, 1000, 64, False, "bf16"), (2, 3, 777, 128, True, "bf16"), (1, 2, 130, 32, True, "bf16"),
         (1, 1, 100, 16, True, "bf16"), (8, 1, 1024, 64, False, "f32"), (1, 1, 100, 16, True, "f32"),
         (2, 2, 333, 128, True, "f32")]


@pytest.mark.parametrize("B,H,N,d,causal,dtype", CASES)
def test_specialized_matches_oracle_and_fa_fwd(fa, B, H, N, d, causal, dtype):
    q, k, v = make_qkv(B, H, N, d, dtype, seed=N + d)
    scale = default_scale(d)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    O, L = fa.forward_specialized(qd, kd, vd, causal=causal, scale=scale)
    O2, L2 = fa.forward(qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    Oref, Lref = oracle.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), causal, scale)
    eo = float(np.abs(O.double().cpu().numpy() - Oref).max())
    el = float(np.abs(L.double().cpu().numpy() - Lref).max())
    same = torch.equal(O, O2) and torch.equal(L, L2)
    print(f"[parity-jit] {dtype} B={B} H={H} N={N} d={d} causal={causal} max|dO|={eo:.3e} max|dL|={el:.3e} "
          f"bitwise-equal-to-fa_fwd={same}", flush=True)
    otol, ltol = TOL[dtype]
    assert eo <= otol and el <= ltol
    assert same


def test_specialized_full_size_sampled(fa):
    """The benchmarked causal bf16 B4 H16 N4096 d128 shape (each XCD takes its eight heads four at a
    time): bitwise equal to fa_fwd on every element, sampled rows against the oracle."""
    w = WORKLOADS["causal_bf16_b4h16n4096d128"]
    q, k, v = w.make()
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    O, L = fa.forward_specialized(qd, kd, vd, causal=True, scale=w.scale)
    O2, L2 = fa.forward(qd, kd, vd, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(O, O2) and torch.equal(L, L2), "specialized and generic kernels differ"
    rows = sample_rows(w.N, 12, seed=w.seed)
    Oref, Lref = oracle.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), True, w.scale,
                                  rows=rows)
    eo = float(np.abs(O.double().cpu().numpy()[:, :, rows] - Oref).max())
    el = float(np.abs(L.double().cpu().numpy()[:, :, rows] - Lref).max())
    print(f"[parity-jit] full size sampled max|dO|={eo:.3e} max|dL|={el:.3e}", flush=True)
    assert eo <= 2e-2 and el <= 1e-2


def test_specialized_cache_reuses_kernel(fa):
    """A second call with the same shape does not compile again."""
    q, k, v = (t.to(DEV) for t in make_qkv(1, 1, 300, 64, "bf16", seed=3))
    fa.forward_specialized(q, k, v)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(5):
        fa.forward_specialized(q, k, v)
    torch.cuda.synchronize()
    assert time.perf_counter() - t0 < 0.2


def test_specialized_on_side_stream(fa):
    """On a stream of its own (a non-null handle: the library loads the kernel on the stream's
    device), ordered after the inputs' copies: bitwise equal to fa_fwd."""
    q, k, v = (t.to(DEV) for t in make_qkv(2, 3, 777, 128, "bf16", seed=11))
    ref_o, ref_l = fa.forward(q, k, v, causal=True, scale=default_scale(128))
    side = torch.cuda.Stream(DEV)
    O = torch.full_like(q, float("nan"))
    L = torch.full((2, 3, 777), float("nan"), dtype=torch.float32, device=DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    fa.fa_fwd_specialized(q, k, v, O, L, 2, 3, 777, 128, True, default_scale(128), side)
    torch.cuda.synchronize()
    assert torch.equal(O, ref_o) and torch.equal(L, ref_l)
