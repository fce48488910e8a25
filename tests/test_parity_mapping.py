"""Random shapes for the workgroup mapping: head counts that split evenly over the eight XCDs,
with K/V large enough that each XCD takes its heads in several groups (needs an MI355X).

Every tile must be written exactly once whatever the head count and group size: O and L
start as NaN and must come back finite, and sampled rows of every head are compared with
the fp64 oracle (standard attention, "Writing a FlashAttention kernel in Metal", section
*Standard attention*; L as in "FlashAttention-2 from PyTorch to Triton", section *What We
Are Building*). FA_MAPPING_CASES raises the count (the same seeds first).
"""

import os

import numpy as np
import pytest
import torch

import oracle
from workloads import default_scale, make_qkv

pytestmark = pytest.mark.gpu

TOL = (2e-2, 1e-2)  # bf16: O, L
_N_CASES = int(os.environ.get("FA_MAPPING_CASES", "12"))


def _case(i):
    r = np.random.RandomState(9000 + i)
    BH = 8 * int(r.choice([1, 2, 3, 5, 6, 7, 9, 12]))
    B = int(r.choice([b for b in (1, 2, 3, 4) if BH % b == 0]))
    d = int(r.choice([64, 128]))
    N = int(r.randint(1536, 4608))
    causal = bool(r.randint(2))
    return dict(B=B, H=BH // B, N=N, d=d, causal=causal, seed=9100 + i)


CASES = [_case(i) for i in range(_N_CASES)]


@pytest.fixture(scope="module")
def fa():
    import tiled_online_softmax_amd

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return tiled_online_softmax_amd


@pytest.mark.parametrize("case", CASES, ids=[f"m{i}" for i in range(_N_CASES)])
def test_mapping_random_shape(fa, case):
    B, H, N, d, causal = case["B"], case["H"], case["N"], case["d"], case["causal"]
    label = f"B{B} H{H} N{N} d{d} causal={causal}"
    print(f"[mapping] {label}", flush=True)
    q, k, v = make_qkv(B, H, N, d, "bf16", seed=case["seed"])
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    O = torch.full_like(qd, float("nan"))
    L = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=dev)
    scale = default_scale(d)
    fa.fa_fwd(qd, kd, vd, O, L, B, H, N, d, causal, scale)
    torch.cuda.synchronize()
    assert torch.isfinite(O).all() and torch.isfinite(L).all(), f"{label}: rows no workgroup wrote"
    rows = np.unique(np.concatenate([np.linspace(0, N - 1, 12).astype(int), [127, 128, 255, 256]]))
    Oref, Lref = oracle.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                  causal, scale, rows=rows)
    o = O.double().cpu().numpy()[:, :, rows]
    lse = L.double().cpu().numpy()[:, :, rows]
    eo = float(np.max(np.abs(o - Oref)))
    el = float(np.max(np.abs(lse - Lref)))
    print(f"[mapping] {label} max|dO|={eo:.3e} max|dL|={el:.3e}", flush=True)
    assert eo <= TOL[0] and el <= TOL[1], f"{label}: O error {eo}, L error {el}"
