"""GPU parity of the small-shape fp32 sweep (the benchmark configurations of "Writing a
FlashAttention kernel in Metal": one sequence, one head, N in {64, 256, 1024, 2048},
d in {32, 64}, causal and not) against the fp64 oracle, every row, at the fp32
tolerances O 1e-5 / L 1e-4."""

import numpy as np
import pytest
import torch

import oracle
from workloads import SMALL_SWEEP

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import tiled_online_softmax_amd

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return tiled_online_softmax_amd


@pytest.mark.parametrize("w", SMALL_SWEEP, ids=lambda w: w.name)
def test_small_sweep_config(fa, w):
    q, k, v = w.make()
    dev = torch.device("cuda:0")
    O, L = fa.forward(q.to(dev), k.to(dev), v.to(dev), causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    Oref, Lref = oracle.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), w.causal, w.scale)
    eo = float(np.abs(O.double().cpu().numpy() - Oref).max())
    el = float(np.abs(L.double().cpu().numpy() - Lref).max())
    print(f"[parity-sweep] {w.name} max|dO|={eo:.3e} max|dL|={el:.3e}", flush=True)
    assert eo <= 1e-5 and el <= 1e-4, (eo, el)
