"""Seeded random configurations through the forward entry points, against the fp64 oracle.

Each case draws, from a fixed numpy seed, an element type, head dimension, causal flag,
batch and head counts, query and key lengths (equal or not), a storage layout, a logit
width and a head repeat factor. Repeating the heads 200 times pushes a bf16 launch past
the grid size at which the kernel splits each tile's keys between two waves, so both
forms of the bf16 kernel meet every layout and length mix. The oracle runs on the
distinct heads; every repeat must equal its first copy bitwise.

Tolerances (max abs error): O 2e-2 / L 1e-2 for bf16; O 1e-5 / L 1e-4 for fp32 with
N(0, 1) inputs, multiplied by sigma^2 when Q and K are drawn with standard deviation
sigma (a score's fp32 rounding error grows with |q||k|, as in the wide-logit test of
test_parity.py).
"""

import os

import numpy as np
import pytest
import torch

import oracle
from workloads import default_scale, make_qkv_cross

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
TOL = {"f32": (1e-5, 1e-4), "bf16": (2e-2, 1e-2)}
LAYOUTS = ("contiguous", "bshd", "padded_rows")


def _case(i):
    r = np.random.RandomState(20261202 + i)
    dtype = ("bf16", "f32")[r.randint(2)]
    d = int((16, 32, 64, 128)[r.randint(4)])
    causal = bool(r.randint(2))
    B, H = int(r.randint(1, 3)), int(r.randint(1, 4))
    Nq = int(r.choice([1, 2, 31, 32, 33, 63, 64, 65, 97, 128, 129, 200, 257, 320]))
    Nk = Nq if r.randint(2) else int(r.choice([1, 17, 64, 65, 100, 191, 256, 300]))
    layout = LAYOUTS[r.randint(3)]
    sigma = float((1.0, 2.0, 4.0)[r.randint(3)]) if dtype == "bf16" else float((1.0, 2.0)[r.randint(2)])
    reps = 200 if r.randint(2) else 1
    return dict(dtype=dtype, d=d, causal=causal, B=B, H=H, Nq=Nq, Nk=Nk, layout=layout, sigma=sigma,
                reps=reps, seed=7000 + i)


# FA_RANDOM_CASES raises the count for a longer sweep (the same seeds first). The fixed
# extra cases are the four bf16 ones (sigma 4 logits, one dominant key with a large value)
# that a 10000-case sweep found above the O tolerance when the row sum added the fp32
# weights instead of the bf16 weights that enter the second product.
_REGRESSION = (301, 1074, 8125, 9886)
_N_RANDOM = int(os.environ.get("FA_RANDOM_CASES", "96"))
CASE_IDS = list(range(_N_RANDOM)) + [i for i in _REGRESSION if i >= _N_RANDOM]
CASES = [_case(i) for i in CASE_IDS]


def _store(t, layout):
    """Device copy of a contiguous [B, H, N, d] CPU tensor in the given storage layout."""
    if layout == "contiguous":
        return t.to(DEV)
    if layout == "bshd":
        return t.transpose(1, 2).contiguous().to(DEV).transpose(1, 2)
    w = torch.zeros(t.shape[:-1] + (t.shape[-1] + 16,), dtype=t.dtype)
    w[..., : t.shape[-1]] = t
    return w.to(DEV)[..., : t.shape[-1]]


@pytest.fixture(scope="module")
def fa():
    import tiled_online_softmax_amd

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return tiled_online_softmax_amd


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in CASE_IDS])
def test_random_configuration(fa, case):
    c = case
    label = " ".join(f"{k}={v}" for k, v in c.items())
    print(f"[random] {label}", flush=True)
    q, k, v = make_qkv_cross(c["B"], c["H"], c["Nq"], c["Nk"], c["d"], c["dtype"], c["seed"], c["sigma"])
    scale = default_scale(c["d"])
    Oref, Lref = oracle.attention_cross(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                        c["causal"], scale)
    H, reps = c["H"], c["reps"]
    qd, kd, vd = (_store(t.repeat(1, reps, 1, 1), c["layout"]) for t in (q, k, v))
    if c["layout"] == "contiguous" and c["Nq"] == c["Nk"]:
        O, L = fa.forward(qd, kd, vd, causal=c["causal"], scale=scale)
    else:
        O, L = fa.forward_strided(qd, kd, vd, causal=c["causal"], scale=scale)
    torch.cuda.synchronize()
    o = O[:, :H].double().cpu().numpy()
    lse = L[:, :H].double().cpu().numpy()
    assert np.isfinite(o).all() and np.isfinite(lse).all(), f"{label}: non-finite output"
    eo, el = float(np.abs(o - Oref).max()), float(np.abs(lse - Lref).max())
    otol, ltol = TOL[c["dtype"]]
    if c["dtype"] == "f32":
        otol, ltol = otol * c["sigma"] ** 2, ltol * c["sigma"] ** 2
    print(f"[random] max|dO|={eo:.3e} (tol {otol:.1e}) max|dL|={el:.3e} (tol {ltol:.1e})", flush=True)
    assert eo <= otol and el <= ltol, f"{label}: O error {eo}, L error {el}"
    for j in range(1, reps):
        assert torch.equal(O[:, j * H:(j + 1) * H], O[:, :H]) and torch.equal(L[:, j * H:(j + 1) * H], L[:, :H])
