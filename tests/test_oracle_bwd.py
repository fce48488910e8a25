"""The backward oracle against its pins (CPU only), and the pins against planted mistakes."""

import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import pins_bwd

# One plausible mistake per line of the gradient: each must fail some pin.
MUTANTS = {
    "dq_scale_dropped": ("gq[i * d + c] = scale * acc;", "gq[i * d + c] = acc;"),
    "dk_scale_dropped": ("gk[j * d + c] = scale * ak;", "gk[j * d + c] = ak;"),
    "jacobian_sign": ("g_row[j] = p_row[j] * (g_row[j] - pdp);", "g_row[j] = p_row[j] * (g_row[j] + pdp);"),
    "jacobian_row_term_dropped": ("g_row[j] = p_row[j] * (g_row[j] - pdp);", "g_row[j] = p_row[j] * g_row[j];"),
    "dv_from_ds": ("av += P[i * N + j] * go[i * d + c];", "av += G[i * N + j] * go[i * d + c];"),
    "dk_transposed": ("ak += G[i * N + j] * q[i * d + c];", "ak += G[j * N + i] * q[i * d + c];"),
    "dp_uses_k": ("dot += go[i * d + c] * v[j * d + c];", "dot += go[i * d + c] * k[j * d + c];"),
    "dq_uses_q": ("acc += g_row[j] * k[j * d + c];", "acc += g_row[j] * q[j * d + c];"),
    "causal_wrong_side": ("if (causal && j > i) {", "if (causal && j < i) {"),
    "softmax_unnormalised": ("p_row[j] = exp(p_row[j] - m) / denom;", "p_row[j] = exp(p_row[j] - m);"),
}


def _grad(Q, K, V, dO, causal, scale):
    return oracle.attention_bwd(Q, K, V, dO, causal, scale)


@pytest.mark.parametrize("pin", pins_bwd.ALL_PINS, ids=lambda p: p.__name__)
def test_backward_oracle_pin(pin):
    pin(_grad)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_backward_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    here = os.path.dirname(oracle.__file__)
    src = open(os.path.join(here, "attention_bwd.c")).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mutant_c = tmp_path / f"{name}.c"
    mutant_c.write_text(src.replace(old, new))
    so = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", str(so),
                    os.path.join(here, "attention.c"), str(mutant_c), "-lm"], check=True)
    lib = oracle.load_library(str(so))

    def grad(Q, K, V, dO, causal, scale):
        return oracle.attention_bwd(Q, K, V, dO, causal, scale, lib=lib)

    caught = []
    for pin in pins_bwd.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(grad)
        except (AssertionError, RuntimeError):
            caught.append(pin.__name__)
    assert caught, f"planted mistake {name!r} passed every pin"


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 5, 17])
def test_stored_statistics_gradient_identity(N, causal):
    """The GPU tests' reference for a backward that reads a stored O and L: its closed form
    (oracle calls with rescaled upstream gradients) equals the backward's formulas
    evaluated directly on a perturbed O and L -- P = exp(S - L'), D = sum_c dO O',
    dS = P (dP - D), dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO -- in fp64."""
    import torch

    from bwd_reference import stored_statistics_gradient

    rng = np.random.RandomState(40 + N + 100 * causal)
    B, H, d, scale = 1, 2, 6, 0.7
    q, k, v, do = (rng.standard_normal((B, H, N, d)) * s for s in (1.5, 1.5, 1.0, 1.0))
    O, L = oracle.attention(q, k, v, causal, scale)
    O2 = O + 1e-2 * rng.standard_normal(O.shape)
    L2 = L + 1e-2 * rng.standard_normal(L.shape)
    ref, stored = stored_statistics_gradient(*(torch.from_numpy(x) for x in (q, k, v, do)),
                                             torch.from_numpy(O2), torch.from_numpy(L2), causal, scale)
    for b in range(B):
        for h in range(H):
            S = scale * q[b, h] @ k[b, h].T
            if causal:
                S = np.where(np.tril(np.ones((N, N), dtype=bool)), S, -np.inf)
            P = np.exp(S - L2[b, h][:, None])
            D = np.sum(do[b, h] * O2[b, h], axis=-1)
            dS = P * (do[b, h] @ v[b, h].T - D[:, None])
            direct = (scale * dS @ k[b, h], scale * dS.T @ q[b, h], P.T @ do[b, h])
            for name, x, y, r in zip(("dQ", "dK", "dV"), stored, direct, ref):
                assert np.allclose(x[b, h], y, rtol=0, atol=1e-12), name
                if N > 1:  # the perturbation is visible in every gradient
                    assert np.abs(x[b, h] - r[b, h]).max() > 1e-6, name
