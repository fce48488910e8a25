"""Pins for the backward oracle (``oracle.attention_bwd``).

Each pin takes ``grad(Q, K, V, dO, causal, scale) -> (dQ, dK, dV)`` and raises
AssertionError if the gradients break a fact that does not come from the
oracle's own formula:

* central differences of the forward oracle (itself pinned in ``pins.py``): the
  gradients are the derivatives of sum(O * dO), brute force on tiny inputs;
* torch's autograd through its own scaled-dot-product attention in fp64;
* closed forms and invariants of the function.

The forward function is the one of "Writing a FlashAttention kernel in Metal",
sections "Standard attention" and "Blockwise attention and causal masking".
"""

from __future__ import annotations

import numpy as np
import torch

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol, what):
    err = float(np.max(np.abs(np.asarray(a) - np.asarray(b))))
    assert err <= tol, f"{what}: max abs error {err:.3e} > {tol:.1e}"


def _loss(Q, K, V, dO, causal, scale):
    O, _ = oracle.attention(Q, K, V, causal, scale)
    return float(np.sum(O * dO))


def pin_central_differences(grad):
    """Every gradient entry equals the central difference of sum(O * dO) (forward
    oracle) on tiny inputs, causal and not, including N = 1 and d = 1."""
    h = 1e-6
    for causal in (False, True):
        for (N, d, seed) in ((1, 3, 1), (2, 1, 2), (3, 2, 3), (5, 4, 4)):
            r = _rng(seed)
            Q, K, V, dO = (r.standard_normal((1, 1, N, d)) for _ in range(4))
            scale = 0.7
            gQ, gK, gV = grad(Q, K, V, dO, causal, scale)
            for name, X, G in (("dQ", Q, gQ), ("dK", K, gK), ("dV", V, gV)):
                num = np.zeros_like(X)
                for idx in np.ndindex(X.shape):
                    Xp = X.copy(); Xp[idx] += h
                    Xm = X.copy(); Xm[idx] -= h
                    args = {"dQ": (Xp, K, V), "dK": (Q, Xp, V), "dV": (Q, K, Xp)}[name]
                    argm = {"dQ": (Xm, K, V), "dK": (Q, Xm, V), "dV": (Q, K, Xm)}[name]
                    num[idx] = (_loss(*args, dO, causal, scale) - _loss(*argm, dO, causal, scale)) / (2 * h)
                _close(G, num, 1e-7, f"{name} vs central differences N={N} d={d} causal={causal}")


def pin_torch_autograd(grad):
    """torch's autograd through its scaled-dot-product attention, fp64 on the CPU."""
    for causal in (False, True):
        r = _rng(11 + causal)
        Q, K, V, dO = (r.standard_normal((2, 3, 17, 8)) for _ in range(4))
        scale = 0.45
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (Q, K, V))
        out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
        out.backward(torch.tensor(dO))
        gQ, gK, gV = grad(Q, K, V, dO, causal, scale)
        _close(gQ, tq.grad.numpy(), 1e-12, f"dQ vs torch autograd causal={causal}")
        _close(gK, tk.grad.numpy(), 1e-12, f"dK vs torch autograd causal={causal}")
        _close(gV, tv.grad.numpy(), 1e-12, f"dV vs torch autograd causal={causal}")


def pin_sums_over_keys(grad):
    """The rows of P sum to 1 and adding one vector to every key leaves O unchanged,
    so sum_j dV[j] = sum_i dO[i] and sum_j dK[j] = 0 (causal or not)."""
    for causal in (False, True):
        r = _rng(21 + causal)
        Q, K, V, dO = (r.standard_normal((1, 2, 23, 5)) for _ in range(4))
        gQ, gK, gV = grad(Q, K, V, dO, causal, 0.6)
        _close(gV.sum(axis=2), dO.sum(axis=2), 1e-12, f"sum of dV rows causal={causal}")
        _close(gK.sum(axis=2), np.zeros_like(gK.sum(axis=2)), 1e-12, f"sum of dK rows causal={causal}")


def pin_single_key(grad):
    """N = 1: O = V, so dV = dO and dQ = dK = 0."""
    r = _rng(31)
    Q, K, V, dO = (r.standard_normal((2, 1, 1, 6)) for _ in range(4))
    gQ, gK, gV = grad(Q, K, V, dO, True, 0.5)
    _close(gV, dO, 0.0, "dV at N=1")
    _close(gQ, np.zeros_like(gQ), 0.0, "dQ at N=1")
    _close(gK, np.zeros_like(gK), 0.0, "dK at N=1")


def pin_uniform_weights(grad):
    """Q = 0, non-causal: every row of P is 1/N, so dV[j] = mean_i dO[i] for every key j;
    causal: P[i][j] = 1/(i+1) for j <= i, so dV[j] = sum_{i >= j} dO[i] / (i + 1)."""
    r = _rng(41)
    N, d = 9, 4
    K, V, dO = (r.standard_normal((1, 1, N, d)) for _ in range(3))
    Q = np.zeros_like(K)
    _, _, gV = grad(Q, K, V, dO, False, 0.8)
    _close(gV[0, 0], np.broadcast_to(dO[0, 0].mean(axis=0), (N, d)), 1e-14, "dV with uniform weights")
    _, _, gV = grad(Q, K, V, dO, True, 0.8)
    w = dO[0, 0] / np.arange(1, N + 1)[:, None]
    expect = np.cumsum(w[::-1], axis=0)[::-1]
    _close(gV[0, 0], expect, 1e-14, "dV with causal uniform weights")


def pin_linear_in_output_gradient(grad):
    """The gradients are linear in dO."""
    r = _rng(51)
    Q, K, V, dA, dB = (r.standard_normal((1, 1, 12, 3)) for _ in range(5))
    a = grad(Q, K, V, dA, True, 0.9)
    b = grad(Q, K, V, dB, True, 0.9)
    c = grad(Q, K, V, dA + 2.0 * dB, True, 0.9)
    for x, y, z, name in zip(a, b, c, ("dQ", "dK", "dV")):
        _close(z, x + 2.0 * y, 1e-12, f"{name} linear in dO")


def pin_key_permutation(grad):
    """Non-causal attention does not depend on the order of the key/value pairs: permuting
    them permutes the rows of dK and dV the same way and leaves dQ unchanged."""
    r = _rng(61)
    Q, K, V, dO = (r.standard_normal((1, 1, 10, 4)) for _ in range(4))
    perm = r.permutation(10)
    gQ, gK, gV = grad(Q, K, V, dO, False, 0.5)
    pQ, pK, pV = grad(Q, K[:, :, perm], V[:, :, perm], dO, False, 0.5)
    _close(pQ, gQ, 1e-12, "dQ under a key permutation")
    _close(pK, gK[:, :, perm], 1e-12, "dK under a key permutation")
    _close(pV, gV[:, :, perm], 1e-12, "dV under a key permutation")


ALL_PINS = [
    pin_central_differences,
    pin_torch_autograd,
    pin_sums_over_keys,
    pin_single_key,
    pin_uniform_weights,
    pin_linear_in_output_gradient,
    pin_key_permutation,
]
