"""Pins for the cross-attention oracle (``oracle.attention_cross``).

Each pin takes ``attn(Q, K, V, causal, scale) -> (O, L)`` with Q [B, H, Nq, d]
and K, V [B, H, Nk, d], and raises AssertionError if the result breaks a fact
that does not come from the oracle's own formula:

* the square oracle (``oracle.attention``, pinned in ``pins.py``) when Nq = Nk;
* torch's scaled-dot-product attention in fp64 with an explicit boolean mask that
  keeps key j for query i when j <= i, the alignment of the kernel in
  "FlashAttention-2 from PyTorch to Triton", section "The Triton Kernel";
* closed forms: zero queries give uniform weights over the admitted keys;
* the causal structure: row i sees exactly the keys 0..min(i, Nk - 1).
"""

from __future__ import annotations

import math

import numpy as np
import torch

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol, what):
    err = float(np.max(np.abs(np.asarray(a) - np.asarray(b))))
    assert err <= tol, f"{what}: max abs error {err:.3e} > {tol:.1e}"


SHAPES = [(1, 1, 1, 1, 3), (1, 2, 5, 9, 4), (2, 1, 9, 5, 4), (1, 1, 17, 3, 8), (1, 1, 3, 17, 8)]


def pin_square_case(attn):
    """Nq = Nk reproduces the square oracle, causal and not."""
    for causal in (False, True):
        for (B, H, N, d, seed) in ((1, 1, 1, 2, 1), (1, 2, 7, 4, 2), (2, 1, 13, 3, 3)):
            r = _rng(seed)
            Q, K, V = (r.standard_normal((B, H, N, d)) for _ in range(3))
            O, L = attn(Q, K, V, causal, 0.6)
            O2, L2 = oracle.attention(Q, K, V, causal, 0.6)
            _close(O, O2, 1e-13, f"O square N={N} causal={causal}")
            _close(L, L2, 1e-13, f"L square N={N} causal={causal}")


def pin_torch_sdpa(attn):
    """torch's scaled-dot-product attention (fp64, CPU) with the top-left mask, and
    torch.logsumexp of the masked scores."""
    for causal in (False, True):
        for (B, H, Nq, Nk, d) in SHAPES:
            r = _rng(Nq * 31 + Nk)
            Q, K, V = (r.standard_normal(s) for s in ((B, H, Nq, d), (B, H, Nk, d), (B, H, Nk, d)))
            scale = 1.0 / math.sqrt(d)
            O, L = attn(Q, K, V, causal, scale)
            q, k, v = (torch.from_numpy(x) for x in (Q, K, V))
            keep = torch.ones(Nq, Nk, dtype=torch.bool)
            if causal:
                keep = torch.arange(Nk)[None, :] <= torch.arange(Nq)[:, None]
            Ot = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=keep, scale=scale)
            S = (q @ k.transpose(-1, -2)) * scale
            Lt = torch.logsumexp(S.masked_fill(~keep, float("-inf")), dim=-1)
            _close(O, Ot.numpy(), 1e-12, f"O vs SDPA {Nq}x{Nk} causal={causal}")
            _close(L, Lt.numpy(), 1e-12, f"L vs logsumexp {Nq}x{Nk} causal={causal}")


def pin_zero_queries(attn):
    """Q = 0: every admitted key has the same score, so O[i] is the mean of the
    admitted value rows and L[i] = log(number admitted)."""
    for causal in (False, True):
        for (Nq, Nk) in ((4, 9), (9, 4), (6, 6)):
            V = _rng(Nq + 5 * Nk).standard_normal((1, 1, Nk, 3))
            K = _rng(7).standard_normal((1, 1, Nk, 3))
            O, L = attn(np.zeros((1, 1, Nq, 3)), K, V, causal, 1.3)
            for i in range(Nq):
                n = min(i + 1, Nk) if causal else Nk
                _close(O[0, 0, i], V[0, 0, :n].mean(axis=0), 1e-13, f"O row {i} {Nq}x{Nk}")
                _close(L[0, 0, i], math.log(n), 1e-13, f"L row {i} {Nq}x{Nk}")


def pin_causal_prefix(attn):
    """Causal row i equals the non-causal result over the keys 0..min(i, Nk - 1)
    alone; rows at or past Nk see every key."""
    for (Nq, Nk) in ((7, 4), (4, 7)):
        r = _rng(Nq * 3 + Nk)
        Q, K, V = (r.standard_normal(s) for s in ((1, 1, Nq, 5), (1, 1, Nk, 5), (1, 1, Nk, 5)))
        O, L = attn(Q, K, V, True, 0.8)
        for i in range(Nq):
            n = min(i + 1, Nk)
            Oi, Li = attn(Q[:, :, i:i + 1], K[:, :, :n], V[:, :, :n], False, 0.8)
            _close(O[0, 0, i], Oi[0, 0, 0], 1e-13, f"O row {i} {Nq}x{Nk}")
            _close(L[0, 0, i], Li[0, 0, 0], 1e-13, f"L row {i} {Nq}x{Nk}")


def pin_single_key(attn):
    """Nk = 1: every weight is 1, so O[i] = V[0] and L[i] = scale q_i . k_0."""
    r = _rng(11)
    Q, K, V = r.standard_normal((1, 1, 6, 4)), r.standard_normal((1, 1, 1, 4)), r.standard_normal((1, 1, 1, 4))
    for causal in (False, True):
        O, L = attn(Q, K, V, causal, 0.9)
        _close(O[0, 0], np.repeat(V[0, 0], 6, axis=0), 1e-14, f"O single key causal={causal}")
        _close(L[0, 0], 0.9 * Q[0, 0] @ K[0, 0, 0], 1e-14, f"L single key causal={causal}")


ALL_PINS = [pin_square_case, pin_torch_sdpa, pin_zero_queries, pin_causal_prefix, pin_single_key]
