"""Pins for the attention oracle: checks against facts fixed by the pages and by
mathematics, not by the oracle's own formula.

Each pin takes ``attn(Q, K, V, causal, scale, rows=None) -> (O, L)`` and raises
AssertionError (or the oracle's RuntimeError) when the implementation is wrong.
``tests/test_oracle.py`` runs them on the oracle, and on copies of the oracle
with planted mistakes to show that each such mistake fails at least one pin.
"""

from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs error {err:.3e} > {tol:.1e}"


def _rng(seed):
    return np.random.default_rng(seed)


def load_two_block_golden():
    """Parse tests/golden/two_block_example.txt (values stated by hand from the page)."""
    rows = []
    exp_scores = None
    l1 = l2 = None
    with open(os.path.join(GOLDEN, "two_block_example.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            if parts[0] == "exp_scores":
                exp_scores = [int(x) for x in parts[1:]]
            elif parts[0] == "l1":
                l1 = int(parts[1])
            elif parts[0] == "l2":
                l2 = int(parts[1])
            elif parts[0] == "row":
                kind, i = parts[1], int(parts[2])
                p = [float(Fraction(x)) for x in parts[3:7]]
                assert parts[7].startswith("L=ln(") and parts[7].endswith(")")
                lval = math.log(float(Fraction(parts[7][5:-1])))
                rows.append((kind == "causal", i, p, lval))
    return exp_scores, l1, l2, rows


def pin_two_block_golden(attn):
    """The page's two-block example, instantiated with e^x = 1, 2, 3, 4."""
    exp_scores, l1, l2, rows = load_two_block_golden()
    # The stated block sums follow from the stated exponentials.
    assert l1 == exp_scores[0] + exp_scores[1] and l2 == l1 + exp_scores[2] + exp_scores[3]
    n = 4
    Q = np.zeros((n, n))
    Q[:, 0] = 1.0
    K = np.zeros((n, n))
    K[:, 0] = np.log(np.array(exp_scores, dtype=np.float64))
    V = np.eye(n)
    for causal in (False, True):
        O, L = attn(Q, K, V, causal, 1.0)
        for (c, i, p, lval) in rows:
            if c != causal:
                continue
            _close(O[i], p, 1e-15, f"two-block P row {i} causal={causal}")
            _close(L[i], lval, 1e-15, f"two-block L row {i} causal={causal}")


def pin_uniform_when_queries_zero(attn):
    """Q = 0 makes every score 0: P is uniform over the admissible keys."""
    r = _rng(11)
    n, d = 37, 8
    Q = np.zeros((n, d))
    K = r.normal(size=(n, d))
    V = r.normal(size=(n, d))
    O, L = attn(Q, K, V, False, 0.7)
    _close(O, np.broadcast_to(V.mean(axis=0), (n, d)), 1e-13, "uniform O (non-causal)")
    _close(L, np.full(n, math.log(n)), 1e-13, "uniform L (non-causal)")
    O, L = attn(Q, K, V, True, 0.7)
    prefix_mean = np.cumsum(V, axis=0) / np.arange(1, n + 1)[:, None]
    _close(O, prefix_mean, 1e-13, "uniform O (causal)")
    _close(L, np.log(np.arange(1, n + 1)), 1e-13, "uniform L (causal)")


def pin_single_key(attn):
    """N = 1: the only weight is 1, O = V and L is the one scaled score."""
    r = _rng(12)
    d = 5
    Q = r.normal(size=(1, d))
    K = r.normal(size=(1, d))
    V = r.normal(size=(1, d))
    for causal in (False, True):
        O, L = attn(Q, K, V, causal, 0.3)
        _close(O, V, 1e-15, "N=1 O")
        s = 0.3 * math.fsum(float(Q[0, c] * K[0, c]) for c in range(d))
        _close(L, [s], 1e-14, "N=1 L")


def pin_two_keys_logistic(attn):
    """N = 2: softmax of two scores is the logistic function of their difference."""
    r = _rng(13)
    d, scale = 3, 0.9
    Q = r.normal(size=(2, d))
    K = r.normal(size=(2, d))
    V = r.normal(size=(2, d))
    S = [[scale * math.fsum(float(Q[i, c] * K[j, c]) for c in range(d)) for j in range(2)]
         for i in range(2)]
    O, L = attn(Q, K, V, False, scale)
    for i in range(2):
        p0 = 1.0 / (1.0 + math.exp(S[i][1] - S[i][0]))
        _close(O[i], p0 * V[0] + (1.0 - p0) * V[1], 1e-14, f"logistic O row {i}")
        _close(L[i], np.logaddexp(S[i][0], S[i][1]), 1e-14, f"logistic L row {i}")
    O, L = attn(Q, K, V, True, scale)
    _close(O[0], V[0], 1e-15, "causal logistic row 0")
    _close(L[0], S[0][0], 1e-14, "causal logistic L row 0")
    p0 = 1.0 / (1.0 + math.exp(S[1][1] - S[1][0]))
    _close(O[1], p0 * V[0] + (1.0 - p0) * V[1], 1e-14, "causal logistic row 1")


def pin_dominant_key(attn):
    """One key with a score 800 above all others takes the whole weight.

    exp(800) overflows fp64, so this also pins the shift by the row maximum that
    the first page's "Online softmax" section applies for numerical stability.
    """
    r = _rng(14)
    n, d = 16, 16
    Q = np.zeros((n, d))
    Q[:, 0] = 1.0
    K = np.zeros((n, d))
    K[5, 0] = 800.0
    V = r.normal(size=(n, d))
    for causal in (False, True):
        O, L = attn(Q, K, V, causal, 1.0)
        # non-causal: the other 15 weights are each e^-800, i.e. 0 in fp64
        rows = slice(5, n) if causal else slice(0, n)
        _close(O[rows], np.broadcast_to(V[5], (n, d))[rows], 1e-15, "dominant O")
        _close(L[rows], np.full(n, 800.0)[rows], 1e-12, "dominant L")
    # causal rows before key 5 never see it: uniform over their own prefix
    _close(O[:5], np.cumsum(V[:5], axis=0) / np.arange(1, 6)[:, None], 1e-14, "pre-dominant rows")


def pin_probabilities(attn):
    """With V = I (N = d) the output rows are the probability rows P.

    Rows of P sum to one ("Standard attention"); P = exp(S - L) with S the scaled
    scores ("What We Are Building" on the Triton page); causal P is zero above the
    diagonal ("Blockwise attention and causal masking").
    """
    r = _rng(15)
    n, scale = 12, 0.45
    Q = r.normal(size=(n, n))
    K = r.normal(size=(n, n))
    S = (Q @ K.T) * scale
    for causal in (False, True):
        P, L = attn(Q, K, np.eye(n), causal, scale)
        assert np.all(P >= 0.0), "negative probability"
        _close(P.sum(axis=1), np.ones(n), 1e-14, f"row sums causal={causal}")
        allowed = np.tril(np.ones((n, n), dtype=bool)) if causal else np.ones((n, n), dtype=bool)
        assert np.all(P[~allowed] == 0.0), "weight on a masked key"
        expect = np.where(allowed, np.exp(np.where(allowed, S, 0.0) - L[:, None]), 0.0)
        _close(P, expect, 1e-14, f"P = exp(S - L) causal={causal}")


def pin_value_linearity(attn):
    """O is linear in V, and V = 1 gives O = 1 (rows of P sum to one)."""
    r = _rng(16)
    n, d = 23, 6
    Q, K = r.normal(size=(n, d)), r.normal(size=(n, d))
    V1, V2 = r.normal(size=(n, d)), r.normal(size=(n, d))
    for causal in (False, True):
        O1, _ = attn(Q, K, V1, causal, 0.5)
        O2, _ = attn(Q, K, V2, causal, 0.5)
        O3, _ = attn(Q, K, 2.0 * V1 - 3.0 * V2, causal, 0.5)
        _close(O3, 2.0 * O1 - 3.0 * O2, 1e-13, "linearity in V")
        O4, _ = attn(Q, K, np.ones((n, d)), causal, 0.5)
        _close(O4, np.ones((n, d)), 1e-14, "constant V")


def pin_key_shift(attn):
    """Adding one vector u to every key shifts row i's scores by scale*q_i.u:
    P (hence O) is unchanged and L moves by exactly that amount."""
    r = _rng(17)
    n, d, scale = 29, 7, 0.6
    Q, K, V = r.normal(size=(n, d)), r.normal(size=(n, d)), r.normal(size=(n, d))
    u = r.normal(size=d)
    for causal in (False, True):
        O, L = attn(Q, K, V, causal, scale)
        O2, L2 = attn(Q, K + u, V, causal, scale)
        _close(O2, O, 1e-13, "key shift O")
        _close(L2, L + scale * (Q @ u), 1e-13, "key shift L")


def pin_permutations(attn):
    """Non-causal attention is invariant to reordering key/value pairs and
    equivariant to reordering queries."""
    r = _rng(18)
    n, d = 31, 5
    Q, K, V = r.normal(size=(n, d)), r.normal(size=(n, d)), r.normal(size=(n, d))
    O, L = attn(Q, K, V, False, 0.8)
    pk = r.permutation(n)
    O2, L2 = attn(Q, K[pk], V[pk], False, 0.8)
    _close(O2, O, 1e-13, "key permutation O")
    _close(L2, L, 1e-13, "key permutation L")
    pq = r.permutation(n)
    O3, L3 = attn(Q[pq], K, V, False, 0.8)
    _close(O3, O[pq], 1e-15, "query permutation O")
    _close(L3, L[pq], 1e-15, "query permutation L")


def pin_causal_prefix(attn):
    """Causal row i equals non-causal attention of query i over keys 0..i."""
    r = _rng(19)
    n, d = 20, 4
    Q, K, V = r.normal(size=(n, d)), r.normal(size=(n, d)), r.normal(size=(n, d))
    O, L = attn(Q, K, V, True, 0.5)
    for i in (0, 1, 7, n - 1):
        # queries 0..i against keys 0..i; only the last row is compared
        Oi, Li = attn(Q[: i + 1], K[: i + 1], V[: i + 1], False, 0.5)
        _close(O[i], Oi[i], 1e-14, f"causal prefix row {i}")
        _close(L[i], Li[i], 1e-14, f"causal prefix L row {i}")


def pin_torch_sdpa(attn):
    """torch's scaled_dot_product_attention in fp64 on the CPU (the SDPA baseline the
    first page benchmarks against), and torch.logsumexp of the masked scores."""
    g = torch.Generator().manual_seed(20)
    B, H, n, d = 2, 3, 50, 16
    scale = 1.0 / math.sqrt(d)
    Q = torch.randn(B, H, n, d, generator=g, dtype=torch.float64)
    K = torch.randn(B, H, n, d, generator=g, dtype=torch.float64)
    V = torch.randn(B, H, n, d, generator=g, dtype=torch.float64)
    for causal in (False, True):
        O, L = attn(Q.numpy(), K.numpy(), V.numpy(), causal, scale)
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=causal, scale=scale)
        _close(O, ref.numpy(), 1e-13, f"SDPA O causal={causal}")
        S = torch.matmul(Q, K.transpose(-1, -2).contiguous()) * scale
        if causal:
            S = S.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
        _close(L, torch.logsumexp(S, dim=-1).numpy(), 1e-13, f"logsumexp L causal={causal}")


def pin_row_subset_and_heads(attn):
    """Selected rows equal the same rows of the full result, and each (b, h) head is
    computed independently of the others."""
    r = _rng(21)
    B, H, n, d = 2, 2, 33, 8
    Q, K, V = (r.normal(size=(B, H, n, d)) for _ in range(3))
    for causal in (False, True):
        O, L = attn(Q, K, V, causal, 0.4)
        rows = [32, 0, 17, 5]
        Os, Ls = attn(Q, K, V, causal, 0.4, rows=rows)
        _close(Os, O[:, :, rows], 0.0, "row subset O")
        _close(Ls, L[:, :, rows], 0.0, "row subset L")
        for b in range(B):
            for h in range(H):
                Oh, Lh = attn(Q[b, h], K[b, h], V[b, h], causal, 0.4)
                _close(O[b, h], Oh, 0.0, f"head ({b},{h}) O")
                _close(L[b, h], Lh, 0.0, f"head ({b},{h}) L")


ALL_PINS = [
    pin_two_block_golden,
    pin_uniform_when_queries_zero,
    pin_single_key,
    pin_two_keys_logistic,
    pin_dominant_key,
    pin_probabilities,
    pin_value_linearity,
    pin_key_shift,
    pin_permutations,
    pin_causal_prefix,
    pin_torch_sdpa,
    pin_row_subset_and_heads,
]
