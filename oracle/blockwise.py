"""fp64 models of the online-softmax recurrences the pages describe.

TEST INFRASTRUCTURE ONLY (see the package docstring). These are not the oracle's
definition of attention -- that is ``attention.c`` -- but the *method* written
out plainly in numpy float64, so the tests can show that the recurrence reaches
the definition's result on the same inputs (tiled, ragged, causal, base 2).

Sources:
* "Writing a FlashAttention kernel in Metal", section "Online softmax": a
  running maximum m (starting at minus infinity) and a running normaliser l
  (starting at zero); each block first rescales l by exp(m - m_new), then adds
  the block's exp(x - m_new).
* same page, section "One-query attention": an unnormalised accumulator u of
  weighted value rows, rescaled by the same factor, divided by l at the end.
* same page, section "Blockwise attention and causal masking": per-row m, l
  and u for a block of query rows; causal masking of keys after the query to
  minus infinity, and ending the key loop at the first block that starts at or
  after the end of the query block.
* "FlashAttention-2 from PyTorch to Triton", sections "What We Are Building"
  and "Step 1": the tiled forward also returns L = m + log(l), and the output
  is divided by l once, after the last key tile.
* "Case Study: metal-flash-attention", online-softmax fragment: the same update
  in base 2, with the correction factor left at one unless the maximum grew.
"""

from __future__ import annotations

import math

import numpy as np

LOG2E = 1.0 / math.log(2.0)


def online_softmax(x, block_size: int):
    """Softmax of a 1-D vector via one pass of running max / running sum over blocks."""
    x = np.asarray(x, dtype=np.float64).reshape(-1)
    m = -math.inf
    l = 0.0
    for lo in range(0, x.size, block_size):
        chunk = x[lo:lo + block_size]
        m_next = max(m, float(chunk.max()))
        # Move the old sum onto the new maximum, then add this block on that scale.
        l = math.exp(m - m_next) * l + float(np.exp(chunk - m_next).sum())
        m = m_next
    return np.exp(x - m) / l


def one_query_attention(q, K, V, block_size: int, scale: float):
    """Attention output for one query vector, streaming key/value blocks.

    Returns (o, lse): the output row and the logsumexp of the scaled scores.
    """
    q = np.asarray(q, dtype=np.float64).reshape(-1)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    m = -math.inf
    l = 0.0
    u = np.zeros(V.shape[1], dtype=np.float64)
    for lo in range(0, K.shape[0], block_size):
        s = (K[lo:lo + block_size] @ q) * scale
        m_next = max(m, float(s.max()))
        alpha = math.exp(m - m_next)
        w = np.exp(s - m_next)
        l = alpha * l + float(w.sum())
        u = alpha * u + w @ V[lo:lo + block_size]
        m = m_next
    return u / l, m + math.log(l)


def blockwise_attention(Q, K, V, q_block: int, k_block: int, causal: bool, scale: float,
                        base2: bool = False, rescale_slack: float = 0.0,
                        reference_lead: float = 0.0):
    """Tiled attention forward over one [N, d] head: returns (O [N, d], L [N]).

    Query rows are taken q_block at a time; for each, key/value rows are streamed
    k_block at a time with per-row running (m, l, u). With ``causal`` the keys after
    a query are masked to minus infinity and the key loop stops at the first block
    lying wholly after the query block. N need not be a multiple of either block.

    ``base2`` runs the same recurrence in base 2: scores are multiplied by log2(e)
    and exponentiated with 2**x; L is brought back to natural log at the end.

    ``rescale_slack`` >= 0 lets a row keep its old reference maximum while the new
    block maximum exceeds it by no more than the slack (in the exponent's base), so
    the rescale of l and u is skipped on such blocks. Because u and l always share
    one reference, u / l and m + log(l) are unchanged in exact arithmetic; slack 0
    is the plain recurrence. Exponentials are then bounded by exp(slack).

    ``reference_lead`` >= 0 sets a reference that moves to the new maximum plus the
    lead, so a row moves it again only after its maximum has grown by more than
    lead + slack; the leading weights are then about exp(-lead). The same exact-
    arithmetic argument applies (any reference gives the same u / l and m + log l);
    lead 0 is the reference at the maximum.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    n, d = Q.shape
    n_keys = K.shape[0]
    expf = (lambda z: np.exp2(z)) if base2 else (lambda z: np.exp(z))
    logf = (lambda z: np.log2(z)) if base2 else (lambda z: np.log(z))
    mult = scale * LOG2E if base2 else scale
    O = np.empty((n, V.shape[1]), dtype=np.float64)
    L = np.empty(n, dtype=np.float64)
    for q0 in range(0, n, q_block):
        rows = min(q_block, n - q0)
        qi = Q[q0:q0 + rows]
        m = np.full((rows, 1), -np.inf)
        l = np.zeros((rows, 1))
        u = np.zeros((rows, V.shape[1]))
        for k0 in range(0, n_keys, k_block):
            if causal and k0 >= q0 + rows:
                break  # this block and all later ones lie after every query here
            kj = K[k0:k0 + k_block]
            vj = V[k0:k0 + k_block]
            s = (qi @ kj.T) * mult
            if causal:
                qpos = np.arange(q0, q0 + rows)[:, None]
                kpos = np.arange(k0, k0 + kj.shape[0])[None, :]
                s = np.where(kpos > qpos, -np.inf, s)
            bmax = s.max(axis=1, keepdims=True)
            grow = bmax > m + rescale_slack
            m_next = np.where(grow, np.maximum(m, bmax) + reference_lead, m)
            with np.errstate(invalid="ignore"):
                alpha = np.where(np.isneginf(m), 0.0, expf(m - m_next))
            w = expf(s - m_next)
            l = alpha * l + w.sum(axis=1, keepdims=True)
            u = alpha * u + w @ vj
            m = m_next
        O[q0:q0 + rows] = u / l
        lse = m + logf(l)
        L[q0:q0 + rows] = (lse / LOG2E if base2 else lse).reshape(-1)
    return O, L
