"""The exact gradient, and the exact result of the backward's formulas evaluated on a
stored forward output O and logsumexp L (test infrastructure: oracle calls only).

The backward recomputes P = exp(S - L) from the stored L and takes D = sum_c dO O from the
stored O ("FlashAttention-2 from PyTorch to Triton", section "What We Are Building").
With lambda_i = L_stored_i - L_i and dD_i = sum_c dO_ic (O_stored_ic - O_ic), the result
of those formulas differs from the exact gradient by terms that are linear in the rows
of dO (alpha_i = exp(-lambda_i) - 1, beta_i = exp(-lambda_i) dD_i):

    dV' = dV + dV[alpha dO]
    dQ' = dQ + dQ[alpha dO] - scale beta (P K)
    dK' = dK + dK[alpha dO] - scale P^T (beta Q)

X[g] is the exact gradient for the upstream gradient g: the backward oracle with dO
replaced by alpha dO, or by beta Q (its dV is P^T (beta Q)); P K is the forward oracle with
V replaced by K.
"""

import numpy as np

import oracle


def stored_statistics_gradient(q, k, v, do, O, L, causal, scale):
    """Exact gradient (dQ, dK, dV) and the exact result of the method's backward formulas
    evaluated on the stored O and L (module docstring), all fp64 numpy from oracle calls."""
    qn, kn, vn, dn = (t.double().numpy() for t in (q, k, v, do))
    ref = oracle.attention_bwd(qn, kn, vn, dn, causal, scale)
    Oref, Lref = oracle.attention(qn, kn, vn, causal, scale)
    lam = L.double().cpu().numpy() - Lref                               # [B, H, N]
    dD = np.sum(dn * (O.double().cpu().numpy() - Oref), axis=-1)        # [B, H, N]
    alpha = np.expm1(-lam)[..., None]
    beta = (np.exp(-lam) * dD)[..., None]
    dq_a, dk_a, dv_a = oracle.attention_bwd(qn, kn, vn, alpha * dn, causal, scale)
    pbq = oracle.attention_bwd(qn, kn, vn, beta * qn, causal, scale)[2]  # P^T (beta Q)
    pk, _ = oracle.attention(qn, kn, kn, causal, scale)                 # P K
    stored = (ref[0] + dq_a - scale * beta * pk, ref[1] + dk_a - scale * pbq, ref[2] + dv_a)
    return ref, stored
