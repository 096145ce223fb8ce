"""Absolute error terms of the backward pass that the relative bars do not cover.

The kernels take Δ_i = dO_i·O_i from the stored output O, rounded to the input
type (the standard recomputing backward pass does the same).  Where a row's
softmax is peaked, the exact dP_ij − Δ_i is tiny and so are dQ and dK, while the
rounding of O perturbs Δ_i by up to E_i = u·Σ_d |dO_id|·|O_id| (u = 2^-8 for
bf16, 2^-11 for fp16: twice the unit roundoff of the stored O).  Through
dS_ij = P_ij (dP_ij − Δ_i) this reaches

    |δdQ_i| <= |scale|·E_i·max_j ‖k_j‖∞                 (Σ_j P_ij = 1)
    |δdK_j| <= |scale|·Σ_i P_ij·E_i·‖q_i‖∞

and leaves dV untouched.  These are added to the relative bars; they matter
only where the exact gradient is of the order of the rounding of O.
"""

from __future__ import annotations

import numpy as np

U_OUT = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11}


def delta_bounds(q, k, do, O_ref, L_ref, scale, causal, dtype, heads):
    """Per (b, h) in heads: (bound for dQ rows [Lq, 1], bound for dK rows [Lk, 1]), fp64."""
    q, k, do = (x.double().numpy() if hasattr(x, "double") else np.asarray(x, dtype=np.float64) for x in (q, k, do))
    out = {}
    for b, h in heads:
        Lq, Lk = q.shape[2], k.shape[2]
        E = U_OUT[dtype] * np.abs(do[b, h] * O_ref[b, h]).sum(axis=1)          # [Lq]
        bq = abs(scale) * E * np.abs(k[b, h]).max()
        qn = np.abs(q[b, h]).max(axis=1)
        bk = np.zeros(Lk)
        for c0 in range(0, Lq, 1024):
            r = np.arange(c0, min(Lq, c0 + 1024))
            S = scale * q[b, h][r] @ k[b, h].T
            if causal:
                S[np.arange(Lk)[None, :] > r[:, None] + (Lk - Lq)] = -np.inf
            P = np.exp(S - L_ref[b, h][r][:, None])
            bk += (P * (E[r] * qn[r])[:, None]).sum(axis=0)
        out[(b, h)] = (bq[:, None], abs(scale) * bk[:, None])
    return out
