"""Rounding of the 16-bit formats and the error allowances of the parity bars.

Pages cited (title, then the section on that page):
  [DF] "FlashAttention数据流优化：MI50显存与带宽瓶颈实战"  (kwkr.cn/news/544806)
  [OP] "FlashAttention优化原理与工程实践"                (lbrq.cn/news/50349)

The forward pass is exact attention computed in tiles ([DF §2.2]), so the GPU
result is compared with the fp64 definition.  What separates them is rounding:
half-precision inputs with an fp32 softmax ([OP §4.1]) and the kernel's own
choices (weights rounded to the input type before they multiply V, O divided by
the sum of those rounded weights, O rounded to the input type at the end).

Forward bar per element (tol = 2e-3 for fp16, 1e-2 for bf16):

    |O_gpu − O_ref| <= tol,
    or, only where the output format itself is coarser than tol there,
    |O_gpu − O_ref| <= half_ulp(|O_ref| + E) + E    when half_ulp(|O_ref| + E) > tol

where E bounds the error of the unrounded fp32 result (see ``fwd_allowance``).
Rounding a value of magnitude in [4, 8) to bf16 (or [8, 16) to fp16) can alone
move it by more than tol, so no implementation that stores O in the input type
can promise tol there; everywhere else the plain tol applies.
"""

from __future__ import annotations

import numpy as np

# stored significand bits and smallest normal exponent of the formats
_FMT = {"fp16": (10, -14), "bf16": (7, -126)}
# unit roundoff of round-to-nearest-even: 2^-(significand bits incl. the implicit one)
_U = {"fp16": 2.0 ** -11, "bf16": 2.0 ** -8}


def unit_roundoff(dtype: str) -> float:
    return _U[dtype]


def _exponent(x: np.ndarray, dtype: str) -> np.ndarray:
    """floor(log2|x|), clamped to the format's smallest normal exponent (exact, via frexp)."""
    _, ex = np.frexp(np.abs(np.asarray(x, dtype=np.float64)))
    return np.maximum(ex.astype(np.int64) - 1, _FMT[dtype][1])


def half_ulp(x, dtype: str) -> np.ndarray:
    """Half the spacing of the format's values at |x|: the largest error of rounding x to nearest."""
    return 0.5 * np.ldexp(1.0, _exponent(x, dtype) - _FMT[dtype][0])


def round_to_dtype(x, dtype: str) -> np.ndarray:
    """x (fp64) rounded to nearest-even fp16 / bf16, returned as fp64 (no overflow handling: |x| < 6e4)."""
    x = np.asarray(x, dtype=np.float64)
    q = np.ldexp(1.0, _exponent(x, dtype) - _FMT[dtype][0])
    return np.rint(x / q) * q


# fp32 budget of one weight before it is rounded: the fp32 score (a dot product of up
# to 128 products accumulated in fp32), the folded scale, the exponent and the
# rescales by the running max each contribute a few units of 2^-24 times the
# score's magnitude; 1e-4 covers scores up to several hundred
EPS_P = 1e-4


def _head_weights(q, k, scale: float, causal: bool, rows: np.ndarray) -> np.ndarray:
    """fp64 softmax weights of the given rows of one head ([R, Lk]), from the definition."""
    Lq, Lk = q.shape[0], k.shape[0]
    S = scale * (q[rows] @ k.T)
    if causal:
        S[np.arange(Lk)[None, :] > rows[:, None] + (Lk - Lq)] = -np.inf
    P = np.exp(S - S.max(axis=1, keepdims=True))
    return P / P.sum(axis=1, keepdims=True)


def fwd_allowance(q, k, v, O_ref, scale: float, causal: bool, dtype: str, rows, keep=None,
                  keep_scale: float = 1.0) -> np.ndarray:
    """E for every element of the given rows of one head ([R, D]).

    The kernel multiplies V by p̃_j = p_j(1 + δ_j), |δ_j| <= u + EPS_P (u: unit
    roundoff of the input type) and divides by Σ p̃_j, so its unrounded output is
    Σ_j w_j (1 + δ_j) v_j / (1 + δ̄) with δ̄ = Σ_j w_j δ_j, whose distance from the
    exact O = Σ_j w_j v_j is

        |Σ_j w_j (δ_j − δ̄)(v_j − O)| / (1 + δ̄) <= 2(u + EPS_P)/(1 − u − EPS_P) · Σ_j w_j |v_j − O|.

    Adding the fp32 accumulation of Σ p̃_j v_j (one rounding per 16 keys along the
    chain, plus the normalisation and the rescales): (n/16 + 4)·2^-24 · Σ_j w_j |v_j|.

    With dropout (``keep``: the [R, Lk] keep mask of the rows, ``keep_scale``: the
    factor of kept weights) the output s·Σ_j w_j keep_j v_j is no longer a convex
    combination and the first term becomes 2(u + EPS_P)/(1 − u − EPS_P)·s·Σ_j w_j keep_j |v_j|.
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    rows = np.asarray(rows, dtype=np.int64)
    W = _head_weights(q, k, scale, causal, rows)
    Lq, Lk = q.shape[0], k.shape[0]
    n = (rows + (Lk - Lq) + 1).clip(max=Lk) if causal else np.full(rows.shape, Lk)
    u = _U[dtype] + EPS_P
    O = np.asarray(O_ref, dtype=np.float64)
    if keep is not None:
        Wk = W * np.asarray(keep, dtype=np.float64) * keep_scale
        dev = mag = Wk @ np.abs(v)
    else:
        dev = np.stack([W[i] @ np.abs(v - O[i]) for i in range(len(rows))]) if len(rows) else np.zeros(O.shape)
        mag = W @ np.abs(v)
    return 2 * u / (1 - u) * dev + ((n / 16 + 4) * 2.0 ** -24)[:, None] * mag


def fwd_check(o_gpu, O_ref, dtype: str, tol: float, allowance=None):
    """Classify a forward result against the bar.

    o_gpu, O_ref: fp64 arrays of one head's rows [R, D].  ``allowance(idx_rows)``
    returns E for those rows ([len, D]); it is called only for rows holding
    elements over tol.  Returns (ok: bool, info: dict).
    """
    err = np.abs(o_gpu - O_ref)
    over = err > tol
    info = {"max_abs_err": float(err.max()) if err.size else 0.0, "n_over_tol": int(over.sum()), "n_allowed": 0}
    if not over.any():
        return True, info
    if allowance is None:
        return False, info
    rows = np.unique(np.nonzero(over)[0])
    E = allowance(rows)
    Orow, erow = O_ref[rows], err[rows]
    hu = half_ulp(np.abs(Orow) + E, dtype)
    granted = hu > tol
    ok_el = (erow <= tol) | (granted & (erow <= hu + E))
    info["n_allowed"] = int((granted & (erow > tol) & ok_el).sum())
    if info["n_allowed"]:
        sel = granted & (erow > tol)
        info["allowed_max_abs_o_ref"] = float(np.abs(Orow[sel]).max())
        info["allowed_max_err"] = float(erow[sel].max())
    if not ok_el.all():
        r, d = np.unravel_index(np.argmax(np.where(ok_el, -np.inf, erow - np.maximum(tol, hu + E))), erow.shape)
        info["worst"] = {"row": int(rows[r]), "dim": int(d), "err": float(erow[r, d]), "o_ref": float(Orow[r, d]),
                         "allowance": float(E[r, d]), "half_ulp": float(hu[r, d])}
        return False, info
    return True, info


# ---------------------------------------------------------------------------------------
# backward pass: the effect of the stored (rounded) O on Δ = dO·O
# ---------------------------------------------------------------------------------------

# twice the unit roundoff of the stored O: |O_stored − O| <= u|O| per element, and the
# kernel's own O differs from the exact O by about as much again
U_OUT = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11}


def delta_bounds(q, k, do, O_ref, L_ref, scale, causal, dtype, heads):
    """Absolute error terms of dQ and dK that the relative bars do not cover.

    The kernels take Δ_i = dO_i·O_i from the stored output O, rounded to the input
    type (the recomputing backward pass of [DF §2.2], third layer, keeps O and the
    row statistics).  Where a row's softmax is peaked, the exact dP_ij − Δ_i is tiny
    and so are dQ and dK, while the rounding of O perturbs Δ_i by up to
    E_i = U_OUT·Σ_d |dO_id|·|O_id|.  Through dS_ij = P_ij (dP_ij − Δ_i) this reaches

        |δdQ_i| <= |scale|·E_i·max_j ‖k_j‖∞                 (Σ_j P_ij = 1)
        |δdK_j| <= |scale|·Σ_i P_ij·E_i·‖q_i‖∞

    and leaves dV untouched.  Per (b, h) in heads: (bound for dQ rows [Lq, 1],
    bound for dK rows [Lk, 1]), fp64.
    """
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
