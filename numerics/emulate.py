"""The kernels' arithmetic carried out on the CPU with their roundings (fp32 / 16-bit).

Pages cited (title, then the section on that page):
  [DF] "FlashAttention数据流优化：MI50显存与带宽瓶颈实战"  (kwkr.cn/news/544806)
  [OP] "FlashAttention优化原理与工程实践"                (lbrq.cn/news/50349)

Forward ([DF §2.2], tiling and streaming softmax; [OP §4.1], half-precision
inputs with an fp32 softmax), per query row, key tiles of ``bc`` keys in order:

  t_j   = fl32(S_ij·c − m)       S_ij = fl32(q_i·k_j), c = fl32(|scale|·log2 e)
  m     moves to the tile max only when that exceeds it by more than ``tau``
        (then the sums and the partial output are scaled by 2^(m_old − m_new))
  p_j   = fl32(2^t_j),  p̃_j = round_dtype(p_j)
  l_f  += Σ p_j (fp32),  l_r += Σ p̃_j (fp32),  Õ += Σ p̃_j v_j (fp32)
  O     = round_dtype(fl32(Õ · fl32(1 / l_O)))    l_O = l_r (or l_f, see ``o_sum``)
  LSE   = fl32((m + log2 l_L)·ln 2)               l_L = l_f (or l_r, see ``lse_sum``)

Backward (recomputation from the kept statistics, [DF §2.2] third layer), with
the stored O and LSE of a forward pass:

  P_ij  = fl32(2^(S_ij·c − LSE_i·log2 e)),  c = fl32(scale·log2 e)
  Δ_i   = fl32(Σ_d dO_id·O_id) from the stored O
  dV_j  = round(Σ_i round(P_ij)·dO_i),  dP_ij = fl32(dO_i·v_j)
  dS_ij = round(fl32(W_ij·(dP_ij − Δ_i)))
  dQ_i  = round(scale·Σ_j dS_ij k_j),  dK_j = round(scale·Σ_i dS_ij q_i)

with W = P in the dQ kernel, and in the dK/dV kernel W = P at D = 64 but
W = round(P), the weights as rounded for the dV product, at D = 128 (its waves
pass them from the one that makes P to the one that makes dS in that form).

Sums are taken in fp32 by numpy (pairwise order) and products of 16-bit values
are exact in fp64 before their fp32 rounding; the kernels' own summation orders
differ at the level of 2^-24 relative, far below the rounding to 16 bits that
these models exist to capture.  ``round_p=False`` and ``exact=True`` switch the
roundings off (then the model is the streaming algorithm in fp64, which must
reproduce the definition).
"""

from __future__ import annotations

import numpy as np

LOG2E = 1.4426950408889634
LN2 = 0.6931471805599453


def _f32(x):
    return np.asarray(x, dtype=np.float32)


def _bf16_rne(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (round to nearest even) -> fp32; finite inputs only."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def round16(x32: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 -> the 16-bit input type with round to nearest even, returned as fp32."""
    if dtype == "bf16":
        return _bf16_rne(x32)
    return np.asarray(x32, dtype=np.float32).astype(np.float16).astype(np.float32)


def fwd_emulate_head(q, k, v, scale: float, causal: bool, dtype: str, rows=None, bc: int = 64, tau: float = 8.0,
                     o_sum: str = "l_r", lse_sum: str = "l_f", round_p: bool = True, exact: bool = False):
    """One head: q [Lq, D], k/v [Lk, D] holding the dtype-rounded inputs (any float array).

    Returns a dict: ``o`` (the stored output, fp64 of the 16-bit values), ``o32``
    (the fp32 result before its final rounding), ``lse`` (fp64 of the fp32 value),
    ``rescales`` (how many times each row's running max moved).
    ``o_sum`` / ``lse_sum`` pick which row sum divides O / enters LSE ("l_r": the
    rounded weights, "l_f": the fp32 weights).
    """
    ft = np.float64 if exact else np.float32
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Lq, D = q.shape
    Lk = k.shape[0]
    rows = np.arange(Lq) if rows is None else np.asarray(rows, dtype=np.int64)
    R = len(rows)
    off = Lk - Lq
    c = ft(abs(scale) * LOG2E) if scale != 0 else ft(LOG2E)
    qs = q[rows] * (np.sign(scale) if scale != 0 else 0.0)   # a negative scale negates Q, zero zeroes it (exact)
    m = np.full(R, -1e30, dtype=ft)
    l_f = np.zeros(R, dtype=ft)
    l_r = np.zeros(R, dtype=ft)
    acc = np.zeros((R, v.shape[1]), dtype=ft)
    moved = np.zeros(R, dtype=np.int64)
    n_t = (Lk + bc - 1) // bc
    for t in range(n_t):
        j = np.arange(t * bc, min(Lk, (t + 1) * bc))
        vis = (j[None, :] <= rows[:, None] + off) if causal else np.ones((R, len(j)), dtype=bool)
        if not vis.any():
            continue
        S = (qs @ k[j].T).astype(ft)                                  # fp32 scores of 16-bit inputs
        S = np.where(vis, S, -np.inf).astype(ft)
        m_tile = (S.max(axis=1) * c).astype(ft)
        grow = m_tile > m + ft(tau)
        m_new = np.where(grow, m_tile, m).astype(ft)
        alpha = np.exp2((m - m_new).astype(ft)).astype(ft)
        moved += grow
        m = m_new
        l_f = (l_f * alpha).astype(ft)
        l_r = (l_r * alpha).astype(ft)
        acc = (acc * alpha[:, None]).astype(ft)
        tt = (S.astype(np.float64) * float(c) - m.astype(np.float64)[:, None]).astype(ft)   # one rounding: FMA
        p = np.exp2(tt).astype(ft)
        pr = round16(p, dtype) if (round_p and not exact) else p
        l_f = (l_f + p.sum(axis=1, dtype=ft)).astype(ft)
        l_r = (l_r + pr.sum(axis=1, dtype=ft)).astype(ft)
        acc = (acc + (pr.astype(np.float64) @ v[j]).astype(ft)).astype(ft)
    lo = l_r if o_sum == "l_r" else l_f
    ll = l_f if lse_sum == "l_f" else l_r
    inv = (ft(1.0) / lo).astype(ft)
    o32 = (acc * inv[:, None]).astype(ft)
    o = o32.astype(np.float64) if exact else round16(o32.astype(np.float32), dtype).astype(np.float64)
    lse = ((m.astype(np.float64) + np.log2(ll.astype(np.float64))).astype(ft) * ft(LN2)).astype(ft)
    return {"o": o, "o32": o32.astype(np.float64), "lse": lse.astype(np.float64), "rescales": moved}


def bwd_emulate_head(q, k, v, o, lse, do, scale: float, causal: bool, dtype: str, exact: bool = False,
                     dk_weights: str = "auto"):
    """One head: the gradients the kernels compute from the stored o, lse (fp64 arrays).

    q [Lq, D], k/v [Lk, D], o/do [Lq, D] hold 16-bit values; lse [Lq] fp32 values.
    Returns (dq, dk, dv) as fp64 arrays of the rounded 16-bit results (exact=True:
    no rounding anywhere, fp64).  dk_weights: the weights dK's dS is formed from,
    "rounded" or "fp32"; "auto" as the kernels do (rounded at D = 128, fp32 at 64).
    """
    ft = np.float64 if exact else np.float32
    rnd = (lambda x: np.asarray(x, dtype=np.float64)) if exact else \
        (lambda x: round16(np.asarray(x, dtype=np.float32), dtype).astype(np.float64))
    q, k, v, o, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, o, do))
    Lq, Lk = q.shape[0], k.shape[0]
    c = ft(scale * LOG2E)
    lse2 = (np.asarray(lse, dtype=ft) * ft(LOG2E)).astype(ft)
    delta = (do * o).sum(axis=1).astype(ft)
    S = (q @ k.T).astype(ft)
    P = np.exp2((S.astype(np.float64) * float(c) - lse2.astype(np.float64)[:, None]).astype(ft)).astype(ft)
    if causal:
        P[np.arange(Lk)[None, :] > np.arange(Lq)[:, None] + (Lk - Lq)] = 0
    dP = (do @ v.T).astype(ft)
    if dk_weights == "auto":
        dk_weights = "rounded" if q.shape[1] == 128 else "fp32"
    dS = (P * (dP - delta[:, None]).astype(ft)).astype(ft)
    Pr, dSr = rnd(P), rnd(dS)
    dSr_k = dSr if dk_weights == "fp32" else rnd((Pr.astype(ft) * (dP - delta[:, None]).astype(ft)).astype(ft))
    dv = rnd((Pr.T @ do).astype(ft))
    dq = rnd(((dSr @ k).astype(ft) * ft(scale)).astype(ft))
    dk = rnd(((dSr_k.T @ q).astype(ft) * ft(scale)).astype(ft))
    return dq, dk, dv
