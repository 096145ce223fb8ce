"""Plain fp64 CPU attention: the definition the fused forward pass must reproduce.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this module; only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may.  It shares no code with the HIP kernels or their
binding.

Pages cited (title, then the section on that page):
  [DF] "FlashAttention数据流优化：MI50显存与带宽瓶颈实战"  (kwkr.cn/news/544806)
  [OP] "FlashAttention优化原理与工程实践"                (lbrq.cn/news/50349)

What is computed.  FlashAttention is exact attention computed in tiles, so the
oracle is the plain definition, not the tiled algorithm:

  * [OP §2.1] the conventional PyTorch form: scores = (q @ kᵀ) * scale over
    [B,H,L,L], a softmax along the last axis, then scores @ v giving [B,H,L,D].
  * [DF §2.1] the same three stages spelled out: QKᵀ, then a per-row softmax
    made of exp, a row sum and a division, then the product with V.
  * [DF §2.2] (second layer, streaming softmax) a row is normalised only after
    all of its key blocks are seen, using a running max and exp-sum; the max and
    exp-sum are the statistics kept for the backward pass ([DF §2.2], third
    layer).  The per-row log-sum-exp returned here is those two numbers folded
    into one: LSE = max + ln(sum_exp), in natural-log units of the scaled logits.
  * [DF §4.1] the ``causal=True`` flag: key j is visible to query row i iff
    j <= i (reading taken: diagonal included).  The pages never define the flag
    for Lq != Lk; the reading taken there is bottom-right alignment — the Lq
    query rows are the last Lq positions of the Lk keys, so j is visible to i iff
    j <= i + (Lk - Lq) — for Lq < Lk (every row still sees key 0), and Lq > Lk
    is rejected (rows with no visible key would have no softmax).

For every (b, h, i), with inputs upcast exactly to fp64:
  A_i   = {0..Lk-1}, or {0..i + Lk - Lq} when causal
  s_ij  = scale * sum_d q[b,h,i,d] * k[b,h,j,d]           for j in A_i
  m_i   = max_{j in A_i} s_ij
  p_ij  = exp(s_ij - m_i),  l_i = sum_{j in A_i} p_ij
  O_i   = sum_{j in A_i} p_ij * v[b,h,j,:] / l_i
  LSE_i = m_i + ln(l_i)

Numerics: fp64 throughout, BLAS for the two products (a library primitive used
as a step), two passes per row (max, then exp and sum).  Rows are processed in
chunks so that a chunk of S never exceeds ``chunk * Lk`` doubles.
Parity pins: tests/test_oracle.py (closed forms, invariants, brute force,
an independent library routine, hand-derived golden fixtures).
"""

from __future__ import annotations

import numpy as np

from .philox import dropout_keep, keep_threshold

__all__ = ["attention_fp64", "attention_head_fp64"]


def _as_f64(x) -> np.ndarray:
    """Exact upcast to fp64 of a numpy array or a CPU torch tensor (any float dtype)."""
    if hasattr(x, "detach"):  # a torch tensor; bf16 has no numpy dtype, so go through torch
        x = x.detach().to("cpu")
        import torch  # local: the oracle itself is numpy; torch only decodes bf16/fp16 bits

        return x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def attention_head_fp64(q, k, v, scale: float, causal: bool, rows=None, chunk: int = 1024,
                        dropout_p: float = 0.0, seed: int = 0, bh: int = 0):
    """One head.  q: [Lq, D], k/v: [Lk, D] (fp64).  Returns (O [R, D], LSE [R]) fp64.

    ``rows`` selects which query rows to evaluate (default: all, in order); each
    row is computed from its own definition, so a subset gives the same values
    as the full computation restricted to it.  ``dropout_p`` > 0 applies dropout
    to the normalised weights with the keep-mask of ``oracle/philox.py`` for
    (``bh``, row, key) and ``seed``; LSE is that of the weights before dropout.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Lq, D = q.shape
    Lk = k.shape[0]
    if k.shape != (Lk, D) or v.shape[0] != Lk:
        raise ValueError("k must be [Lk, D] and v must be [Lk, Dv]")
    if causal and Lq > Lk:
        raise ValueError("causal attention is defined here only for Lq <= Lk (bottom-right alignment)")
    off = Lk - Lq  # causal: query row i sits at key position i + off
    rows = np.arange(Lq) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.shape[0]
    O = np.empty((R, v.shape[1]), dtype=np.float64)
    LSE = np.empty((R,), dtype=np.float64)
    kT = np.ascontiguousarray(k.T)
    for c0 in range(0, R, chunk):
        r = rows[c0 : c0 + chunk]
        # stage 1: scores of the selected rows against every key ([OP §2.1], [DF §2.1])
        S = (q[r] @ kT) * scale
        if causal:
            # [DF §4.1] causal flag; reading: key j visible to row i iff j <= i + (Lk - Lq)
            S[np.arange(Lk)[None, :] > r[:, None] + off] = -np.inf
        # stage 2: softmax as max, exp, row sum ([DF §2.1] stage 2, [DF §2.2] second layer)
        m = S.max(axis=1)
        P = np.exp(S - m[:, None])
        l = P.sum(axis=1)
        if dropout_p:
            # [DF §4.1] dropout on the weights: kept ones scaled by 256/T (reading in philox.py)
            P = P * dropout_keep(bh, r, np.arange(Lk), dropout_p, seed) * (256.0 / keep_threshold(dropout_p))
        # stage 3: product with V, normalised once per row ([DF §2.1] stage 3, [DF §2.2])
        O[c0 : c0 + chunk] = (P @ v) / l[:, None]
        LSE[c0 : c0 + chunk] = m + np.log(l)
    return O, LSE


def attention_fp64(q, k, v, scale: float, causal: bool, rows=None, heads=None, chunk: int = 1024,
                   dropout_p: float = 0.0, seed: int = 0):
    """Batched attention.  q: [B,H,Lq,D], k/v: [B,H,Lk,D] (numpy or CPU torch, any float dtype).

    Returns (O, LSE) as fp64 numpy arrays of shapes [B,H,R,D] and [B,H,R], where R
    is ``len(rows)`` (default: every query row).  ``heads`` optionally restricts the
    computation to a list of (b, h) pairs; the other heads are then left as NaN.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, L, D]")
    B, H, Lq, D = q.shape
    if k.shape[:2] != (B, H) or v.shape[:3] != k.shape[:3] or k.shape[3] != D:
        raise ValueError("shape mismatch between q, k and v")
    R = Lq if rows is None else len(rows)
    O = np.full((B, H, R, v.shape[3]), np.nan)
    LSE = np.full((B, H, R), np.nan)
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    for b, h in pairs:
        O[b, h], LSE[b, h] = attention_head_fp64(q[b, h], k[b, h], v[b, h], scale, causal, rows, chunk,
                                                 dropout_p, seed, b * H + h)
    return O, LSE
