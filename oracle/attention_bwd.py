"""Plain fp64 CPU gradients of attention: the definition the backward kernels must reproduce.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this module; only the tests may.  It shares no code with the HIP kernels or
their binding.

Pages cited (title, then the section on that page):
  [DF] "FlashAttention数据流优化：MI50显存与带宽瓶颈实战"  (kwkr.cn/news/544806)

What is computed.  [DF §2.2] (third layer, recomputation) says the backward
pass keeps no score matrix: it recomputes the score blocks from Q and K with the
softmax statistics the forward pass kept.  The pages give no gradient formulas,
so the target is the exact gradient of the forward definition (the one in
``oracle/attention.py``) for an upstream gradient dO of the output:

  O_i  = sum_j P_ij v_j,   P_ij = exp(s_ij) / sum_{j' in A_i} exp(s_ij'),
  s_ij = scale * q_i . k_j  (j in A_i; P_ij = 0 outside A_i)

and, by the chain rule (the softmax Jacobian of each row applied to dP):

  dV_j  = sum_i P_ij dO_i                       (from O = P V)
  dP_ij = dO_i . v_j
  dS_ij = P_ij * (dP_ij - sum_j' P_ij' dP_ij')  (row-wise softmax Jacobian)
  dQ_i  = scale * sum_j dS_ij k_j
  dK_j  = scale * sum_i dS_ij q_i

The visible sets A_i are the forward's: all keys, or j <= i + (Lk - Lq) when
causal (Lq <= Lk).  The softmax is recomputed here from Q and K directly (max
subtracted for range, then normalised), not from a stored LSE, so the
definition does not depend on any forward output.

Numerics: fp64 throughout, BLAS for the products (library primitives used as
steps), rows in chunks so a chunk of S never exceeds ``chunk * Lk`` doubles;
dK and dV accumulate over the chunks.  Parity pins: tests/test_oracle_bwd.py
(central finite differences of the forward oracle, torch autograd in fp64 on
the CPU, closed forms and invariants, planted mistakes).
"""

from __future__ import annotations

import numpy as np

from .philox import dropout_keep, keep_threshold

__all__ = ["attention_bwd_fp64", "attention_bwd_head_fp64"]


def _as_f64(x) -> np.ndarray:
    """Exact upcast to fp64 of a numpy array or a CPU torch tensor (any float dtype)."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch  # local: decodes bf16/fp16 bits only

        return x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def attention_bwd_head_fp64(q, k, v, do, scale: float, causal: bool, chunk: int = 1024, dropout_p: float = 0.0,
                            seed: int = 0, bh: int = 0):
    """One head.  q, do: [Lq, D]; k, v: [Lk, D] (fp64).  Returns (dQ [Lq,D], dK [Lk,D], dV [Lk,D]).

    With ``dropout_p`` > 0 the forward output is O = (P ∘ M) V, M = keep·256/T the
    dropout factors of ``oracle/philox.py`` for (``bh``, row, key) and ``seed``."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    Lq, D = q.shape
    Lk = k.shape[0]
    if k.shape != (Lk, D) or v.shape[0] != Lk or do.shape != (Lq, v.shape[1]):
        raise ValueError("q, do must be [Lq, D]; k, v must be [Lk, D]")
    if causal and Lq > Lk:
        raise ValueError("causal attention is defined here only for Lq <= Lk (bottom-right alignment)")
    off = Lk - Lq
    dQ = np.empty_like(q)
    dK = np.zeros_like(k)
    dV = np.zeros_like(v)
    for c0 in range(0, Lq, chunk):
        r = np.arange(c0, min(Lq, c0 + chunk))
        # recompute the forward's probabilities of these rows ([DF §2.2], third layer)
        S = (q[r] @ k.T) * scale
        if causal:
            S[np.arange(Lk)[None, :] > r[:, None] + off] = -np.inf
        E = np.exp(S - S.max(axis=1, keepdims=True))
        P = E / E.sum(axis=1, keepdims=True)
        # dropout factors M (all ones without dropout): O = (P ∘ M) V
        M = None
        if dropout_p:
            M = dropout_keep(bh, r, np.arange(Lk), dropout_p, seed) * (256.0 / keep_threshold(dropout_p))
        Pd = P if M is None else P * M
        # gradient to V, and to P through the dropout factors
        dV += Pd.T @ do[r]
        dP = do[r] @ v.T
        if M is not None:
            dP = dP * M
        # row-wise softmax Jacobian: dS = P * (dP - <P, dP>_row)
        dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
        # s = scale * q . k: gradients to q and k
        dQ[r] = scale * (dS @ k)
        dK += scale * (dS.T @ q[r])
    return dQ, dK, dV


def attention_bwd_fp64(q, k, v, do, scale: float, causal: bool, heads=None, chunk: int = 1024,
                       dropout_p: float = 0.0, seed: int = 0):
    """Batched gradients.  q, do: [B,H,Lq,D]; k, v: [B,H,Lk,D] (numpy or CPU torch, any float dtype).

    Returns (dQ, dK, dV) as fp64 numpy arrays of the inputs' shapes.  ``heads``
    optionally restricts the computation to a list of (b, h) pairs; the other
    heads are left as NaN.
    """
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4 or do.shape != q.shape[:3] + (v.shape[3],):
        raise ValueError("q, do must be [B, H, Lq, D] and k, v [B, H, Lk, D]")
    B, H = q.shape[:2]
    if k.shape[:2] != (B, H) or v.shape[:3] != k.shape[:3] or k.shape[3] != q.shape[3]:
        raise ValueError("shape mismatch between q, k and v")
    dQ = np.full(q.shape, np.nan)
    dK = np.full(k.shape, np.nan)
    dV = np.full(v.shape, np.nan)
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    for b, h in pairs:
        dQ[b, h], dK[b, h], dV[b, h] = attention_bwd_head_fp64(q[b, h], k[b, h], v[b, h], do[b, h], scale,
                                                               causal, chunk, dropout_p, seed, b * H + h)
    return dQ, dK, dV
