"""fp64 model of the tiled, streaming-softmax forward pass (CPU, slow, for pinning).

TEST INFRASTRUCTURE ONLY (same rule as ``oracle.attention``: only tests, the
smoke check and the CPU-baseline leg of the bench may import it).

Pages cited:
  [DF] "FlashAttention数据流优化：MI50显存与带宽瓶颈实战"  (kwkr.cn/news/544806)
  [OP] "FlashAttention优化原理与工程实践"                (lbrq.cn/news/50349)

This is the method, step by step, in the pages' order and notation:
  * [DF §2.2] first layer: Q is cut into blocks of ``block_q`` rows and K/V into
    blocks of ``block_k`` rows; each (Q block, K block) pair yields a local score
    tile that goes straight into the softmax and into the product with the
    matching V block, without the full score matrix ever existing.
  * [DF §2.2] second layer: while the key blocks of a row stream in, the row
    keeps its current max and its exp-sum; when all blocks are done the row is
    normalised with them.  Keeping a running max means earlier partial sums and
    partial outputs were taken relative to an older max, so they are rescaled by
    exp(old_max - new_max) whenever the max grows (the step that makes the
    blocked result equal to the plain definition).
  * [OP §2.1] the loop structure: an outer loop over query blocks i that loads
    Q_i, an inner loop over key blocks j that loads K_j, V_j and forms
    S_ij = Q_i K_jᵀ * scale, and a final store of O_i.  The page's sketch applies
    a per-block softmax with no rescale; read literally that equals attention only
    when there is a single key block, so the running-max form above is taken as
    what the sketch stands for.
  * [DF §4.1] causal flag: key j visible to row i iff j <= i.

Everything is fp64, so the result equals ``oracle.attention.attention_fp64`` up to
rounding order (the test requires 1e-12).  It exists to pin that the streaming
recurrence — which the GPU kernel implements in fp32 with base-2 exponentials —
is the definition, for the tile sizes and tile order the kernel uses.
"""

from __future__ import annotations

import numpy as np

__all__ = ["streaming_attention_fp64"]


def streaming_attention_fp64(q, k, v, scale: float, causal: bool, block_q: int = 128, block_k: int = 64,
                             key_block_order=None):
    """Streaming attention for one head.  q: [Lq,D], k/v: [Lk,D].  Returns (O, LSE) fp64.

    ``key_block_order`` optionally permutes the order in which key blocks are
    visited (any order must give the same result up to rounding).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Lq, D = q.shape
    Lk = k.shape[0]
    if causal and Lq != Lk:
        raise ValueError("causal attention is defined here only for Lq == Lk")
    O = np.zeros((Lq, v.shape[1]))
    LSE = np.zeros((Lq,))
    n_kb = (Lk + block_k - 1) // block_k
    order = list(range(n_kb)) if key_block_order is None else list(key_block_order)
    for i0 in range(0, Lq, block_q):                      # outer loop: load Q_i
        Qi = q[i0 : i0 + block_q]
        rows = np.arange(i0, i0 + Qi.shape[0])
        m = np.full(Qi.shape[0], -np.inf)                 # running row max
        l = np.zeros(Qi.shape[0])                         # running exp-sum
        acc = np.zeros((Qi.shape[0], v.shape[1]))         # un-normalised partial O
        for jb in order:                                  # inner loop: load K_j, V_j
            j0 = jb * block_k
            Kj, Vj = k[j0 : j0 + block_k], v[j0 : j0 + block_k]
            S = (Qi @ Kj.T) * scale                       # local score tile
            if causal:
                S[np.arange(j0, j0 + Kj.shape[0])[None, :] > rows[:, None]] = -np.inf
            m_new = np.maximum(m, S.max(axis=1))
            # rows that have seen no visible key yet keep a -inf max; use 0 as base
            base = np.where(np.isfinite(m_new), m_new, 0.0)
            alpha = np.exp(m - base)                      # rescale of earlier partials
            P = np.exp(S - base[:, None])
            l = alpha * l + P.sum(axis=1)
            acc = alpha[:, None] * acc + P @ Vj
            m = m_new
        O[i0 : i0 + Qi.shape[0]] = acc / l[:, None]       # normalise once per row
        LSE[i0 : i0 + Qi.shape[0]] = m + np.log(l)
    return O, LSE
