"""Philox4x32-10 counter-based random numbers and the dropout keep-mask built on them, numpy.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this module; only the tests may.  It shares no code with the HIP kernels.

Pages cited (title, then the section on that page):
  [DF] "FlashAttention数据流优化：MI50显存与带宽瓶颈实战"  (kwkr.cn/news/544806)

[DF §4.1] passes a dropout probability to the attention call and gives no random
number generator.  The reading taken: dropout draws its bits from Philox4x32-10,
the counter-based generator published by Salmon, Moraes, Dror and Shaw
("Parallel random numbers: as easy as 1, 2, 3", SC 2011), so that any element's
bits can be recomputed from its coordinates in the forward and backward passes
without storing a mask.  The generator, from that publication:

  * state: a 4-word counter X and a 2-word key K (32-bit words);
  * one round: with the products M0·X0 and M1·X2 split into high and low words,
        X ← (hi(M1·X2) ⊕ X1 ⊕ K0,  lo(M1·X2),  hi(M0·X0) ⊕ X3 ⊕ K1,  lo(M0·X0)),
    M0 = 0xD2511F53, M1 = 0xCD9E8D57;
  * ten rounds; between rounds the key advances by the Weyl constants
    W0 = 0x9E3779B9 (2^32 / golden ratio) and W1 = 0xBB67AE85 (2^32·(√3 − 1)).

Mask (reading, identical in every kernel and here): for (batch·head bh, query row
i, key j), the counter is (j // 4, i // 4, bh, 0) and the key (seed low word,
seed high word).  The 16 output bytes (word w, byte b, little-endian) cover the
4 x 4 block of rows 4·(i // 4) + w and keys 4·(j // 4) + b.  An element is kept
iff its byte < T, with T = round((1 − p)·256) in [1, 256]; kept weights are
scaled by 256 / T, so the expected output equals the output without dropout.

Pins (tests/test_oracle_dropout.py): the Weyl constants against their closed
forms, byte uniformity and independence statistics, the keep fraction,
unbiasedness of the dropped-out attention over many seeds, and the generator's
output words bit for bit against rocRAND's Philox4x32-10 engine (an independent
implementation, its header built for the host) on random and extreme counters
and keys.  The mask layout above is a reading of the pages' silence, not a pin.
"""

from __future__ import annotations

import numpy as np

__all__ = ["philox4x32_10", "keep_threshold", "dropout_keep"]

M0 = np.uint64(0xD2511F53)
M1 = np.uint64(0xCD9E8D57)
W0 = 0x9E3779B9
W1 = 0xBB67AE85
MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0: int, k1: int):
    """Philox4x32-10 of counters (arrays of uint32, broadcast together) under key (k0, k1).

    Returns four uint32 arrays (the output words 0..3)."""
    x0, x1, x2, x3 = (np.asarray(c, dtype=np.uint64) & MASK32 for c in (c0, c1, c2, c3))
    x0, x1, x2, x3 = np.broadcast_arrays(x0, x1, x2, x3)
    ka, kb = k0 & 0xFFFFFFFF, k1 & 0xFFFFFFFF
    for r in range(10):
        p0 = M0 * x0  # < 2^64: exact in uint64
        p1 = M1 * x2
        hi0, lo0 = p0 >> np.uint64(32), p0 & MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & MASK32
        x0, x1, x2, x3 = hi1 ^ x1 ^ np.uint64(ka), lo1, hi0 ^ x3 ^ np.uint64(kb), lo0
        ka, kb = (ka + W0) & 0xFFFFFFFF, (kb + W1) & 0xFFFFFFFF
    return tuple(x.astype(np.uint32) for x in (x0, x1, x2, x3))


def keep_threshold(p: float) -> int:
    """T = round((1 − p)·256), for 0 <= p < 1 with T >= 1 (else ValueError)."""
    if not (0.0 <= p < 1.0):
        raise ValueError("dropout probability must be in [0, 1)")
    t = int(np.floor((1.0 - p) * 256.0 + 0.5))
    if t < 1:
        raise ValueError("dropout probability too close to 1 (keep threshold 0)")
    return min(t, 256)


def dropout_keep(bh: int, rows, keys, p: float, seed: int) -> np.ndarray:
    """Boolean keep-mask [len(rows), len(keys)] of one (batch·head) for probability p and seed."""
    rows = np.asarray(rows, dtype=np.int64)
    keys = np.asarray(keys, dtype=np.int64)
    T = keep_threshold(p)
    if T == 256:
        return np.ones((rows.shape[0], keys.shape[0]), dtype=bool)
    I, J = np.meshgrid(rows, keys, indexing="ij")
    words = philox4x32_10(J // 4, I // 4, np.full(I.shape, bh), np.zeros(I.shape), seed & 0xFFFFFFFF,
                          (seed >> 32) & 0xFFFFFFFF)
    w = np.stack(words, axis=0)                             # [4, R, K]
    word = np.take_along_axis(w, (I % 4)[None].astype(np.int64), axis=0)[0]
    byte = (word >> (8 * (J % 4)).astype(np.uint32)) & np.uint32(0xFF)
    return byte < np.uint32(T)
