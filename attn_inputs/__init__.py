"""Seeded synthetic inputs for the attention forward pass (shared by tests, bench and smoke).

This module only draws and rounds numbers; it holds none of the attention
arithmetic (no softmax, no weighted sums).  The one place it forms dot products
is the peaked-softmax recipe of the numerics-stress workload, which needs the
logit of each row's target key to exceed the others by a set margin.

Pages cited:
  [DF] "FlashAttention数据流优化：MI50显存与带宽瓶颈实战"  (kwkr.cn/news/544806)

Recipe (fixed before any GPU run; the seeds are part of the workload):
  * numpy ``Generator(PCG64(seed))``; Q, then K, then V drawn with
    ``standard_normal`` in C order over [B, H, L, D] (drawing in consecutive
    chunks gives the same stream as one draw);
  * each value multiplied by its sigma in fp64, cast to fp32 (round to nearest
    even), then to fp16/bf16 (round to nearest even) with torch;
  * the numerics-stress workload then draws one target key per query row and
    moves that row of Q along its target key so the target's logit exceeds every
    other logit of the row by ``boost`` (before Q is rounded).

The workloads:
  * ``tiny``        B1 H1 L128 D64 fp16, non-causal — the 128×128×64 example of
                    [DF §2.1].
  * ``llama7b_2k``  B1 H32 L2048 D128 fp16, causal — the Llama-2-7B attention
                    shape of [DF §3.1] (sequence 2048, batch 1, 32 heads of 128).
  * ``train7b_4k``  B4 H32 L4096 D128 bf16, causal — the 7B, 4K-context training
                    shape of [DF §1].
  * ``stress_8k``   B2 H16 L8192 D64 bf16, non-causal, Q ~ N(0, 3²) plus a
                    20-logit boost of one key per row (peaked softmax).
  * ``long_16k``    B1 H32 L16384 D128 bf16, causal.
iid Gaussians stand in for the activations of the Llama models the pages run;
no weights or datasets are used.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np
from threadpoolctl import threadpool_limits

__all__ = ["Workload", "WORKLOADS", "make_inputs", "make_custom", "draw_normal", "round_to"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Lq: int
    Lk: int
    D: int
    dtype: str          # "fp16" | "bf16"
    causal: bool
    seed: int
    sigma_q: float = 1.0
    boost: float | None = None   # logit margin of one target key per row (None: no boost)
    description: str = ""
    splits: int = 1              # key splits the workload is timed with (fa_fwd_splitkv when > 1)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def flops(self) -> float:
        """4·B·H·Lq·Lk·D, halved when causal (the metric's convention).

        Causal with Lq < Lk (queries aligned with the last Lq keys) counts
        4·B·H·Lq·(Lk − Lq/2)·D, which is the same convention: Lq = Lk gives half.
        """
        if self.causal:
            return 4.0 * self.B * self.H * self.Lq * (self.Lk - self.Lq / 2) * self.D
        return 4.0 * self.B * self.H * self.Lq * self.Lk * self.D

    @property
    def hbm_bytes(self) -> int:
        """Algorithmic HBM bytes: Q, K, V read once, O written once (dtype), LSE written (fp32)."""
        return 2 * (2 * self.B * self.H * self.Lq * self.D + 2 * self.B * self.H * self.Lk * self.D) \
            + 4 * self.B * self.H * self.Lq


WORKLOADS: dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny", 1, 1, 128, 128, 64, "fp16", False, 1001,
                 description="B=1 H=1 Lq=Lk=128 D=64 fp16 non-causal"),
        Workload("llama7b_2k", 1, 32, 2048, 2048, 128, "fp16", True, 1002,
                 description="Llama-2-7B attention shape: B=1 H=32 L=2048 D=128 fp16 causal"),
        Workload("train7b_4k", 4, 32, 4096, 4096, 128, "bf16", True, 1003,
                 description="7B 4K-context training shape: B=4 H=32 L=4096 D=128 bf16 causal"),
        Workload("stress_8k", 2, 16, 8192, 8192, 64, "bf16", False, 1004, sigma_q=3.0, boost=20.0,
                 description="numerics stress: B=2 H=16 L=8192 D=64 bf16 non-causal, peaked softmax"),
        Workload("long_16k", 1, 32, 16384, 16384, 128, "bf16", True, 1005,
                 description="long sequence: B=1 H=32 L=16384 D=128 bf16 causal"),
    ]
}


# Inference shapes whose query tiles alone leave most of the 256 CUs idle: timed
# with key splits (fa_fwd_splitkv).  Causal ones align the queries with the last
# Lq keys (a prefill chunk or a decode step over a KV cache).
SPLIT_WORKLOADS: dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("kvcache_16k", 1, 32, 256, 16384, 128, "bf16", False, 1006, splits=8,
                 description="256 queries over a 16K KV cache: B=1 H=32 Lq=256 Lk=16384 D=128 bf16, 8 key splits"),
        Workload("decode_32k", 1, 8, 1, 32768, 128, "bf16", True, 1007, splits=32,
                 description="one decode step over a 32K KV cache: B=1 H=8 Lq=1 Lk=32768 D=128 bf16 causal, "
                             "32 key splits"),
        Workload("prefill_chunk_8k", 2, 32, 512, 8192, 128, "bf16", True, 1008, splits=2,
                 description="a 512-row prefill chunk after 7.7K cached keys: B=2 H=32 Lq=512 Lk=8192 D=128 bf16 "
                             "causal, 2 key splits"),
    ]
}

ALL_WORKLOADS: dict[str, Workload] = {**WORKLOADS, **SPLIT_WORKLOADS}


def _torch_dtype(dtype: str):
    import torch

    return {"fp16": torch.float16, "bf16": torch.bfloat16}[dtype]


def draw_normal(rng: np.random.Generator, shape, chunk: int = 1 << 23) -> np.ndarray:
    """standard_normal over ``shape`` in C order, drawn in consecutive chunks (fp64)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float64)
    for s in range(0, n, chunk):
        out[s : s + chunk] = rng.standard_normal(min(chunk, n - s))
    return out.reshape(shape)


def round_to(x: np.ndarray, dtype: str):
    """fp64 → fp32 (RNE) → fp16/bf16 (RNE).  Returns a contiguous CPU torch tensor."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(_torch_dtype(dtype)).contiguous()


def _boost_head(q: np.ndarray, k: np.ndarray, targets: np.ndarray, scale: float, margin: float,
                chunk: int = 1024, max_iter: int = 32) -> np.ndarray:
    """Move each row of q along its target key so that its target logit leads by ``margin``.

    q: [L, D] fp64 (not yet rounded), k: [L, D] fp64 (already rounded), targets: [L].
    With s_j = scale·q·k_j and rho_j = k_t·k_j/|k_t|², adding (c/|k_t|²)·k_t to q shifts
    s_t by scale·c and s_j by scale·c·rho_j.  The margin is piecewise linear in c; Newton
    on the currently largest competitor j* converges in a few steps.
    """
    q = q.copy()
    kT = np.ascontiguousarray(k.T)
    for r0 in range(0, q.shape[0], chunk):
        t = targets[r0 : r0 + chunk]
        n = t.shape[0]
        ar = np.arange(n)
        kt = k[t]                                   # [n, D] target keys
        nt = np.einsum("nd,nd->n", kt, kt)          # |k_t|²
        S = (q[r0 : r0 + n] @ kT) * scale           # [n, L] logits before the boost
        rho = (kt @ kT) / nt[:, None]               # [n, L]
        st = S[ar, t]
        c = np.zeros(n)
        jstar = np.full(n, -1)
        for _ in range(max_iter):
            comp = S + (scale * c)[:, None] * rho
            comp[ar, t] = -np.inf
            jn = comp.argmax(axis=1)
            c = (margin + S[ar, jn] - st) / (scale * (1.0 - rho[ar, jn]))
            if np.array_equal(jn, jstar):
                break
            jstar = jn
        q[r0 : r0 + n] += (c / nt)[:, None] * kt
    return q


def make_inputs(w: Workload | str, seed: int | None = None) -> dict:
    """Draw the workload's Q, K, V (CPU torch tensors of the workload's dtype).

    Returns a dict with q, k, v, scale, causal, dtype, the workload, and (for a
    boosted workload) the per-row target key indices as an int64 numpy array.
    """
    if isinstance(w, str):
        w = ALL_WORKLOADS[w]
    seed = w.seed if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    qs = (w.B, w.H, w.Lq, w.D)
    ks = (w.B, w.H, w.Lk, w.D)
    q64 = draw_normal(rng, qs) * w.sigma_q
    k = round_to(draw_normal(rng, ks), w.dtype)
    v = round_to(draw_normal(rng, ks), w.dtype)
    targets = None
    if w.boost is not None:
        import torch

        targets = rng.integers(0, w.Lk, size=(w.B, w.H, w.Lq))
        k64 = k.to(torch.float64).numpy()
        heads = [(b, h) for b in range(w.B) for h in range(w.H)]

        def one(bh):
            b, h = bh
            q64[b, h] = _boost_head(q64[b, h], k64[b, h], targets[b, h], w.scale, w.boost)

        # heads are independent; single-threaded BLAS per head keeps the bits
        # independent of the worker count
        with threadpool_limits(1), ThreadPoolExecutor(max_workers=max(1, min(16, os.cpu_count() or 1))) as ex:
            list(ex.map(one, heads))
    q = round_to(q64, w.dtype)
    return dict(q=q, k=k, v=v, scale=w.scale, causal=w.causal, dtype=w.dtype, workload=w, targets=targets)


def make_dout(shape, dtype: str, seed: int, sigma: float = 1.0):
    """An upstream gradient dO for the backward pass: standard normal × sigma over ``shape`` in C
    order from PCG64(seed), rounded as Q, K, V are.  Returns a CPU torch tensor."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return round_to(draw_normal(rng, tuple(shape)) * sigma, dtype)


def make_custom(B: int, H: int, Lq: int, Lk: int, D: int, dtype: str, causal: bool, seed: int,
                sigma_q: float = 1.0, sigma_k: float = 1.0, sigma_v: float = 1.0) -> dict:
    """Same recipe for an arbitrary shape (parity edge cases)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = round_to(draw_normal(rng, (B, H, Lq, D)) * sigma_q, dtype)
    k = round_to(draw_normal(rng, (B, H, Lk, D)) * sigma_k, dtype)
    v = round_to(draw_normal(rng, (B, H, Lk, D)) * sigma_v, dtype)
    return dict(q=q, k=k, v=v, scale=1.0 / math.sqrt(D), causal=causal, dtype=dtype)
