"""The fp64 oracle over every (batch, head) of a workload, one head per worker process.

Test infrastructure: the parity tests use it to compare every row of the full-size
workloads.  Each worker runs the unmodified ``oracle.attention_head_fp64`` with
single-threaded BLAS (``np.exp`` is single-threaded anyway, so heads in parallel
use the cores better than threads inside one head).  Inputs travel as fp32
(exact for fp16/bf16 values) and are widened to fp64 in the worker.
"""

from __future__ import annotations

import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np


def worker_count() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _one_head(args):
    from threadpoolctl import threadpool_limits

    from oracle import attention_head_fp64

    q, k, v, scale, causal, rows = args
    with threadpool_limits(1):
        O, L = attention_head_fp64(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), scale, causal,
                                   rows=rows)
    return O, L


def oracle_all_heads(q, k, v, scale: float, causal: bool, rows=None, heads=None, procs: int | None = None,
                     timeout: float = 900.0):
    """q [B,H,Lq,D], k/v [B,H,Lk,D] (CPU torch or numpy, 16-bit values).  Returns fp64 (O, LSE) with
    shapes [B,H,R,D] and [B,H,R] (R = len(rows) or Lq); heads not in ``heads`` are NaN."""
    to32 = lambda x: x.float().numpy() if hasattr(x, "float") else np.asarray(x, dtype=np.float32)
    q, k, v = to32(q), to32(k), to32(v)
    B, H, Lq, D = q.shape
    R = Lq if rows is None else len(rows)
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    O = np.full((B, H, R, v.shape[3]), np.nan)
    L = np.full((B, H, R), np.nan)
    jobs = [(q[b, h], k[b, h], v[b, h], scale, causal, rows) for b, h in pairs]
    n = min(procs or worker_count(), len(jobs))
    if n <= 1:
        res = map(_one_head, jobs)
        for (b, h), (o, l) in zip(pairs, res):
            O[b, h], L[b, h] = o, l
        return O, L
    # spawned (not forked) workers: the parent may hold GPU runtime threads; a worker that
    # cannot start makes map() raise instead of waiting for ever
    with ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn")) as ex:
        for (b, h), (o, l) in zip(pairs, ex.map(_one_head, jobs, timeout=timeout)):
            O[b, h], L[b, h] = o, l
    return O, L
