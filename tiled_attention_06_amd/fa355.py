"""The forward call under its short name: ``fa355.fwd(q, k, v, *, causal=False, scale=None) -> (o, lse)``.

``from tiled_attention_06_amd import fa355``.  Argument marshalling only, through
``fa_fwd`` of the package (the C ``fa_fwd`` for dense tensors, ``fa_fwd_strided``
for views): q [B, H, Lq, D], k and v [B, H, Lk, D] (fp16 or bf16, on one GPU);
``scale`` None means 1/sqrt(D); o is allocated in q's shape and dtype, lse as
float32 [B, H, Lq]; the kernel runs on torch's current stream.  A non-zero status
raises ``FaError`` (a RuntimeError) with ``fa_status_string``'s text.
"""

from __future__ import annotations

from . import FaError, fa_fwd

__all__ = ["fwd", "FaError"]


def fwd(q, k, v, *, causal: bool = False, scale: float | None = None):
    return fa_fwd(q, k, v, causal=causal, scale=scale)
