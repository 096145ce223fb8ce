"""CPU oracle for the fused attention forward pass — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports it, and the two share no code.

* ``attention_fp64``: the plain definition of softmax attention with the
  per-row log-sum-exp, fp64, numpy.
* ``streaming_attention_fp64``: the tiled streaming-softmax method in fp64, used
  to pin that the recurrence equals the definition.
* ``attention_bwd_fp64``: the exact gradients (dQ, dK, dV) of that definition
  for an upstream gradient of the output, fp64, numpy.
"""

from .attention import attention_fp64, attention_head_fp64
from .attention_bwd import attention_bwd_fp64, attention_bwd_head_fp64
from .streaming import streaming_attention_fp64

__all__ = ["attention_fp64", "attention_head_fp64", "streaming_attention_fp64", "attention_bwd_fp64",
           "attention_bwd_head_fp64"]
