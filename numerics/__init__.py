"""CPU models of the kernels' rounding, and the error bounds the parity tests use.

TEST INFRASTRUCTURE ONLY, like ``oracle/``: the tests, ``bench.py``'s parity
check and nothing on the product path import it.  It shares no code with the HIP
kernels or their binding, and it does not import the oracle.

``emulate``: the forward and backward passes carried out in fp32 on the CPU with
every rounding the kernels make (fp32 scores, base-2 exponent with the scale
folded in, the lazily moved running max, weights rounded to the input type
before they multiply V, the two row sums, the rounded outputs).  It predicts the
size of the error the GPU must show against the fp64 oracle; it is not a second
oracle of the method (the oracle is the definition).

``bounds``: per-element and per-row error allowances that follow from those
roundings, used to state the parity bars.
"""

from .bounds import delta_bounds, fwd_allowance, half_ulp, round_to_dtype, unit_roundoff
from .emulate import bwd_emulate_head, fwd_emulate_head

__all__ = ["bwd_emulate_head", "delta_bounds", "fwd_allowance", "fwd_emulate_head", "half_ulp", "round_to_dtype",
           "unit_roundoff"]
