"""fa_fwd_splitkv_noalloc (through the C ABI) against fa_fwd_splitkv and the fp64 oracle.

The allocation-free entry point runs the same kernels as fa_fwd_splitkv with the
partials in the library's own device array instead of a caller's workspace, so
its outputs must equal fa_fwd_splitkv's bit for bit, and both must meet the
parity bar against the oracle.  Two calls in a row, the second smaller, check
that what the first call leaves in the shared array does not leak into the
second.
"""

from __future__ import annotations

import pytest
import torch

import attn_inputs as ai
import tiled_attention_06_amd as fa
from oracle import attention_fp64

from test_parity import compare, note

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CALLS = [  # B, H, Lq, Lk, D, dtype, causal, splits (the second call is smaller than the first)
    (1, 8, 256, 4000, 128, "bf16", False, 8),
    (1, 2, 100, 1500, 64, "fp16", True, 3),
]


def _run(inp, splits, noalloc):
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
    if noalloc:
        fa.fa_fwd_splitkv_noalloc(q, k, v, o, lse, causal=inp["causal"], scale=inp["scale"], num_splits=splits)
    else:
        fa.fa_fwd_splitkv(q, k, v, o, lse, causal=inp["causal"], scale=inp["scale"], num_splits=splits)
    return o, lse


def test_noalloc_matches_workspace_call_twice():
    inputs = [ai.make_custom(B, H, Lq, Lk, D, dt, c, seed=180_000 + i) for i, (B, H, Lq, Lk, D, dt, c, _)
              in enumerate(CALLS)]
    # both no-alloc calls back to back on one stream, then the workspace calls
    got = []
    for inp, (B, H, Lq, Lk, D, dt, c, s) in zip(inputs, CALLS):
        note(f"noalloc B{B} H{H} Lq{Lq} Lk{Lk} D{D} {dt} causal={c} splits={s}")
        assert fa.fa_fwd_splitkv_workspace_size(B, H, Lq, D, s) <= fa.FA_NOALLOC_SCRATCH_BYTES
        got.append(_run(inp, s, True))
    want = [_run(inp, cfg[-1], False) for inp, cfg in zip(inputs, CALLS)]
    torch.cuda.synchronize()
    for (o1, l1), (o2, l2), inp, cfg in zip(got, want, inputs, CALLS):
        assert torch.equal(o1.cpu(), o2.cpu()) and torch.equal(l1.cpu(), l2.cpu()), f"differs from fa_fwd_splitkv {cfg}"
        O_ref, L_ref = attention_fp64(inp["q"], inp["k"], inp["v"], inp["scale"], inp["causal"])
        compare(o1, l1, O_ref, L_ref, cfg[5], f"noalloc {cfg}", src=inp)


def test_noalloc_rejects_partials_beyond_the_array():
    inp = ai.make_custom(1, 32, 256, 300, 128, "bf16", False, seed=180_010)
    assert fa.fa_fwd_splitkv_workspace_size(1, 32, 256, 128, 16) > fa.FA_NOALLOC_SCRATCH_BYTES
    with pytest.raises(fa.FaError) as e:
        _run(inp, 16, True)
    assert e.value.code == -12
