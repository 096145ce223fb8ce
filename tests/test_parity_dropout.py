"""GPU parity of dropout (fa_fwd_dropout, fa_bwd_dropout through the C ABI) against the fp64 oracle.

The keep bits are integer decisions on Philox4x32-10 bytes, taken identically by
the kernels and by oracle/philox.py: a single differing bit changes an output row
by O(1), far beyond the bars.  The bars are those of the dropout-free tests: the
forward's (2e-3 fp16 / 1e-2 bf16 per element, or, only where the output format is
coarser than that, its rounding plus the bound of the kernel's weight rounding,
numerics.fwd_allowance with the keep mask; LSE 1e-3) and the backward's (per slab,
relative to the slab's max and rms).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import attn_inputs as ai
import tiled_attention_06_amd as fa
from oracle import attention_bwd_fp64, attention_fp64

from test_parity import compare as compare_fwd, note
from test_parity_bwd import compare as compare_bwd

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = [  # B, H, Lq, Lk, D, dtype, causal, p, seed
    (1, 2, 300, 300, 128, "bf16", True, 0.1, 1234),
    (2, 3, 257, 400, 64, "fp16", False, 0.5, 2 ** 63 + 12345),
    (1, 2, 100, 1000, 128, "fp16", True, 0.3, 77),
    (1, 1, 1, 777, 64, "bf16", False, 0.9, 5),
    (1, 2, 520, 520, 64, "bf16", True, 0.25, 99),
    (2, 2, 333, 270, 128, "bf16", False, 0.2, 4242),
]
IDS = [f"B{b}H{h}_{lq}x{lk}_D{d}_{dt}_{'c' if c else 'nc'}_p{p}" for b, h, lq, lk, d, dt, c, p, _ in CASES]


@pytest.mark.parametrize("B,H,Lq,Lk,D,dtype,causal,p,seed", CASES, ids=IDS)
def test_dropout_forward(B, H, Lq, Lk, D, dtype, causal, p, seed):
    inp = ai.make_custom(B, H, Lq, Lk, D, dtype, causal, seed=110_000 + Lq + Lk)
    note(f"dropout fwd B{B} H{H} Lq{Lq} Lk{Lk} D{D} {dtype} causal={causal} p={p} seed={seed}")
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
    fa.fa_fwd_dropout(q, k, v, o, lse, causal=causal, scale=inp["scale"], dropout_p=p, seed=seed)
    _, lse0 = fa.fa_fwd(q, k, v, causal=causal, scale=inp["scale"])
    torch.cuda.synchronize()
    O_ref, L_ref = attention_fp64(inp["q"], inp["k"], inp["v"], inp["scale"], causal, dropout_p=p, seed=seed)
    compare_fwd(o, lse, O_ref, L_ref, dtype, "dropout fwd", src=dict(inp, dropout_p=p, seed=seed))
    assert torch.equal(lse.cpu(), lse0.cpu()), "LSE must not depend on dropout"


@pytest.mark.parametrize("D,dtype,causal,p", [(128, "bf16", True, 0.2), (64, "fp16", False, 0.6)])
def test_dropout_forward_wide_grids(D, dtype, causal, p):
    # The cases above run 128-row workgroups (grids of at most 256 items); 257 heads of 65
    # rows run the 256-row form, here with 1 to 8 key tiles so that its pipelined loop, its
    # last full tile and its masked tiles all take the dropout path.
    for Lk in (81, 145, 256, 337, 465, 512):
        seed = 3_000_000 + Lk + D
        inp = ai.make_custom(1, 257, 65, Lk, D, dtype, causal, seed=140_000 + Lk + D)
        note(f"dropout fwd wide H257 Lq65 Lk{Lk} D{D} {dtype} causal={causal} p={p} seed={seed}")
        q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
        o = torch.full_like(q, float("nan"))
        lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
        fa.fa_fwd_dropout(q, k, v, o, lse, causal=causal, scale=inp["scale"], dropout_p=p, seed=seed)
        torch.cuda.synchronize()
        heads = [(0, 0), (0, 130), (0, 256)]
        O_ref, L_ref = attention_fp64(inp["q"], inp["k"], inp["v"], inp["scale"], causal, heads=heads,
                                      dropout_p=p, seed=seed)
        compare_fwd(o.cpu(), lse.cpu(), O_ref, L_ref, dtype, f"dropout fwd wide Lk{Lk}",
                    src=dict(inp, dropout_p=p, seed=seed), heads=heads)


@pytest.mark.parametrize("B,H,Lq,Lk,D,dtype,causal,p,seed", CASES, ids=IDS)
def test_dropout_backward(B, H, Lq, Lk, D, dtype, causal, p, seed):
    inp = ai.make_custom(B, H, Lq, Lk, D, dtype, causal, seed=120_000 + Lq + Lk)
    do = ai.make_dout((B, H, Lq, D), dtype, seed=130_000 + Lq)
    note(f"dropout bwd B{B} H{H} Lq{Lq} Lk{Lk} D{D} {dtype} causal={causal} p={p} seed={seed}")
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    o, lse = fa.fa_fwd(q, k, v, causal=causal, scale=inp["scale"], dropout_p=p, seed=seed)
    dq, dk, dv = (torch.full_like(t, float("nan")) for t in (q, k, v))
    fa.fa_bwd(q, k, v, o, do.to(DEV), lse, dq, dk, dv, causal=causal, scale=inp["scale"], dropout_p=p, seed=seed)
    torch.cuda.synchronize()
    ref = attention_bwd_fp64(inp["q"], inp["k"], inp["v"], do, inp["scale"], causal, dropout_p=p, seed=seed)
    compare_bwd((dq.cpu(), dk.cpu(), dv.cpu()), ref, dtype, "dropout bwd")


def test_zero_probability_is_the_plain_call():
    inp = ai.make_custom(1, 2, 333, 333, 128, "bf16", True, seed=140_001)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    o1, l1 = fa.fa_fwd(q, k, v, causal=True)
    o2, l2 = fa.fa_fwd_dropout(q, k, v, causal=True, dropout_p=0.0, seed=123)
    torch.cuda.synchronize()
    assert torch.equal(o1.cpu(), o2.cpu()) and torch.equal(l1.cpu(), l2.cpu())


def test_flash_attention_dropout_autograd():
    inp = ai.make_custom(2, 2, 200, 200, 64, "fp16", True, seed=150_001)
    do = ai.make_dout((2, 2, 200, 64), "fp16", seed=150_002)
    q, k, v = (inp[n].to(DEV).requires_grad_(True) for n in ("q", "k", "v"))
    o = fa.flash_attention(q, k, v, causal=True, dropout_p=0.2, seed=4242)
    o.backward(do.to(DEV))
    torch.cuda.synchronize()
    O_ref, _ = attention_fp64(inp["q"], inp["k"], inp["v"], inp["scale"], True, dropout_p=0.2, seed=4242)
    err = np.abs(o.detach().double().cpu().numpy() - O_ref).max()
    note(f"  autograd dropout fwd max err {err:.3e}")
    assert err <= 2e-3
    ref = attention_bwd_fp64(inp["q"], inp["k"], inp["v"], do, inp["scale"], True, dropout_p=0.2, seed=4242)
    compare_bwd((q.grad.cpu(), k.grad.cpu(), v.grad.cpu()), ref, "fp16", "autograd dropout")


def test_keep_fraction_on_gpu():
    # V = one-hot columns per key block makes O count the kept weight mass; with uniform weights (q = 0)
    # the dropped-out output averages (256/T)·keep over the keys, whose mean is near 1.
    B, H, L, D = 1, 4, 1024, 64
    q = torch.zeros(B, H, L, D, dtype=torch.bfloat16, device=DEV)
    k = torch.randn(B, H, L, D, dtype=torch.bfloat16, device=DEV)
    v = torch.ones(B, H, L, D, dtype=torch.bfloat16, device=DEV)
    o, _ = fa.fa_fwd_dropout(q, k, v, dropout_p=0.5, seed=31337)
    torch.cuda.synchronize()
    m = o.float().mean().item()
    note(f"  mean of dropped-out ones: {m:.4f}")
    assert abs(m - 1.0) < 0.01


def test_dropout_train_shape_sampled():
    # the 7B 4K training shape with p = 0.1: forward rows and backward heads sampled against the oracle
    from test_parity import _sample

    w = ai.WORKLOADS["train7b_4k"]
    inp = ai.make_inputs(w)
    do = ai.make_dout((w.B, w.H, w.Lq, w.D), w.dtype, seed=w.seed + 100)
    p, seed = 0.1, 2024
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    o, lse = fa.fa_fwd_dropout(q, k, v, causal=True, scale=w.scale, dropout_p=p, seed=seed)
    dq, dk, dv = fa.fa_bwd(q, k, v, o, do.to(DEV), lse, causal=True, scale=w.scale, dropout_p=p, seed=seed)
    torch.cuda.synchronize()
    heads, rows = _sample(w, seed=11)
    O_ref, L_ref = attention_fp64(inp["q"], inp["k"], inp["v"], w.scale, True, rows=rows, heads=heads,
                                  dropout_p=p, seed=seed)
    compare_fwd(o.cpu()[:, :, rows], lse.cpu()[:, :, rows], O_ref, L_ref, w.dtype, "dropout train",
                src=dict(inp, dropout_p=p, seed=seed), heads=heads, rows=rows)
    bh = [(0, 0), (w.B - 1, w.H - 1)]
    ref = attention_bwd_fp64(inp["q"], inp["k"], inp["v"], do, w.scale, True, heads=bh, dropout_p=p, seed=seed)
    compare_bwd((dq.cpu(), dk.cpu(), dv.cpu()), ref, w.dtype, "dropout train bwd", heads=bh)


@pytest.mark.parametrize("p,seed", [(0.1, 7), (0.5, 2 ** 40 + 3), (0.9, 12345)])
def test_dropout_masks_bit_exact(p, seed):
    """Read each kernel's keep bits back exactly and compare them with oracle/philox.py bit for bit.

    With 128 keys, D = 128, q = 0 (uniform weights 1/128, exact), v = I and dO chosen per kernel:
      forward:  O[i, d]  > 0  iff key d is kept for row i;
      dK/dV:    dO = I  gives  dV[j, i] > 0  iff key j is kept for row i;
      dQ:       k = I, dO = 1 (so dP = 1) gives  dQ[i, d] > 0  iff key d is kept for row i
                (dS = P (M − Δ) with Δ ≈ 1 < 256/T for kept keys, −P Δ < 0 for dropped ones).
    """
    from oracle.philox import dropout_keep

    B, H, L, D = 1, 3, 128, 128
    dt = torch.bfloat16
    eye = torch.eye(L, dtype=dt, device=DEV).expand(B, H, L, D).contiguous()
    q = torch.zeros(B, H, L, D, dtype=dt, device=DEV)
    k = torch.randn(B, H, L, D, dtype=dt, device=DEV)
    o, lse = fa.fa_fwd_dropout(q, k, eye, dropout_p=p, seed=seed)
    ones = torch.ones(B, H, L, D, dtype=dt, device=DEV)
    _, _, dv = fa.fa_bwd(q, k, eye, o, eye, lse, dropout_p=p, seed=seed)
    o2, lse2 = fa.fa_fwd_dropout(q, eye, eye, dropout_p=p, seed=seed)
    dq, _, _ = fa.fa_bwd(q, eye, eye, o2, ones, lse2, dropout_p=p, seed=seed)
    torch.cuda.synchronize()
    for h in range(H):
        want = dropout_keep(h, np.arange(L), np.arange(L), p, seed)        # [row, key]
        got_fwd = (o[0, h].float().cpu().numpy() > 0)
        got_dkdv = (dv[0, h].float().cpu().numpy() > 0).T
        got_dq = (dq[0, h].float().cpu().numpy() > 0)
        note(f"  head {h}: keep fraction {want.mean():.3f}")
        assert np.array_equal(got_fwd, want), f"forward mask differs in {np.sum(got_fwd != want)} places"
        assert np.array_equal(got_dkdv, want), f"dK/dV mask differs in {np.sum(got_dkdv != want)} places"
        assert np.array_equal(got_dq, want), f"dQ mask differs in {np.sum(got_dq != want)} places"
