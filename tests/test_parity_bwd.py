"""GPU parity of the backward pass (fa_bwd through the C ABI) against the fp64 gradient oracle.

The GPU backward takes o and lse from the GPU forward pass on the same rounded
q, k, v; the oracle differentiates the definition in fp64 from q, k, v and dO
alone.  Bar, per (batch, head) slab and per gradient g ∈ {dq, dk, dv}:

    max |g_gpu − g_ref| ≤ TOL · max |g_ref|    and    rms(g_gpu − g_ref) ≤ TOL_RMS · rms(g_ref)

with TOL = 1e-2 (bf16) / 2e-3 (fp16) and TOL_RMS = 6e-3 / 8e-4, plus an absolute
1e-5 for slabs whose exact gradient is 0 (one visible key: the kernel's dP − Δ is
then an fp32 rounding residue, ~1e-7 at unit-scale inputs).  Derivation: the
kernels round P and dS to the input type as matrix-core operands and round the
outputs; the CPU model of exactly those roundings in fp32 (numerics.emulate, with
O and LSE from the modelled forward pass) gives at most 5.5e-3 / 1.2e-3 of the
slab's max and 3.1e-3 / 4.0e-4 of its rms, at L = 300..1024, D = 64 and 128,
causal and not (tests/test_numerics.py).  The bars are 1.7–2.0x those.
Outputs are pre-filled with NaN so that an unwritten element fails.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import attn_inputs as ai
import tiled_attention_06_amd as fa
from oracle import attention_bwd_fp64

pytestmark = pytest.mark.gpu

TOL = {"fp16": 2e-3, "bf16": 1e-2}
TOL_RMS = {"fp16": 8e-4, "bf16": 6e-3}
ABS = 1e-5
DEV = "cuda:0"


def note(msg: str):
    print(msg, flush=True)


def run_bwd(inp, do, causal, scale=None, fwd=None):
    """Gradients through fa_bwd; ``fwd``: (o, lse) to use instead of running fa_fwd here."""
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    dod = do.to(DEV)
    o, lse = fa.fa_fwd(q, k, v, causal=causal, scale=scale) if fwd is None else (x.to(DEV) for x in fwd)
    dq, dk, dv = (torch.full_like(t, float("nan")) for t in (q, k, v))
    fa.fa_bwd(q, k, v, o, dod, lse, dq, dk, dv, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def compare(got, ref, dtype, what, heads=None, extra=None):
    """extra: optional {(b, h): (dq row bounds, dk row bounds)} added to the bars (numerics.delta_bounds)."""
    names = ("dq", "dk", "dv")
    for t, (name, g, r) in enumerate(zip(names, got, ref)):
        g = g.double().numpy()
        pairs = heads if heads is not None else [(b, h) for b in range(g.shape[0]) for h in range(g.shape[1])]
        for b, h in pairs:
            gs, rs = g[b, h], r[b, h]
            assert np.isfinite(gs).all(), f"{what} {name} ({b},{h}): non-finite (unwritten?)"
            err = np.abs(gs - rs)
            if extra is not None and t < 2:
                err = np.maximum(err - extra[(b, h)][t], 0.0)  # what the rounding of O does not explain
            mx, rms = np.abs(rs).max(), np.sqrt((rs ** 2).mean())
            e_max, e_rms = err.max(), np.sqrt((err ** 2).mean())
            note(f"  {what} {name} ({b},{h}): max err {e_max:.3e} (max |ref| {mx:.3e}), rms err {e_rms:.3e} "
                 f"(rms ref {rms:.3e})")
            assert e_max <= TOL[dtype] * mx + ABS, f"{what} {name} ({b},{h}): max err {e_max} > {TOL[dtype]} * {mx}"
            assert e_rms <= TOL_RMS[dtype] * rms + ABS, f"{what} {name} ({b},{h}): rms err {e_rms} > {TOL_RMS[dtype]} * {rms}"


CASES = [  # B, H, Lq, Lk, D, dtype, causal
    (1, 2, 64, 64, 64, "bf16", False), (1, 2, 300, 300, 128, "bf16", True), (2, 3, 257, 257, 64, "fp16", True),
    (1, 2, 100, 1000, 128, "fp16", True), (1, 2, 1000, 100, 64, "bf16", False), (1, 1, 1, 1, 128, "bf16", False),
    (1, 1, 1, 1, 64, "fp16", True), (1, 2, 129, 65, 128, "fp16", False), (1, 1, 513, 513, 128, "bf16", True),
    (1, 2, 200, 333, 64, "bf16", True), (1, 1, 640, 640, 128, "fp16", False),
    (2, 2, 200, 333, 128, "bf16", True), (1, 3, 70, 130, 128, "fp16", True),
]


@pytest.mark.parametrize("B,H,Lq,Lk,D,dtype,causal", CASES,
                         ids=[f"B{b}H{h}_{lq}x{lk}_D{d}_{dt}_{'c' if c else 'nc'}" for b, h, lq, lk, d, dt, c in CASES])
def test_bwd_matches_oracle(B, H, Lq, Lk, D, dtype, causal):
    inp = ai.make_custom(B, H, Lq, Lk, D, dtype, causal, seed=50_000 + Lq + 3 * Lk + D)
    do = ai.make_dout((B, H, Lq, D), dtype, seed=60_000 + Lq + Lk)
    note(f"bwd B{B} H{H} Lq{Lq} Lk{Lk} D{D} {dtype} causal={causal}")
    got = run_bwd(inp, do, causal)
    ref = attention_bwd_fp64(inp["q"], inp["k"], inp["v"], do, inp["scale"], causal)
    compare(got, ref, dtype, "bwd")


@pytest.mark.parametrize("scale", [0.0, -0.2, 0.35])
def test_bwd_scale_values(scale):
    inp = ai.make_custom(1, 2, 200, 260, 64, "bf16", True, seed=70_001)
    do = ai.make_dout((1, 2, 200, 64), "bf16", seed=70_002)
    note(f"bwd scale {scale}")
    got = run_bwd(inp, do, True, scale=scale)
    ref = attention_bwd_fp64(inp["q"], inp["k"], inp["v"], do, scale, True)
    if scale == 0.0:
        assert float(got[0].abs().max()) == 0.0 and float(got[1].abs().max()) == 0.0  # dq = dk = 0 exactly
        g, r = got[2].double().numpy(), ref[2]
        assert np.abs(g - r).max() <= TOL["bf16"] * np.abs(r).max()
    else:
        compare(got, ref, "bf16", f"bwd scale {scale}")


def test_bwd_sum_rules_at_train_shape():
    # 7B 4K training shape: every row of P sums to one (Σ_j dV_j = Σ_i dO_i) and the key-shift
    # invariance (Σ_j dK_j = 0) hold on every head; two heads against the oracle in full
    w = ai.WORKLOADS["train7b_4k"]
    inp = ai.make_inputs(w)
    do = ai.make_dout((w.B, w.H, w.Lq, w.D), w.dtype, seed=80_003)
    note("bwd train7b_4k: GPU")
    got = run_bwd(inp, do, True)
    dv_sum = got[2].double().sum(dim=2)
    do_sum = do.double().sum(dim=2)
    rel = ((dv_sum - do_sum).abs().max() / do_sum.abs().max()).item()
    note(f"  sum rule dV: {rel:.2e}")
    assert rel <= 1e-2
    dk_sum = got[1].double().sum(dim=2).abs().max().item()
    dk_scale = got[1].double().abs().sum(dim=2).max().item()
    note(f"  sum rule dK: {dk_sum:.3e} of {dk_scale:.3e}")
    assert dk_sum <= 1e-2 * dk_scale
    heads = [(0, 0), (3, 31)]
    note("bwd train7b_4k: oracle on two heads")
    ref = attention_bwd_fp64(inp["q"], inp["k"], inp["v"], do, w.scale, True, heads=heads)
    compare(got, ref, w.dtype, "bwd train7b_4k", heads=heads)


def test_bwd_peaked_softmax():
    # the numerics-stress recipe (Q ~ N(0, 3²) boosted so one key per row leads by 20 logits) at L = 1024:
    # dQ and dK are then ~1e-7, of the order of what rounding the stored O moves Δ by (numerics.delta_bounds)
    import dataclasses

    from numerics import delta_bounds
    from oracle import attention_fp64

    w = dataclasses.replace(ai.WORKLOADS["stress_8k"], B=1, H=2, Lq=1024, Lk=1024)
    inp = ai.make_inputs(w)
    do = ai.make_dout((1, 2, 1024, 64), "bf16", seed=95_001)
    note("bwd peaked softmax (stress recipe, L=1024)")
    got = run_bwd(inp, do, False)
    ref = attention_bwd_fp64(inp["q"], inp["k"], inp["v"], do, w.scale, False)
    O_ref, L_ref = attention_fp64(inp["q"], inp["k"], inp["v"], w.scale, False)
    extra = delta_bounds(inp["q"], inp["k"], do, O_ref, L_ref, w.scale, False, "bf16", [(0, 0), (0, 1)])
    compare(got, ref, "bf16", "bwd peaked", extra=extra)


@pytest.mark.parametrize("name", ["llama7b_2k", "stress_8k", "long_16k"])
def test_bwd_workload_sampled(name):
    # the other workloads at full size: every head on the GPU, one or two heads in full against the oracle
    from numerics import delta_bounds
    from oracle import attention_fp64

    w = ai.WORKLOADS[name]
    inp = ai.make_inputs(w)
    do = ai.make_dout((w.B, w.H, w.Lq, w.D), w.dtype, seed=w.seed + 100)
    note(f"bwd {name}: GPU")
    got = run_bwd(inp, do, w.causal)
    heads = [(w.B - 1, w.H - 1)] if name == "long_16k" else [(0, 0), (w.B - 1, w.H - 1)]
    note(f"bwd {name}: oracle on {heads}")
    ref = attention_bwd_fp64(inp["q"], inp["k"], inp["v"], do, w.scale, w.causal, heads=heads)
    O_ref, L_ref = attention_fp64(inp["q"], inp["k"], inp["v"], w.scale, w.causal, heads=heads)
    extra = delta_bounds(inp["q"], inp["k"], do, O_ref, L_ref, w.scale, w.causal, w.dtype, heads)
    compare(got, ref, w.dtype, f"bwd {name}", heads=heads, extra=extra)


@pytest.mark.parametrize("D,dtype,causal", [(64, "fp16", True), (128, "bf16", False)])
def test_bwd_wide_grid_and_geometry(D, dtype, causal):
    # 300 heads of 300 rows: 600 dQ workgroups (ragged tails), checked on three heads against the oracle;
    # the first 4 heads alone (a grid smaller than the CU count), given the same forward outputs, must
    # give bit-identical gradients (the forward itself runs another form for 4 heads)
    inp = ai.make_custom(1, 300, 300, 300, D, dtype, causal, seed=95_000 + D)
    do = ai.make_dout((1, 300, 300, D), dtype, seed=95_100 + D)
    note(f"bwd wide B1 H300 300x300 D{D} {dtype} causal={causal}")
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    o, lse = fa.fa_fwd(q, k, v, causal=causal)
    got = run_bwd(inp, do, causal, fwd=(o, lse))
    heads = [(0, 0), (0, 150), (0, 299)]
    ref = attention_bwd_fp64(inp["q"], inp["k"], inp["v"], do, inp["scale"], causal, heads=heads)
    compare(got, ref, dtype, "bwd wide", heads=heads)
    few = {n: inp[n][:, :4].contiguous() for n in ("q", "k", "v")}
    got4 = run_bwd({**inp, **few}, do[:, :4].contiguous(), causal,
                   fwd=(o[:, :4].contiguous(), lse[:, :4].contiguous()))
    for name, x, y in zip(("dq", "dk", "dv"), got, got4):
        assert torch.equal(x[:, :4], y), f"{name} of the first 4 heads depends on the grid"


def test_bwd_deterministic():
    inp = ai.make_custom(1, 4, 700, 700, 128, "bf16", True, seed=90_001)
    do = ai.make_dout((1, 4, 700, 128), "bf16", seed=90_002)
    a = run_bwd(inp, do, True)
    b = run_bwd(inp, do, True)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("dropout_p", [0.0, 0.2])
def test_bwd_deterministic_many_workgroups(dropout_p):
    # a grid of 16 heads x 12 key blocks per head, three calls: the weights that the dK/dV kernel's waves pass
    # to each other through LDS, and every other exchange, must give the same bits each time
    inp = ai.make_custom(2, 8, 1500, 1500, 128, "bf16", True, seed=90_011)
    do = ai.make_dout((2, 8, 1500, 128), "bf16", seed=90_012).to(DEV)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    o, lse = fa.fa_fwd(q, k, v, causal=True, dropout_p=dropout_p, seed=77)
    runs = []
    for _ in range(3):
        g = [torch.full_like(t, float("nan")) for t in (q, k, v)]
        fa.fa_bwd(q, k, v, o, do, lse, *g, causal=True, dropout_p=dropout_p, seed=77)
        torch.cuda.synchronize()
        runs.append([x.cpu() for x in g])
    for r in runs[1:]:
        for x, y in zip(runs[0], r):
            assert torch.equal(x, y)


def test_flash_attention_autograd():
    inp = ai.make_custom(2, 2, 320, 320, 64, "fp16", True, seed=91_001)
    do = ai.make_dout((2, 2, 320, 64), "fp16", seed=91_002)
    q, k, v = (inp[n].to(DEV).requires_grad_(True) for n in ("q", "k", "v"))
    o = fa.flash_attention(q, k, v, causal=True)
    o.backward(do.to(DEV))
    torch.cuda.synchronize()
    got = (q.grad.cpu(), k.grad.cpu(), v.grad.cpu())
    ref = attention_bwd_fp64(inp["q"], inp["k"], inp["v"], do, inp["scale"], True)
    compare(got, ref, "fp16", "autograd")
    direct = run_bwd(inp, do, True)
    for x, y in zip(got, direct):
        assert torch.equal(x, y)


def _blhd(t):
    """A [B, H, L, D] view of [B, L, H, D] storage holding t's values."""
    return t.transpose(1, 2).contiguous().transpose(1, 2)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_strided_matches_dense_bitwise(causal):
    # q, k, v, o, dout and dq, dk, dv all as [B, L, H, D] views: the same bits as the dense call
    inp = ai.make_custom(2, 3, 300, 333, 128, "bf16", causal, seed=96_001)
    do = ai.make_dout((2, 3, 300, 128), "bf16", seed=96_002)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    dod = do.to(DEV)
    o, lse = fa.fa_fwd(q, k, v, causal=causal)
    ref = fa.fa_bwd(q, k, v, o, dod, lse, causal=causal)
    qs, ks, vs, os_, ds = (_blhd(t) for t in (q, k, v, o, dod))
    outs = [torch.full((t.shape[0], t.shape[2], t.shape[1], t.shape[3]), float("nan"), dtype=t.dtype,
                       device=DEV).transpose(1, 2) for t in (q, k, v)]
    got = fa.fa_bwd(qs, ks, vs, os_, ds, lse, *outs, causal=causal)
    torch.cuda.synchronize()
    assert not got[0].is_contiguous()
    for a, b in zip(ref, got):
        assert torch.equal(a.cpu(), b.cpu().contiguous())


def test_bwd_qkvpacked_in_place():
    # forward and backward on views of one packed qkv buffer [B, L, 3, H, D], gradients into a packed dqkv
    B, L, H, D = 2, 257, 4, 64
    inp = ai.make_custom(B, H, L, L, D, "fp16", True, seed=97_001)
    do = ai.make_dout((B, H, L, D), "fp16", seed=97_002)
    qkv = torch.stack([inp[n].transpose(1, 2) for n in ("q", "k", "v")], dim=2).contiguous().to(DEV)
    q, k, v = (qkv[:, :, j].transpose(1, 2) for j in range(3))
    o, lse = fa.fa_fwd(q, k, v, causal=True)
    dqkv = torch.full_like(qkv, float("nan"))
    dq, dk, dv = (dqkv[:, :, j].transpose(1, 2) for j in range(3))
    fa.fa_bwd(q, k, v, o, do.to(DEV), lse, dq, dk, dv, causal=True)
    torch.cuda.synchronize()
    ref = attention_bwd_fp64(inp["q"], inp["k"], inp["v"], do, inp["scale"], True)
    compare((dq.cpu().contiguous(), dk.cpu().contiguous(), dv.cpu().contiguous()), ref, "fp16", "bwd packed")


def test_flash_attention_on_blhd_views():
    # the autograd function on [B, L, H, D] tensors (as transposed views), no copies, with dropout
    B, L, H, D = 1, 300, 2, 128
    inp = ai.make_custom(B, H, L, L, D, "bf16", True, seed=98_001)
    do = ai.make_dout((B, H, L, D), "bf16", seed=98_002)
    leaves = [inp[n].transpose(1, 2).contiguous().to(DEV).requires_grad_(True) for n in ("q", "k", "v")]
    q, k, v = (t.transpose(1, 2) for t in leaves)
    o = fa.flash_attention(q, k, v, causal=True, dropout_p=0.15, seed=99)
    o.backward(do.to(DEV))
    torch.cuda.synchronize()
    from oracle import attention_fp64

    O_ref, _ = attention_fp64(inp["q"], inp["k"], inp["v"], inp["scale"], True, dropout_p=0.15, seed=99)
    assert np.abs(o.detach().double().cpu().numpy() - O_ref).max() <= TOL["bf16"]
    ref = attention_bwd_fp64(inp["q"], inp["k"], inp["v"], do, inp["scale"], True, dropout_p=0.15, seed=99)
    grads = tuple(t.grad.transpose(1, 2).cpu().contiguous() for t in leaves)
    compare(grads, ref, "bf16", "autograd views")
