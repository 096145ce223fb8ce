"""The rounding models (numerics/) that set the parity bars: pinned to the oracle and to exact arithmetic.

CPU only.  Pages cited (title, then the section on that page):
  [DF] "FlashAttention数据流优化：MI50显存与带宽瓶颈实战"  (kwkr.cn/news/544806)
  [OP] "FlashAttention优化原理与工程实践"                (lbrq.cn/news/50349)

* With its roundings switched off the forward model is the streaming update of
  [DF §2.2] in fp64 and must reproduce the definition (the oracle); the backward
  model must reproduce the fp64 gradient oracle.
* The 16-bit rounding helpers agree with torch's conversions and with hand values.
* With its roundings on, the model reproduces the error budget behind the
  choices of which row sum divides O and which enters LSE: at the 7B 4K training
  shape (bf16, causal, D = 128), rows 0..31 of every head, seeds 7, 11, 12345
  the output-rounding floor is 7.7e-3..7.8e-3, O divided by the sum of the
  rounded weights stays within 9.1e-3 (under the 1e-2 bar) while O divided by
  the fp32 sum reaches 1.1e-2 on one seed, and LSE from the fp32 sum is within
  5e-7 while LSE from the rounded sum exceeds the 1e-3 bar on every seed.
* The allowance of the forward bar covers the model's own error, and the
  backward bars sit above the model's gradients' errors.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import attn_inputs as ai
from numerics import bwd_emulate_head, fwd_allowance, fwd_emulate_head, half_ulp, round_to_dtype, unit_roundoff
from numerics.bounds import fwd_check
from oracle import attention_bwd_fp64, attention_head_fp64

TOL = {"fp16": 2e-3, "bf16": 1e-2}


def _head(inp, b=0, h=0):
    return tuple(inp[n][b, h].double().numpy() for n in ("q", "k", "v"))


# ------------------------------------------------------------------------------------------
# rounding helpers
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_round_to_dtype_matches_torch(dtype):
    r = np.random.default_rng(3)
    x32 = np.concatenate([r.standard_normal(20000) * s for s in (1e-3, 0.3, 1.0, 7.0, 300.0)]).astype(np.float32)
    tdt = torch.float16 if dtype == "fp16" else torch.bfloat16
    want = torch.from_numpy(x32).to(tdt).double().numpy()
    got = round_to_dtype(x32.astype(np.float64), dtype)
    assert np.array_equal(got, want)


def test_half_ulp_hand_values():
    # bf16 keeps 8 significant bits, fp16 11: half the spacing at [1,2) is 2^-8 and 2^-11
    assert half_ulp(1.0, "bf16") == 2.0 ** -8 and half_ulp(1.999, "bf16") == 2.0 ** -8
    assert half_ulp(3.0, "bf16") == 2.0 ** -7 and half_ulp(-4.0, "bf16") == 2.0 ** -6
    assert half_ulp(4.0, "fp16") == 2.0 ** -9 and half_ulp(8.0, "fp16") == 2.0 ** -8
    assert half_ulp(2.0 ** -20, "fp16") == 2.0 ** -25  # subnormal spacing 2^-24
    assert unit_roundoff("bf16") == 2.0 ** -8 and unit_roundoff("fp16") == 2.0 ** -11
    # where the format is coarser than the bar: bf16 from |x| = 4, fp16 from |x| = 8
    assert half_ulp(3.99, "bf16") < TOL["bf16"] < half_ulp(4.0, "bf16")
    assert half_ulp(7.99, "fp16") < TOL["fp16"] < half_ulp(8.0, "fp16")
    x = np.random.default_rng(4).standard_normal(10000) * 5
    for dt in ("fp16", "bf16"):
        assert (np.abs(round_to_dtype(x, dt) - x) <= half_ulp(x, dt)).all()


# ------------------------------------------------------------------------------------------
# exact mode = the definition
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("Lq,Lk,D,causal,scale", [(200, 200, 64, True, None), (150, 333, 128, False, None),
                                                   (70, 300, 64, True, None), (129, 129, 128, True, -0.3),
                                                   (65, 65, 64, False, 0.0), (100, 100, 128, False, 2.5)])
def test_forward_model_exact_mode_is_the_definition(Lq, Lk, D, causal, scale):
    inp = ai.make_custom(1, 1, Lq, Lk, D, "bf16", causal, seed=90_000 + Lq + Lk)
    q, k, v = _head(inp)
    sc = inp["scale"] if scale is None else scale
    O, L = attention_head_fp64(q, k, v, sc, causal)
    e = fwd_emulate_head(q, k, v, sc, causal, "bf16", exact=True)
    assert np.abs(e["o"] - O).max() <= 1e-12
    assert np.abs(e["lse"] - L).max() <= 1e-12
    # and a small tile with a small slack: many rescales, same result
    e = fwd_emulate_head(q, k, v, sc, causal, "bf16", exact=True, bc=16, tau=0.5)
    assert np.abs(e["o"] - O).max() <= 1e-12


@pytest.mark.parametrize("Lq,Lk,D,causal", [(120, 120, 64, True), (90, 200, 128, False), (60, 150, 64, True)])
def test_backward_model_exact_mode_is_the_gradient(Lq, Lk, D, causal):
    inp = ai.make_custom(1, 1, Lq, Lk, D, "fp16", causal, seed=91_000 + Lq + Lk)
    do = ai.make_dout((1, 1, Lq, D), "fp16", seed=91_500 + Lq).double().numpy()
    q, k, v = _head(inp)
    O, L = attention_head_fp64(q, k, v, inp["scale"], causal)
    g = bwd_emulate_head(q, k, v, O, L, do[0, 0], inp["scale"], causal, "fp16", exact=True)
    ref = attention_bwd_fp64(inp["q"], inp["k"], inp["v"], do, inp["scale"], causal)
    for x, r in zip(g, ref):
        assert np.abs(x - r[0, 0]).max() <= 1e-10 * max(1.0, np.abs(r).max())


# ------------------------------------------------------------------------------------------
# the error budget (which row sum goes where)
# ------------------------------------------------------------------------------------------

def _budget(dtype, B, H, L, D, seed):
    inp = ai.make_custom(B, H, L, L, D, dtype, True, seed=seed)
    q, k, v = (inp[n].double().numpy() for n in ("q", "k", "v"))
    r = dict(floor=0.0, o_lr=0.0, o_lf=0.0, lse_lf=0.0, lse_lr=0.0)
    for b in range(B):
        for h in range(H):
            O, Lse = attention_head_fp64(q[b, h], k[b, h], v[b, h], inp["scale"], True)
            a = fwd_emulate_head(q[b, h], k[b, h], v[b, h], inp["scale"], True, dtype)
            f = fwd_emulate_head(q[b, h], k[b, h], v[b, h], inp["scale"], True, dtype, o_sum="l_f", lse_sum="l_r")
            r["floor"] = max(r["floor"], float(np.abs(round_to_dtype(O, dtype) - O).max()))
            r["o_lr"] = max(r["o_lr"], float(np.abs(a["o"] - O).max()))
            r["o_lf"] = max(r["o_lf"], float(np.abs(f["o"] - O).max()))
            r["lse_lf"] = max(r["lse_lf"], float(np.abs(a["lse"] - Lse).max()))
            r["lse_lr"] = max(r["lse_lr"], float(np.abs(f["lse"] - Lse).max()))
    return r


def test_error_budget_bf16_train_shape():
    # rows 0..31 of all 128 heads of the 4x32 head grid, D = 128, bf16, causal: a row sees only
    # keys 0..i, so a 32-key draw per head is the same sample as the first rows of a longer one
    res = {s: _budget("bf16", 4, 32, 32, 128, s) for s in (7, 11, 12345)}
    for s, r in res.items():
        assert 7.4e-3 <= r["floor"] <= 2.0 ** -7, (s, r)          # bf16 half-ulp on [2, 4)
        assert r["o_lr"] <= 9.5e-3 < TOL["bf16"], (s, r)           # l_r for O: under the bar
        assert r["lse_lf"] <= 1e-6, (s, r)                         # l_f for LSE: far under 1e-3
        assert r["lse_lr"] > 1e-3, (s, r)                          # l_r for LSE would break the LSE bar
    assert max(r["o_lf"] for r in res.values()) > TOL["bf16"]      # l_f for O breaks the O bar on one seed


def test_error_budget_fp16_llama_shape():
    r = _budget("fp16", 1, 32, 64, 128, 7)
    assert 9e-4 <= r["floor"] <= 2.0 ** -10
    assert r["o_lr"] <= 1.1e-3 < TOL["fp16"]
    assert r["lse_lf"] <= 1e-6 and r["lse_lr"] < 1e-3


# ------------------------------------------------------------------------------------------
# the forward bar's allowance covers the modelled kernel
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,L,D,causal,sq,sv", [("bf16", 300, 128, True, 1.0, 1.0), ("fp16", 300, 64, True, 1.0, 1.0),
                                                    ("bf16", 400, 64, False, 6.0, 1.0), ("bf16", 400, 64, False, 6.0, 3.0),
                                                    ("fp16", 200, 128, False, 6.0, 4.0), ("bf16", 256, 128, True, 3.0, 2.5)])
def test_allowance_covers_the_model(dtype, L, D, causal, sq, sv):
    inp = ai.make_custom(1, 2, L, L, D, dtype, causal, seed=92_000 + L + D, sigma_q=sq, sigma_v=sv)
    for h in range(2):
        q, k, v = _head(inp, 0, h)
        O, _ = attention_head_fp64(q, k, v, inp["scale"], causal)
        e = fwd_emulate_head(q, k, v, inp["scale"], causal, dtype)
        E = fwd_allowance(q, k, v, O, inp["scale"], causal, dtype, np.arange(L))
        assert (np.abs(e["o32"] - O) <= E).all()                   # the unrounded model within E
        if sv == 1.0:
            # and, for unit-variance values (every workload's), the stored model within the bar.  With
            # V ~ N(0, 9) outputs in [2, 4) carry a bf16 rounding floor of 7.8e-3 plus a weight-rounding
            # error proportional to V's spread, and the plain 1e-2 is out of reach for any kernel that
            # feeds bf16 weights to the matrix cores
            ok, info = fwd_check(e["o"], O, dtype, TOL[dtype],
                                 lambda rows: fwd_allowance(q, k, v, O[rows], inp["scale"], causal, dtype, rows))
            assert ok, info


def test_bar_grants_the_allowance_only_where_the_format_is_coarse():
    # one head with V large enough that some outputs reach 4..8 (bf16 half-ulp 0.0156 > 1e-2)
    inp = ai.make_custom(1, 1, 64, 64, 64, "bf16", True, seed=93_001, sigma_v=4.0)
    q, k, v = _head(inp)
    O, _ = attention_head_fp64(q, k, v, inp["scale"], True)
    allow = lambda rows: fwd_allowance(q, k, v, O[rows], inp["scale"], True, "bf16", rows)
    big = np.argwhere((np.abs(O) >= 4.2) & (np.abs(O) < 7.5))
    small = np.argwhere((np.abs(O) > 0.5) & (np.abs(O) < 3.5))
    assert len(big) and len(small)
    o = O.copy()
    i = tuple(big[0])
    o[i] += 0.012 * np.sign(O[i])                                  # within half-ulp(4..8) but over tol
    ok, info = fwd_check(o, O, "bf16", 1e-2, allow)
    assert ok and info["n_allowed"] == 1, info
    o = O.copy()
    j = tuple(small[0])
    o[j] += 0.011                                                  # over tol where bf16 is fine enough
    ok, info = fwd_check(o, O, "bf16", 1e-2, allow)
    assert not ok and info["worst"]["row"] == j[0], info
    o = O.copy()
    o[i] += 0.05 * np.sign(O[i])                                   # beyond even the allowance
    assert not fwd_check(o, O, "bf16", 1e-2, allow)[0]


# ------------------------------------------------------------------------------------------
# the backward bars against the modelled kernels
# ------------------------------------------------------------------------------------------

BWD_TOL = {"fp16": (2e-3, 8e-4), "bf16": (1e-2, 6e-3)}   # max err / max|ref|, rms err / rms(ref)


def test_backward_bars_cover_the_model():
    worst = {dt: [0.0, 0.0] for dt in BWD_TOL}
    for dtype in ("bf16", "fp16"):
        for L, D, causal in ((300, 128, True), (300, 64, False), (1024, 128, True), (513, 64, True)):
            inp = ai.make_custom(1, 2, L, L, D, dtype, causal, seed=50_000 + L + D)
            do = ai.make_dout((1, 2, L, D), dtype, seed=60_000 + L).double().numpy()
            ref = attention_bwd_fp64(inp["q"], inp["k"], inp["v"], do, inp["scale"], causal)
            for h in range(2):
                q, k, v = _head(inp, 0, h)
                f = fwd_emulate_head(q, k, v, inp["scale"], causal, dtype)
                g = bwd_emulate_head(q, k, v, f["o"], f["lse"], do[0, h], inp["scale"], causal, dtype)
                for x, r in zip(g, ref):
                    rr = r[0, h]
                    e = np.abs(x - rr)
                    worst[dtype][0] = max(worst[dtype][0], e.max() / np.abs(rr).max())
                    worst[dtype][1] = max(worst[dtype][1], math.sqrt((e ** 2).mean() / (rr ** 2).mean()))
    for dt, (mx, rms) in worst.items():
        # the modelled kernels' errors, and a margin of at least 1.5x below each bar
        assert mx * 1.5 <= BWD_TOL[dt][0] and rms * 1.5 <= BWD_TOL[dt][1], (dt, mx, rms)
    assert worst["bf16"][0] > 3e-3 and worst["fp16"][0] > 3e-4    # the bars are not vacuous either
