"""Pins for the fp64 CPU gradient oracle: what the mathematics fixes, independent of its code.

Pages cited:
  [DF] "FlashAttention数据流优化：MI50显存与带宽瓶颈实战"  (kwkr.cn/news/544806)

[DF §2.2] (third layer) recomputes the score blocks in the backward pass; the
gradients themselves are those of the forward definition.  Each ``pin_*`` takes a
callable ``grad(q, k, v, do, scale, causal) -> (dQ, dK, dV)`` on [B, H, L, D]
arrays and raises AssertionError when the callable is wrong.  The pins run
against the oracle (they must hold) and against copies of the oracle with a
planted mistake (each copy must fail at least one pin).  The strongest pin is a
central finite difference of the forward oracle (itself pinned in
test_oracle.py), which shares nothing with the gradient formulas.
"""

from __future__ import annotations

import math
import os
import sys
import types

import numpy as np
import pytest

from oracle import attention_bwd_fp64, attention_fp64

HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE_SRC = os.path.join(os.path.dirname(HERE), "oracle", "attention_bwd.py")


def _inputs(seed, B=1, H=2, Lq=7, Lk=7, D=3):
    r = np.random.default_rng(seed)
    return (r.standard_normal((B, H, Lq, D)), r.standard_normal((B, H, Lk, D)),
            r.standard_normal((B, H, Lk, D)), r.standard_normal((B, H, Lq, D)))


SHAPES = [  # (Lq, Lk, D, causal)
    (7, 7, 3, False), (6, 6, 3, True), (4, 9, 2, True), (5, 3, 2, False), (1, 5, 2, True),
]


# --------------------------------------------------------------------------------------------
# pins
# --------------------------------------------------------------------------------------------

def pin_finite_differences(grad):
    """Central differences of f = sum(dO * O(q, k, v)) through the forward oracle, every element
    of q, k and v, agree with the gradients (truncation error O(h^2) ~ 1e-10)."""
    h = 1e-5
    for n, (Lq, Lk, D, causal) in enumerate(SHAPES):
        q, k, v, do = _inputs(100 + n, 1, 1, Lq, Lk, D)
        scale = 0.7

        def f(q_, k_, v_):
            O, _ = attention_fp64(q_, k_, v_, scale, causal)
            return float((O * do).sum())

        dQ, dK, dV = grad(q, k, v, do, scale, causal)
        for name, x, g in (("q", q, dQ), ("k", k, dK), ("v", v, dV)):
            num = np.empty_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
                args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
                num[idx] = (f(*args_p) - f(*args_m)) / (2 * h)
            np.testing.assert_allclose(g, num, rtol=0, atol=1e-7,
                                       err_msg=f"d{name}, shape {(Lq, Lk, D)}, causal={causal}")


def pin_finite_differences_dropout(grad):
    """With dropout (a fixed keep-mask for a given seed), central differences of the forward
    oracle agree with the gradients, every element of q, k and v."""
    h = 1e-5
    for n, (Lq, Lk, D, causal) in enumerate([(7, 7, 3, False), (5, 9, 2, True)]):
        q, k, v, do = _inputs(150 + n, 1, 2, Lq, Lk, D)
        scale, p, seed = 0.6, 0.3, 1234 + n

        def f(q_, k_, v_):
            O, _ = attention_fp64(q_, k_, v_, scale, causal, dropout_p=p, seed=seed)
            return float((O * do).sum())

        dQ, dK, dV = grad(q, k, v, do, scale, causal, dropout_p=p, seed=seed)
        for name, x, g in (("q", q, dQ), ("k", k, dK), ("v", v, dV)):
            num = np.empty_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
                args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
                num[idx] = (f(*args_p) - f(*args_m)) / (2 * h)
            np.testing.assert_allclose(g, num, rtol=0, atol=1e-7,
                                       err_msg=f"dropout d{name}, shape {(Lq, Lk, D)}, causal={causal}")


def pin_autograd(grad):
    """torch autograd through scaled_dot_product_attention on the CPU in float64 (with an explicit
    boolean mask for the bottom-right causal rule) gives the same gradients to 1e-12."""
    import torch

    for n, (Lq, Lk, D, causal) in enumerate(SHAPES + [(33, 40, 16, True), (40, 33, 16, False)]):
        q, k, v, do = _inputs(200 + n, 2, 2, Lq, Lk, D)
        scale = 1.0 / math.sqrt(D)
        tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
        mask = None
        if causal:
            mask = torch.arange(Lk)[None, :] <= torch.arange(Lq)[:, None] + (Lk - Lq)
        out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
        out.backward(torch.from_numpy(do))
        dQ, dK, dV = grad(q, k, v, do, scale, causal)
        np.testing.assert_allclose(dQ, tq.grad.numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(dK, tk.grad.numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(dV, tv.grad.numpy(), rtol=0, atol=1e-12)


def pin_sum_rules(grad):
    """Every row of P sums to one, so sum_j dV_j = sum_i dO_i; adding one vector to every key
    shifts each row's logits by a constant and leaves P unchanged, so sum_j dK_j = 0."""
    for n, (Lq, Lk, D, causal) in enumerate(SHAPES):
        q, k, v, do = _inputs(300 + n, 2, 3, Lq, Lk, D)
        _, dK, dV = grad(q, k, v, do, 0.9, causal)
        np.testing.assert_allclose(dV.sum(axis=2), do.sum(axis=2), rtol=0, atol=1e-12)
        np.testing.assert_allclose(dK.sum(axis=2), 0.0, rtol=0, atol=1e-12)


def pin_equal_keys(grad):
    """All keys equal: P is uniform over each row's visible keys, so dQ = 0 and
    dV_j = sum over the rows i that see key j of dO_i / |A_i|."""
    for Lq, Lk, D, causal in [(5, 5, 3, False), (5, 5, 3, True), (3, 6, 2, True)]:
        q, k, v, do = _inputs(400 + Lq + Lk, 1, 1, Lq, Lk, D)
        k[:] = k[:, :, :1, :]
        dQ, _, dV = grad(q, k, v, do, 1.3, causal)
        np.testing.assert_allclose(dQ, 0.0, rtol=0, atol=1e-12)
        off = Lk - Lq
        want = np.zeros_like(v)
        for i in range(Lq):
            n_vis = (i + off + 1) if causal else Lk
            want[0, 0, :n_vis] += do[0, 0, i] / n_vis
        np.testing.assert_allclose(dV, want, rtol=0, atol=1e-12)


def pin_closed_form(grad):
    """One query at q = 0 against two keys (D = 1): P = (1/2, 1/2), so dV = (g/2, g/2),
    dS = (g(v0 - v1)/4, -g(v0 - v1)/4), dQ = scale*g*(v0 - v1)*(k0 - k1)/4 and dK = 0."""
    k0, k1, v0, v1, g, scale = 0.5, -1.5, 2.0, -1.0, 3.0, 0.25
    q = np.zeros((1, 1, 1, 1))
    k = np.array([k0, k1]).reshape(1, 1, 2, 1)
    v = np.array([v0, v1]).reshape(1, 1, 2, 1)
    do = np.array([g]).reshape(1, 1, 1, 1)
    dQ, dK, dV = grad(q, k, v, do, scale, False)
    assert abs(dQ[0, 0, 0, 0] - scale * g * (v0 - v1) * (k0 - k1) / 4) < 1e-15
    np.testing.assert_allclose(dK.ravel(), [0.0, 0.0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(dV.ravel(), [g / 2, g / 2], rtol=0, atol=1e-15)


def pin_causal_edges(grad):
    """Causal, Lq = Lk: row 0 sees only key 0 (P = 1, so dQ_0 = 0) and the last key is seen only
    by the last row (dV_last = P_last,last * dO_last, with that P from the forward oracle's LSE)."""
    L, D, scale = 6, 3, 0.8
    q, k, v, do = _inputs(500, 1, 1, L, L, D)
    dQ, _, dV = grad(q, k, v, do, scale, True)
    np.testing.assert_allclose(dQ[0, 0, 0], 0.0, rtol=0, atol=1e-15)
    _, lse = attention_fp64(q, k, v, scale, True)
    p_last = math.exp(scale * float(q[0, 0, -1] @ k[0, 0, -1]) - lse[0, 0, -1])
    np.testing.assert_allclose(dV[0, 0, -1], p_last * do[0, 0, -1], rtol=0, atol=1e-13)


def pin_zero_upstream(grad):
    """dO = 0 gives zero gradients."""
    q, k, v, do = _inputs(600, 1, 2, 5, 5, 3)
    for g in grad(q, k, v, np.zeros_like(do), 0.5, True):
        assert np.all(g == 0)


PINS = [pin_finite_differences, pin_finite_differences_dropout, pin_autograd, pin_sum_rules, pin_equal_keys,
        pin_closed_form, pin_causal_edges, pin_zero_upstream]


def _oracle_grad(q, k, v, do, scale, causal, **kw):
    # rows in chunks of 4, so the pins also cover the accumulation of dK and dV over chunks
    return attention_bwd_fp64(q, k, v, do, scale, causal, chunk=4, **kw)


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin_holds_for_oracle(pin):
    pin(_oracle_grad)


# --------------------------------------------------------------------------------------------
# planted mistakes: each must be caught by at least one pin
# --------------------------------------------------------------------------------------------

MUTANTS = {
    "dropped_row_term": ("dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))", "dS = P * dP"),
    "row_term_sign": ("dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))",
                      "dS = P * (dP + (P * dP).sum(axis=1, keepdims=True))"),
    "row_term_unnormalised": ("(P * dP).sum(axis=1, keepdims=True)", "(E * dP).sum(axis=1, keepdims=True)"),
    "dq_without_scale": ("dQ[r] = scale * (dS @ k)", "dQ[r] = dS @ k"),
    "dk_without_scale": ("dK += scale * (dS.T @ q[r])", "dK += dS.T @ q[r]"),
    "dq_from_values": ("dQ[r] = scale * (dS @ k)", "dQ[r] = scale * (dS @ v)"),
    "dk_from_upstream": ("dK += scale * (dS.T @ q[r])", "dK += scale * (dS.T @ do[r])"),
    "dp_from_keys": ("dP = do[r] @ v.T", "dP = do[r] @ k.T"),
    "dv_unnormalised": ("dV += Pd.T @ do[r]", "dV += E.T @ do[r]"),
    "softmax_unnormalised": ("P = E / E.sum(axis=1, keepdims=True)", "P = E"),
    "no_causal_mask": ("S[np.arange(Lk)[None, :] > r[:, None] + off] = -np.inf", "pass"),
    "mask_top_left": ("> r[:, None] + off] = -np.inf", "> r[:, None]] = -np.inf"),
    "mask_excludes_diagonal": ("> r[:, None] + off] = -np.inf", ">= r[:, None] + off] = -np.inf"),
    "dk_overwritten_per_chunk": ("dK += scale * (dS.T @ q[r])", "dK = scale * (dS.T @ q[r])"),
    "dv_overwritten_per_chunk": ("dV += Pd.T @ do[r]", "dV = Pd.T @ do[r]"),
    "dropout_missing_in_dp": ("            dP = dP * M", "            pass"),
    "dropout_missing_in_dv": ("Pd = P if M is None else P * M", "Pd = P"),
    "dropout_unscaled": ("* (256.0 / keep_threshold(dropout_p))", ""),
    "scale_missing_in_scores": ("S = (q[r] @ k.T) * scale", "S = q[r] @ k.T"),
}


def _load_mutant(name):
    old, new = MUTANTS[name]
    with open(ORACLE_SRC, encoding="utf-8") as f:
        src = f.read()
    assert old in src, f"mutation anchor for {name} not found in the oracle"
    src = src.replace(old, new, 1)
    mod = types.ModuleType(f"oracle.oracle_bwd_mutant_{name}")
    mod.__dict__["__name__"] = mod.__name__
    mod.__dict__["__package__"] = "oracle"  # the oracle's relative imports resolve in its package
    sys.modules[mod.__name__] = mod
    exec(compile(src, ORACLE_SRC + f"<{name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    mod = _load_mutant(name)

    def grad(q, k, v, do, scale, causal, **kw):
        return mod.attention_bwd_fp64(q, k, v, do, scale, causal, chunk=4, **kw)

    failures = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(grad)
        except Exception as e:  # AssertionError, or a shape error the mistake causes
            failures.append((pin.__name__, type(e).__name__))
    assert failures, f"no pin catches the planted mistake {name!r}"


def test_heads_subset_matches_full():
    q, k, v, do = _inputs(700, 2, 3, 9, 11, 4)
    full = attention_bwd_fp64(q, k, v, do, 0.5, True)
    part = attention_bwd_fp64(q, k, v, do, 0.5, True, heads=[(1, 2), (0, 1)])
    for a, b in zip(full, part):
        np.testing.assert_array_equal(a[1, 2], b[1, 2])
        np.testing.assert_array_equal(a[0, 1], b[0, 1])
        assert np.isnan(b[0, 0]).all()


def test_causal_with_more_queries_than_keys_is_rejected():
    q, k, v, do = _inputs(701, 1, 1, 5, 4, 2)
    with pytest.raises(ValueError):
        attention_bwd_fp64(q, k, v, do, 0.5, True)
