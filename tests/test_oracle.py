"""Pins for the fp64 CPU oracle: what the pages and the mathematics fix, independent of the oracle's code.

Pages cited:
  [DF] "FlashAttention数据流优化：MI50显存与带宽瓶颈实战"  (kwkr.cn/news/544806)
  [OP] "FlashAttention优化原理与工程实践"                (lbrq.cn/news/50349)

Each ``pin_*`` takes an attention callable ``attn(q, k, v, scale, causal) -> (O, LSE)``
on [B, H, L, D] arrays and raises AssertionError when the callable is wrong.  The
pins run against the oracle (they must hold) and against copies of the oracle with
a planted mistake (each copy must fail at least one pin), which is how the set is
shown to catch a dropped term, a wrong sign, an off-by-one mask, a transposed
operand or a wrong normaliser.
"""

from __future__ import annotations

import json
import math
import os
import sys
import types

import numpy as np
import pytest

from oracle import attention_fp64, attention_head_fp64, streaming_attention_fp64

HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE_SRC = os.path.join(os.path.dirname(HERE), "oracle", "attention.py")


def _rng(seed):
    return np.random.default_rng(seed)


def _qkv(seed, B=1, H=2, Lq=9, Lk=9, D=4, sq=1.0, sk=1.0, sv=1.0):
    r = _rng(seed)
    return (r.standard_normal((B, H, Lq, D)) * sq, r.standard_normal((B, H, Lk, D)) * sk,
            r.standard_normal((B, H, Lk, D)) * sv)


def _allowed(i, Lk, causal):
    return range(0, i + 1) if causal else range(Lk)


# --------------------------------------------------------------------------------------------
# pins
# --------------------------------------------------------------------------------------------

def pin_golden(attn):
    """Hand-derived rational cases ([DF §2.1] stages, [OP §2.1] naive form, [DF §4.1] causal)."""
    with open(os.path.join(HERE, "golden", "hand_derived.json"), encoding="utf-8") as f:
        cases = json.load(f)["cases"]
    logs = {"ln2": math.log(2.0), "ln3": math.log(3.0), "ln5": math.log(5.0)}
    for c in cases:
        q = np.array(c["q"], dtype=np.float64)[None, None]
        k = np.array(c["k"], dtype=np.float64)[None, None]
        v = np.array(c["v"], dtype=np.float64)[None, None]
        O, LSE = attn(q, k, v, logs[c["scale"]], c["causal"])
        np.testing.assert_allclose(O[0, 0], np.array(c["o"]), rtol=1e-13, atol=1e-13, err_msg=c["name"])
        np.testing.assert_allclose(np.exp(LSE[0, 0]), np.array(c["exp_lse"]), rtol=1e-13, err_msg=c["name"])


def pin_brute_force(attn):
    """Scalar loops with exact summation (math.fsum) on tiny shapes, causal and not."""
    for seed, (L, D) in enumerate([(1, 1), (2, 2), (3, 8), (5, 2), (17, 8)]):
        for causal in (False, True):
            q, k, v = _qkv(100 + seed, 1, 1, L, L, D)
            scale = 0.37 + 0.1 * seed
            O, LSE = attn(q, k, v, scale, causal)
            for i in range(L):
                js = list(_allowed(i, L, causal))
                s = [scale * math.fsum(q[0, 0, i, d] * k[0, 0, j, d] for d in range(D)) for j in js]
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                tot = math.fsum(w)
                for d in range(D):
                    ref = math.fsum(w[t] * v[0, 0, j, d] for t, j in enumerate(js)) / tot
                    assert abs(O[0, 0, i, d] - ref) <= 1e-13 * (1 + abs(ref)), (L, D, causal, i, d)
                assert abs(LSE[0, 0, i] - (mx + math.log(tot))) <= 1e-13 * (1 + abs(mx)), (L, D, causal, i)
    # a non-square, non-causal case
    q, k, v = _qkv(7, 1, 1, 3, 5, 2)
    O, LSE = attn(q, k, v, 0.5, False)
    for i in range(3):
        s = [0.5 * math.fsum(q[0, 0, i, d] * k[0, 0, j, d] for d in range(2)) for j in range(5)]
        mx = max(s)
        w = [math.exp(x - mx) for x in s]
        tot = math.fsum(w)
        for d in range(2):
            ref = math.fsum(w[j] * v[0, 0, j, d] for j in range(5)) / tot
            assert abs(O[0, 0, i, d] - ref) <= 1e-13


def pin_probabilities(attn):
    """V = identity makes O the attention weights: rows are distributions ([DF §2.1] stage 2),
    zero on masked keys, with ratios exp(scale·q_i·(k_j − k_j')) and LSE_i = s_ij − ln P_ij."""
    for causal in (False, True):
        L, D = 11, 3
        q, k, _ = _qkv(21, 1, 1, L, L, D)
        v = np.eye(L)[None, None]
        scale = 0.8
        P, LSE = attn(q, k, v, scale, causal)
        P, LSE = P[0, 0], LSE[0, 0]
        assert np.all(P >= 0)
        np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-14)
        if causal:
            assert np.all(np.triu(P, 1) == 0.0)
        for i in range(L):
            js = list(_allowed(i, L, causal))
            for j in js:
                s_ij = scale * float(q[0, 0, i] @ k[0, 0, j])
                assert abs(LSE[i] - (s_ij - math.log(P[i, j]))) <= 1e-12
            j0 = js[0]
            for j in js[1:]:
                ratio = math.exp(scale * float(q[0, 0, i] @ (k[0, 0, j] - k[0, 0, j0])))
                assert abs(P[i, j] / P[i, j0] - ratio) <= 1e-12 * ratio


def pin_zero_queries(attn):
    """Q = 0: every visible logit is 0, so O_i is the mean of the visible V rows (a prefix mean
    when causal) and LSE_i = ln|A_i| exactly."""
    for causal in (False, True):
        _, k, v = _qkv(31, 2, 3, 13, 13, 5)
        q = np.zeros_like(k)
        O, LSE = attn(q, k, v, 0.9, causal)
        for i in range(13):
            n = i + 1 if causal else 13
            np.testing.assert_allclose(O[:, :, i], v[:, :, :n].mean(axis=2), rtol=1e-13, atol=1e-14)
            np.testing.assert_allclose(LSE[:, :, i], math.log(n), rtol=0, atol=1e-14)


def pin_constant_values(attn):
    """A constant V (every row equal to c) gives O = c for every row: O is a convex combination."""
    for causal in (False, True):
        q, k, _ = _qkv(41, 1, 2, 10, 10, 4, sq=2.0)
        c = np.array([1.5, -2.25, 0.0, 7.0])
        v = np.broadcast_to(c, (1, 2, 10, 4)).copy()
        O, _ = attn(q, k, v, 0.6, causal)
        np.testing.assert_allclose(O, np.broadcast_to(c, O.shape), rtol=1e-14, atol=1e-14)


def pin_one_large_logit(attn):
    """One key per row leads the rest by Δ: |O_i − v_t| ≤ 2·max|V|·(n−1)·e^−Δ and
    0 ≤ LSE_i − s_it ≤ (n−1)·e^−Δ (the running-max case of [DF §2.2]), causal and not."""
    L = D = 24
    delta = 20.0
    r = _rng(51)
    k = np.eye(L) + 0.05 * r.standard_normal((L, D))     # nearly orthogonal keys
    v = r.standard_normal((L, D))
    scale = 0.5
    for causal in (False, True):
        targets = [int(r.integers(0, i + 1)) if causal else int(r.integers(0, L)) for i in range(L)]
        q = np.zeros((L, D))
        for i, t in enumerate(targets):
            vis = [j for j in _allowed(i, L, causal) if j != t]
            base = 0.1 * r.standard_normal(D)
            for _ in range(50):
                g = scale * (k @ base)
                if not vis:
                    break
                mj = max(vis, key=lambda j: g[j])
                if abs(g[t] - g[mj] - delta) < 1e-10:
                    break
                base = base + (delta + g[mj] - g[t]) / (scale * (k[t] @ k[t] - k[t] @ k[mj])) * k[t]
            q[i] = base
        O, LSE = attn(q[None, None], k[None, None], v[None, None], scale, causal)
        for i, t in enumerate(targets):
            n = i + 1 if causal else L
            s_it = scale * float(q[i] @ k[t])
            bound_o = 2 * np.abs(v).max() * (n - 1) * math.exp(-delta)
            bound_l = (n - 1) * math.exp(-delta)
            assert np.abs(O[0, 0, i] - v[t]).max() <= bound_o + 1e-12
            assert -1e-12 <= LSE[0, 0, i] - s_it <= bound_l + 1e-12
        # the bound is nearly attained: the leader is not the only visible key
        assert max(LSE[0, 0, i] - scale * float(q[i] @ k[t]) for i, t in enumerate(targets)) > 0


def pin_sdpa(attn):
    """torch's scaled_dot_product_attention on the CPU in float64 and torch.logsumexp of the
    masked scaled scores (the library form of [OP §2.1]) agree to 1e-12."""
    import torch

    for causal in (False, True):
        for (L, D) in [(16, 8), (33, 16)]:
            q, k, v = _qkv(61 + L, 2, 2, L, L, D)
            scale = 1.0 / math.sqrt(D)
            tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
            ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
            S = (tq @ tk.transpose(-1, -2)) * scale
            if causal:
                S = S.masked_fill(torch.ones(L, L, dtype=torch.bool).triu(1), float("-inf"))
            ref_lse = torch.logsumexp(S, dim=-1)
            O, LSE = attn(q, k, v, scale, causal)
            np.testing.assert_allclose(O, ref.numpy(), rtol=0, atol=1e-12)
            np.testing.assert_allclose(LSE, ref_lse.numpy(), rtol=0, atol=1e-12)


def pin_invariances(attn):
    """(i) permuting key rows of K and V together leaves O, LSE unchanged (non-causal);
    (ii) adding w to every key shifts row i's logits by scale·q_i·w: O unchanged, LSE shifted;
    (iii) O is linear in V; (iv) permuting query rows permutes O, LSE (non-causal)."""
    q, k, v = _qkv(71, 1, 2, 12, 15, 6)
    scale = 0.45
    O, LSE = attn(q, k, v, scale, False)
    perm = _rng(72).permutation(15)
    O2, L2 = attn(q, k[:, :, perm], v[:, :, perm], scale, False)
    np.testing.assert_allclose(O2, O, atol=1e-13)
    np.testing.assert_allclose(L2, LSE, atol=1e-13)
    w = _rng(73).standard_normal(6)
    O3, L3 = attn(q, k + w, v, scale, False)
    np.testing.assert_allclose(O3, O, atol=1e-12)
    np.testing.assert_allclose(L3, LSE + scale * (q @ w), atol=1e-12)
    v2 = _rng(74).standard_normal(v.shape)
    O4, _ = attn(q, k, 2.0 * v - 3.0 * v2, scale, False)
    O5, _ = attn(q, k, v2, scale, False)
    np.testing.assert_allclose(O4, 2.0 * O - 3.0 * O5, atol=1e-12)
    qp = _rng(75).permutation(12)
    O6, L6 = attn(q[:, :, qp], k, v, scale, False)
    np.testing.assert_allclose(O6, O[:, :, qp], atol=1e-13)
    np.testing.assert_allclose(L6, LSE[:, :, qp], atol=1e-13)
    # causal: the key shift still only moves LSE (every row keeps the same visible set)
    qc, kc, vc = _qkv(76, 1, 1, 10, 10, 4)
    Oc, Lc = attn(qc, kc, vc, scale, True)
    wc = _rng(77).standard_normal(4)
    Oc2, Lc2 = attn(qc, kc + wc, vc, scale, True)
    np.testing.assert_allclose(Oc2, Oc, atol=1e-12)
    np.testing.assert_allclose(Lc2, Lc + scale * (qc @ wc), atol=1e-12)


def pin_causal_prefix(attn):
    """Causal row i equals non-causal attention of row i over keys 0..i alone ([DF §4.1]);
    and a causal row never depends on later keys (changing K, V after row i leaves it)."""
    q, k, v = _qkv(81, 1, 1, 14, 14, 5)
    scale = 0.7
    O, LSE = attn(q, k, v, scale, True)
    for i in (0, 1, 6, 13):
        Oi, Li = attn(q[:, :, i : i + 1], k[:, :, : i + 1], v[:, :, : i + 1], scale, False)
        np.testing.assert_allclose(O[:, :, i], Oi[:, :, 0], atol=1e-13)
        np.testing.assert_allclose(LSE[:, :, i], Li[:, :, 0], atol=1e-13)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, 8:] += 5.0
    v2[:, :, 8:] -= 3.0
    O2, L2 = attn(q, k2, v2, scale, True)
    np.testing.assert_allclose(O2[:, :, :8], O[:, :, :8], atol=0)
    np.testing.assert_allclose(L2[:, :, :8], LSE[:, :, :8], atol=0)
    assert np.abs(O2[:, :, 8:] - O[:, :, 8:]).max() > 1e-3


def pin_scale_homogeneity(attn):
    """Scaling q by a and the scale by 1/a leaves everything unchanged; scale = 0 averages V."""
    q, k, v = _qkv(91, 1, 2, 7, 9, 3)
    O, LSE = attn(q, k, v, 0.6, False)
    O2, L2 = attn(2.0 * q, k, v, 0.3, False)
    np.testing.assert_allclose(O2, O, atol=1e-13)
    np.testing.assert_allclose(L2, LSE, atol=1e-13)
    O3, L3 = attn(q, k, v, 0.0, False)
    np.testing.assert_allclose(O3, np.broadcast_to(v.mean(axis=2, keepdims=True), O3.shape), atol=1e-14)
    np.testing.assert_allclose(L3, math.log(9), atol=1e-14)


def pin_causal_bottom_right(attn):
    """Causal with Lq < Lk (reading: the queries are the last Lq positions of the keys, so key j
    is visible to row i iff j <= i + Lk - Lq): scalar loops with exact summation; torch's
    float64 scaled_dot_product_attention with that boolean mask; row i equals non-causal
    attention over the key prefix 0..i+Lk-Lq; the last row sees every key."""
    import torch

    for seed, (Lq, Lk, D) in enumerate([(1, 5, 2), (3, 7, 4), (6, 6, 3), (2, 9, 8)]):
        q, k, v = _qkv(400 + seed, 1, 1, Lq, Lk, D)
        scale = 0.41 + 0.1 * seed
        O, LSE = attn(q, k, v, scale, True)
        for i in range(Lq):
            js = range(0, i + Lk - Lq + 1)
            s_ = [scale * math.fsum(q[0, 0, i, d] * k[0, 0, j, d] for d in range(D)) for j in js]
            mx = max(s_)
            w = [math.exp(x - mx) for x in s_]
            tot = math.fsum(w)
            for d in range(D):
                ref = math.fsum(w[t] * v[0, 0, j, d] for t, j in enumerate(js)) / tot
                assert abs(O[0, 0, i, d] - ref) <= 1e-13 * (1 + abs(ref)), (Lq, Lk, i, d)
            assert abs(LSE[0, 0, i] - (mx + math.log(tot))) <= 1e-13 * (1 + abs(mx)), (Lq, Lk, i)
    q, k, v = _qkv(410, 2, 2, 11, 30, 8)
    scale = 0.3
    O, LSE = attn(q, k, v, scale, True)
    mask = torch.arange(30)[None, :] <= torch.arange(11)[:, None] + 19
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
    S = ((tq @ tk.transpose(-1, -2)) * scale).masked_fill(~mask, float("-inf"))
    np.testing.assert_allclose(O, ref.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(LSE, torch.logsumexp(S, dim=-1).numpy(), rtol=0, atol=1e-12)
    for i in (0, 5, 10):
        Oi, Li = attn(q[:, :, i : i + 1], k[:, :, : i + 20], v[:, :, : i + 20], scale, False)
        np.testing.assert_allclose(O[:, :, i], Oi[:, :, 0], atol=1e-13)
        np.testing.assert_allclose(LSE[:, :, i], Li[:, :, 0], atol=1e-13)


PINS = [pin_golden, pin_brute_force, pin_probabilities, pin_zero_queries, pin_constant_values,
        pin_one_large_logit, pin_sdpa, pin_invariances, pin_causal_prefix, pin_scale_homogeneity,
        pin_causal_bottom_right]


def _oracle_attn(q, k, v, scale, causal):
    return attention_fp64(q, k, v, scale, causal)


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin_holds_for_oracle(pin):
    pin(_oracle_attn)


# --------------------------------------------------------------------------------------------
# planted mistakes: each must be caught by at least one pin
# --------------------------------------------------------------------------------------------

MUTANTS = {
    "dropped_scale": ("S = (q[r] @ kT) * scale", "S = (q[r] @ kT)"),
    "negated_scale": ("S = (q[r] @ kT) * scale", "S = (q[r] @ kT) * -scale"),
    "mask_excludes_diagonal": ("> r[:, None] + off] = -np.inf", ">= r[:, None] + off] = -np.inf"),
    "mask_one_extra_key": ("> r[:, None] + off] = -np.inf", "> r[:, None] + off + 1] = -np.inf"),
    "mask_transposed": ("> r[:, None] + off] = -np.inf", "< r[:, None] + off] = -np.inf"),
    "mask_top_left": ("> r[:, None] + off] = -np.inf", "> r[:, None]] = -np.inf"),
    "mask_offset_reversed": ("> r[:, None] + off] = -np.inf", "> r[:, None] - off] = -np.inf"),
    "no_max_in_lse": ("LSE[c0 : c0 + chunk] = m + np.log(l)", "LSE[c0 : c0 + chunk] = np.log(l)"),
    "lse_base2": ("m + np.log(l)", "m + np.log2(l)"),
    "no_normalisation": ("(P @ v) / l[:, None]", "(P @ v)"),
    "keys_as_values": ("(P @ v) / l[:, None]", "(P @ k) / l[:, None]"),
    "values_as_keys": ("S = (q[r] @ kT) * scale", "S = (q[r] @ v.T) * scale"),
    "exp2_not_exp": ("P = np.exp(S - m[:, None])", "P = np.exp2(S - m[:, None])"),
    "max_not_subtracted_in_sum": ("l = P.sum(axis=1)", "l = np.exp(S).sum(axis=1)"),
    "first_key_dropped": ("m = S.max(axis=1)", "S[:, 0] = -np.inf\n        m = S.max(axis=1)"),
    "transposed_scores": ("S = (q[r] @ kT) * scale", "S = (k[r] @ q.T) * scale if False else (q[r] @ kT).T[: len(r)] * scale"),
}


def _load_mutant(name):
    old, new = MUTANTS[name]
    with open(ORACLE_SRC, encoding="utf-8") as f:
        src = f.read()
    assert old in src, f"mutation anchor for {name} not found in the oracle"
    src = src.replace(old, new, 1)
    mod = types.ModuleType(f"oracle.oracle_mutant_{name}")
    mod.__dict__["__name__"] = mod.__name__
    mod.__dict__["__package__"] = "oracle"  # the oracle's relative imports resolve in its package
    sys.modules[mod.__name__] = mod
    exec(compile(src, ORACLE_SRC + f"<{name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    mod = _load_mutant(name)

    def attn(q, k, v, scale, causal):
        return mod.attention_fp64(q, k, v, scale, causal)

    failures = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(attn)
        except Exception as e:  # AssertionError, or a shape error the mistake causes
            failures.append((pin.__name__, type(e).__name__))
    assert failures, f"no pin catches the planted mistake {name!r}"


# --------------------------------------------------------------------------------------------
# the streaming recurrence equals the definition (the method the kernel implements)
# --------------------------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("bq,bk", [(128, 64), (64, 64), (16, 8), (7, 5), (1, 1)])
def test_streaming_equals_definition(causal, bq, bk):
    r = _rng(5)
    L, D = 97, 16
    q = r.standard_normal((L, D)) * 2.0
    k = r.standard_normal((L, D))
    v = r.standard_normal((L, D))
    O_ref, L_ref = attention_head_fp64(q, k, v, 0.3, causal)
    O, LSE = streaming_attention_fp64(q, k, v, 0.3, causal, bq, bk)
    np.testing.assert_allclose(O, O_ref, atol=1e-12)
    np.testing.assert_allclose(LSE, L_ref, atol=1e-12)


def test_streaming_key_block_order_is_irrelevant():
    r = _rng(6)
    L, D = 80, 8
    q, k, v = (r.standard_normal((L, D)) for _ in range(3))
    O_ref, L_ref = attention_head_fp64(q, k, v, 0.5, True)
    O, LSE = streaming_attention_fp64(q, k, v, 0.5, True, 32, 16, key_block_order=[4, 0, 3, 1, 2])
    np.testing.assert_allclose(O, O_ref, atol=1e-12)
    np.testing.assert_allclose(LSE, L_ref, atol=1e-12)


def test_rows_subset_matches_full():
    q, k, v = _qkv(3, 2, 2, 40, 40, 8)
    O, LSE = attention_fp64(q, k, v, 0.35, True)
    rows = [0, 5, 39, 17]
    Os, Ls = attention_fp64(q, k, v, 0.35, True, rows=rows, chunk=3)
    # same definition per row; only BLAS blocking (rounding order) differs between chunkings
    np.testing.assert_allclose(Os, O[:, :, rows], rtol=0, atol=1e-14)
    np.testing.assert_allclose(Ls, LSE[:, :, rows], rtol=0, atol=1e-14)


def test_causal_with_more_queries_than_keys_is_rejected():
    q, k, v = _qkv(420, 1, 1, 6, 4, 2)
    with pytest.raises(ValueError):
        attention_fp64(q, k, v, 0.5, True)
