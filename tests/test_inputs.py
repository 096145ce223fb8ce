"""The seeded synthetic-input recipe: determinism, stream layout, rounding and the peaked-softmax boost."""

from __future__ import annotations

import dataclasses
import hashlib
import math

import numpy as np
import pytest
import torch

import attn_inputs as ai


def _digest(t: torch.Tensor) -> str:
    return hashlib.sha256(t.contiguous().view(torch.int16).numpy().tobytes()).hexdigest()


def test_same_seed_same_bits_and_different_seed_differs():
    a = ai.make_inputs("tiny")
    b = ai.make_inputs("tiny")
    c = ai.make_inputs("tiny", seed=1234)
    for key in ("q", "k", "v"):
        assert _digest(a[key]) == _digest(b[key])
        assert _digest(a[key]) != _digest(c[key])
    assert a["q"].dtype == torch.float16 and a["q"].shape == (1, 1, 128, 64)


def test_chunked_draw_equals_one_shot():
    r1 = np.random.Generator(np.random.PCG64(9))
    r2 = np.random.Generator(np.random.PCG64(9))
    x = ai.draw_normal(r1, (3, 5, 7, 11), chunk=13)
    y = r2.standard_normal(3 * 5 * 7 * 11).reshape(3, 5, 7, 11)
    np.testing.assert_array_equal(x, y)


def test_draw_order_q_then_k_then_v():
    w = ai.WORKLOADS["tiny"]
    inp = ai.make_inputs(w)
    r = np.random.Generator(np.random.PCG64(w.seed))
    n = w.B * w.H * w.Lq * w.D
    raw = r.standard_normal(3 * n)
    for i, key in enumerate(("q", "k", "v")):
        ref = ai.round_to(raw[i * n : (i + 1) * n].reshape(inp[key].shape), w.dtype)
        assert torch.equal(inp[key], ref)


@pytest.mark.parametrize("dtype,ulp_bits", [("fp16", 10), ("bf16", 7)])
def test_rounding_is_nearest(dtype, ulp_bits):
    r = np.random.Generator(np.random.PCG64(3))
    x = r.standard_normal(20000) * 3.0
    t = ai.round_to(x, dtype).to(torch.float64).numpy()
    # |x - round(x)| <= half an ulp of the rounded value's binade (plus the fp32 step)
    e = np.floor(np.log2(np.maximum(np.abs(x), 1e-30)))
    min_e = -14 if dtype == "fp16" else -126          # below this the format is subnormal
    half_ulp = 2.0 ** (np.maximum(e, min_e) - ulp_bits - 1)
    assert np.all(np.abs(x - t) <= half_ulp * (1 + 1e-6) + 2.0 ** (e - 24))


def test_moments_and_sigma():
    inp = ai.make_inputs("tiny")
    for key in ("q", "k", "v"):
        x = inp[key].double().numpy()
        assert abs(x.mean()) < 0.05 and abs(x.std() - 1.0) < 0.05


def test_workload_table():
    w = ai.WORKLOADS
    assert [x.name for x in w.values()] == ["tiny", "llama7b_2k", "train7b_4k", "stress_8k", "long_16k"]
    assert (w["train7b_4k"].B, w["train7b_4k"].H, w["train7b_4k"].Lq, w["train7b_4k"].D) == (4, 32, 4096, 128)
    assert w["train7b_4k"].causal and w["train7b_4k"].dtype == "bf16"
    assert w["stress_8k"].scale == 0.125 and w["stress_8k"].boost == 20.0
    assert math.isclose(w["train7b_4k"].flops, 4 * 4 * 32 * 4096 * 4096 * 128 / 2)


def test_split_workload_flops_and_bytes():
    s = ai.SPLIT_WORKLOADS
    assert set(s) == {"kvcache_16k", "decode_32k", "prefill_chunk_8k"} and not set(s) & set(ai.WORKLOADS)
    # causal with Lq < Lk: row i sees Lk - Lq + i + 1 keys; the count is Lq·(Lk - Lq/2) + Lq/2
    w = s["prefill_chunk_8k"]
    pairs = sum(w.Lk - w.Lq + i + 1 for i in range(w.Lq))
    assert math.isclose(w.flops, 4 * w.B * w.H * w.D * (pairs - w.Lq / 2))
    d = s["decode_32k"]
    assert math.isclose(d.flops, 4 * 8 * 32768 * 128 - 4 * 8 * 128 / 2)
    assert d.hbm_bytes == 2 * (2 * 8 * 128 + 2 * 8 * 32768 * 128) + 4 * 8
    assert ai.make_inputs("decode_32k")["q"].shape == (1, 8, 1, 128)


def test_boost_margin_after_rounding():
    """A reduced stress workload (same recipe, L=1024): each row's target logit leads every other
    logit by about 20 after Q is rounded to bf16; targets cover the key range."""
    w = dataclasses.replace(ai.WORKLOADS["stress_8k"], B=1, H=2, Lq=1024, Lk=1024)
    inp = ai.make_inputs(w)
    q = inp["q"].double().numpy()
    k = inp["k"].double().numpy()
    t = inp["targets"]
    margins = []
    for h in range(2):
        S = (q[0, h] @ k[0, h].T) * w.scale
        st = S[np.arange(w.Lq), t[0, h]]
        S[np.arange(w.Lq), t[0, h]] = -np.inf
        margins.append(st - S.max(axis=1))
    m = np.concatenate(margins)
    assert m.min() > 19.5 and m.max() < 20.5, (m.min(), m.max())
    assert len(np.unique(t)) > 0.5 * w.Lk
    # K and V are untouched by the boost: they equal a plain draw with the same seed
    r = np.random.Generator(np.random.PCG64(w.seed))
    ai.draw_normal(r, (1, 2, 1024, 64))
    assert torch.equal(inp["k"], ai.round_to(ai.draw_normal(r, (1, 2, 1024, 64)), "bf16"))
