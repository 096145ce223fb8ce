"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle on the same rounded inputs.

Bar per element, tol = 2e-3 (fp16) or 1e-2 (bf16), |LSE_gpu − LSE_ref| <= 1e-3:

    |O_gpu − O_ref| <= tol,
    or, only where the output format itself is coarser than tol,
    |O_gpu − O_ref| <= half_ulp(|O_ref| + E) + E     where half_ulp(|O_ref| + E) > tol,

with E the bound on the unrounded fp32 result's error that follows from the
kernel's roundings (numerics.fwd_allowance; the CPU model of those roundings stays
within it, tests/test_numerics.py).  The format is coarser than tol only for
|O| >= 4 in bf16 and |O| >= 8 in fp16; everywhere else the plain tol applies.
Every comparison reports the plain max-abs error, how many elements exceeded tol
and how many of those the format's rounding explains.

Outputs are pre-filled with NaN so that an element the kernel fails to write fails
the test.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest
import torch

import attn_inputs as ai
import tiled_attention_06_amd as fa
from numerics import fwd_allowance, half_ulp, round_to_dtype
from numerics.bounds import fwd_check
from oracle import attention_fp64
from oracle.philox import dropout_keep, keep_threshold
from oracle_pool import oracle_all_heads

pytestmark = pytest.mark.gpu

TOL = {"fp16": 2e-3, "bf16": 1e-2}
LSE_TOL = 1e-3
DEV = "cuda:0"


def ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """The spacing of the format's values at |x| (used for slack in hull checks)."""
    return 2.0 * half_ulp(x, dtype)


def note(msg: str):
    print(msg, flush=True)


def run_gpu(inp, stream=None):
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
    fa.fa_fwd(q, k, v, o, lse, causal=inp["causal"], scale=inp["scale"], stream=stream)
    torch.cuda.synchronize()
    return o, lse


def _np(x):
    return x.double().cpu().numpy() if torch.is_tensor(x) else np.asarray(x, dtype=np.float64)


def compare(o, lse, O_ref, L_ref, dtype, what="", src=None, heads=None, rows=None):
    """o, O_ref: [B,H,R,D]; lse, L_ref: [B,H,R].  ``src``: the inputs dict (q, k, v on the CPU, scale,
    causal, and optionally dropout_p / seed) from which the allowance of elements over tol is computed
    (without it, the plain tol applies everywhere); ``heads``: the (b, h) pairs to check (default all);
    ``rows``: the query rows that the R axis holds (default 0..R-1).  Returns the statistics."""
    o, lse, O_ref, L_ref = _np(o), _np(lse), _np(O_ref), _np(L_ref)
    B, H, R = O_ref.shape[:3]
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    rows = np.arange(R) if rows is None else np.asarray(rows)
    st = {"max_abs_err": 0.0, "max_abs_err_lse": 0.0, "floor": 0.0, "err_vs_rounded_ref": 0.0, "n_over_tol": 0,
          "n_allowed": 0, "max_abs_o_ref": 0.0, "elements": 0}
    tol = TOL[dtype]
    for b, h in pairs:
        ob, Ob, lb, Lb = o[b, h], O_ref[b, h], lse[b, h], L_ref[b, h]
        assert np.isfinite(ob).all(), f"{what} ({b},{h}): non-finite O (unwritten or NaN)"
        assert np.isfinite(lb).all(), f"{what} ({b},{h}): non-finite LSE (unwritten or NaN)"
        allowance = None
        if src is not None:
            qh, kh, vh = (src[n][b, h].double().numpy() for n in ("q", "k", "v"))
            p = src.get("dropout_p", 0.0)

            def allowance(idx, qh=qh, kh=kh, vh=vh, Ob=Ob, b=b, h=h, p=p):
                r_ = rows[idx]
                keep = None
                if p:
                    keep = dropout_keep(b * H + h, r_, np.arange(kh.shape[0]), p, src["seed"])
                return fwd_allowance(qh, kh, vh, Ob[idx], src["scale"], src["causal"], dtype, r_, keep=keep,
                                     keep_scale=256.0 / keep_threshold(p) if p else 1.0)
        ok, info = fwd_check(ob, Ob, dtype, tol, allowance)
        rnd = round_to_dtype(Ob, dtype)
        st["max_abs_err"] = max(st["max_abs_err"], info["max_abs_err"])
        st["floor"] = max(st["floor"], float(np.abs(rnd - Ob).max()))
        st["err_vs_rounded_ref"] = max(st["err_vs_rounded_ref"], float(np.abs(ob - rnd).max()))
        st["n_over_tol"] += info["n_over_tol"]
        st["n_allowed"] += info["n_allowed"]
        st["max_abs_o_ref"] = max(st["max_abs_o_ref"], float(np.abs(Ob).max()))
        st["max_abs_err_lse"] = max(st["max_abs_err_lse"], float(np.abs(lb - Lb).max()))
        st["elements"] += int(ob.size)
        if not ok:
            raise AssertionError(f"{what} ({b},{h}): O outside the bar ({info}); worst {info.get('worst')}")
    note(f"  {what}: max|dO|={st['max_abs_err']:.3e} (floor {st['floor']:.3e}, vs rounded ref "
         f"{st['err_vs_rounded_ref']:.3e}) max|dLSE|={st['max_abs_err_lse']:.3e} max|O|={st['max_abs_o_ref']:.2f} "
         f"over tol {st['n_over_tol']} (explained by the format: {st['n_allowed']}) of {st['elements']}")
    assert st["max_abs_err_lse"] <= LSE_TOL, f"{what}: LSE error {st['max_abs_err_lse']:.4e}"
    return st


def _report(name: str, stats: dict):
    """Per-workload numbers for the measurement record, when FA_PARITY_REPORT_DIR is set."""
    d = os.environ.get("FA_PARITY_REPORT_DIR")
    if d:
        os.makedirs(d, exist_ok=True)
        with open(os.path.join(d, f"{name}.json"), "w") as f:
            json.dump(stats, f, indent=1)


# ------------------------------------------------------------------------------------------
# edge shapes (full comparison)
# ------------------------------------------------------------------------------------------

EDGE = [(1, 2, L, L, D, dt, c) for D in (64, 128) for dt in ("fp16", "bf16") for c in (False, True)
        for L in (1, 2, 63, 64, 65, 127, 128, 129, 1000)]
EDGE += [(1, 1, Lq, Lk, D, dt, False) for D in (64, 128) for dt in ("fp16", "bf16")
         for (Lq, Lk) in ((1, 300), (200, 77), (129, 1000), (1000, 129), (64, 1))]
EDGE += [(3, 5, 100, 100, 128, "bf16", True), (2, 3, 257, 257, 64, "fp16", True),
         (1, 1, 4097, 4097, 128, "bf16", True), (1, 1, 4097, 4097, 64, "fp16", False)]


@pytest.mark.parametrize("B,H,Lq,Lk,D,dtype,causal", EDGE,
                         ids=[f"B{b}H{h}_{lq}x{lk}_D{d}_{dt}_{'c' if c else 'nc'}" for b, h, lq, lk, d, dt, c in EDGE])
def test_edge_shapes(B, H, Lq, Lk, D, dtype, causal):
    seed = 10_000 + 97 * Lq + 13 * Lk + D + (1 if causal else 0) + (2 if dtype == "bf16" else 0)
    inp = ai.make_custom(B, H, Lq, Lk, D, dtype, causal, seed=seed)
    note(f"edge B{B} H{H} Lq{Lq} Lk{Lk} D{D} {dtype} causal={causal} seed={seed}")
    o, lse = run_gpu(inp)
    O_ref, L_ref = attention_fp64(inp["q"], inp["k"], inp["v"], inp["scale"], causal)
    compare(o, lse, O_ref, L_ref, dtype, "edge", src=inp)


# Grids of 256-row workgroups larger than the CU count (256 on MI355X) run that form; smaller
# ones (every case above) run 128-row workgroups whose 8 waves form two key groups.  These cases
# keep ragged tails and both sides of that boundary covered for the 256-row form.
WIDE = [(1, 300, 300, 300, 64, "fp16", True), (1, 300, 300, 300, 128, "bf16", False),
        (2, 130, 129, 1000, 128, "bf16", False), (1, 257, 65, 65, 64, "bf16", True),
        (1, 256, 65, 65, 128, "fp16", True), (1, 257, 65, 65, 128, "fp16", True),
        (4, 40, 700, 700, 128, "bf16", True)]


@pytest.mark.parametrize("B,H,Lq,Lk,D,dtype,causal", WIDE,
                         ids=[f"B{b}H{h}_{lq}x{lk}_D{d}_{dt}_{'c' if c else 'nc'}" for b, h, lq, lk, d, dt, c in WIDE])
def test_wide_grids(B, H, Lq, Lk, D, dtype, causal):
    seed = 20_000 + 7 * H + 97 * Lq + 13 * Lk + D + (1 if causal else 0)
    inp = ai.make_custom(B, H, Lq, Lk, D, dtype, causal, seed=seed)
    note(f"wide B{B} H{H} Lq{Lq} Lk{Lk} D{D} {dtype} causal={causal} seed={seed}")
    o, lse = run_gpu(inp)
    O_ref, L_ref = attention_fp64(inp["q"], inp["k"], inp["v"], inp["scale"], causal)
    compare(o, lse, O_ref, L_ref, dtype, "wide", src=inp)


@pytest.mark.parametrize("D,dtype,causal", [(128, "bf16", False), (128, "fp16", True), (64, "bf16", False),
                                            (64, "fp16", True)])
def test_step_counts(D, dtype, causal):
    # The 256-row form's software-pipelined loop joins its waves after every second step and
    # copies tiles on a schedule that depends on the step's parity; before the last full tile
    # and the masked tiles it returns to one join per step.  257 heads of 65 query rows (257
    # workgroups: that form) with 1 to 10 key tiles, full or ragged, end the loop after every
    # count of steps, odd and even, and with 0 to 3 tiles left to copy.
    for Lk in (64, 81, 128, 145, 192, 209, 256, 273, 320, 337, 384, 401, 448, 465, 512, 529, 576, 640):
        if causal and Lk < 65:
            continue  # causal needs Lq <= Lk
        seed = 32_000 + Lk + D + (1 if causal else 0)
        inp = ai.make_custom(1, 257, 65, Lk, D, dtype, causal, seed=seed)
        note(f"step counts H257 Lq65 Lk{Lk} D{D} {dtype} causal={causal} seed={seed}")
        o, lse = run_gpu(inp)
        heads = [(0, 0), (0, 128), (0, 256)]
        sub = {x: inp[x][:, [h for _, h in heads]] for x in ("q", "k", "v")}
        O_ref, L_ref = attention_fp64(sub["q"], sub["k"], sub["v"], inp["scale"], causal)
        idx = [h for _, h in heads]
        compare(o[:, idx], lse[:, idx], O_ref, L_ref, dtype, f"step counts Lk{Lk}", src={**inp, **sub})


@pytest.mark.parametrize("D,dtype,causal", [(128, "bf16", True), (64, "fp16", False), (128, "fp16", False)])
def test_geometry_forms(D, dtype, causal):
    # 300 heads of 520 rows (3 query tiles of 256: 900 workgroups, the 256-row form) and the first 4
    # heads alone (12 workgroups of 128 rows: the two-key-group form) both against the oracle on
    # those heads.  Within one form a row does not depend on the rest of the grid: the first 296
    # heads (888 workgroups, whose count lets the XCD-aware order run) and the first 8 heads (24
    # workgroups) must reproduce the larger launches bit for bit.
    inp = ai.make_custom(1, 300, 520, 520, D, dtype, causal, seed=31_000 + D)
    note(f"geometry B1 H300 L520 D{D} {dtype} causal={causal}")
    sub = lambda n: {**inp, **{x: inp[x][:, :n].contiguous() for x in ("q", "k", "v")}}
    o_all, l_all = run_gpu(inp)
    o_296, l_296 = run_gpu(sub(296))
    o_few, l_few = run_gpu(sub(4))
    o_8, l_8 = run_gpu(sub(8))
    assert torch.equal(o_all[:, :296], o_296) and torch.equal(l_all[:, :296], l_296), \
        "256-row form: result depends on the grid"
    assert torch.equal(o_8[:, :4], o_few) and torch.equal(l_8[:, :4], l_few), \
        "two-key-group form: result depends on the grid"
    few = sub(4)
    O_ref, L_ref = attention_fp64(few["q"], few["k"], few["v"], inp["scale"], causal)
    compare(o_all[:, :4], l_all[:, :4], O_ref, L_ref, dtype, "geometry 256-row form", src=few)
    compare(o_few, l_few, O_ref, L_ref, dtype, "geometry two-key-group form", src=few)
    if causal:  # row 0 sees key 0 alone in either form: O equals v_0 exactly
        assert torch.equal(o_few[:, :, 0].cpu(), few["v"][:, :, 0])
        assert torch.equal(o_all[:, :4, 0].cpu(), few["v"][:, :, 0])


@pytest.mark.parametrize("H,L,D,dtype,causal", [
    (32, 2048, 128, "fp16", True),   # 512 items: XCD blocks of 64 items, two head pairs each
    (18, 1900, 128, "bf16", True),   # 270 items in one block (270 is no multiple of 16)
    (19, 1900, 64, "bf16", False),   # 285 items: the middle one runs alone
])
def test_paired_form(H, L, D, dtype, causal):
    # Two-key-group grids with more items than CUs (256 on this GPU) run two items per
    # workgroup, a heavy causal query tile and then a light one, the second one's Q rows and
    # first K tiles requested while the first one's results are merged and stored.  A row's
    # result does not depend on that: the first heads alone (at most 256 items, one per
    # workgroup) reproduce those heads bit for bit, and both match the oracle.
    inp = ai.make_custom(1, H, L, L, D, dtype, causal, seed=37_000 + H)
    note(f"paired form B1 H{H} L{L} D{D} {dtype} causal={causal}")
    n = H // 2
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        # the full grid runs paired, the subset one item per workgroup (both in 128-row items)
        n_items = H * -(-L // 128)
        assert fa.fa_fwd_launch_shape(1, H, L, L, D, causal) == ((n_items + 1) // 2, 128, 2)
        assert fa.fa_fwd_launch_shape(1, n, L, L, D, causal) == (n * -(-L // 128), 128, 1)
    sub = {**inp, **{x: inp[x][:, :n].contiguous() for x in ("q", "k", "v")}}
    o_all, l_all = run_gpu(inp)
    o_sub, l_sub = run_gpu(sub)
    assert torch.equal(o_all[:, :n], o_sub) and torch.equal(l_all[:, :n], l_sub), \
        "two-key-group form: result depends on the pairing of items"
    heads = [0, H - 1]
    pick = {**inp, **{x: inp[x][:, heads].contiguous() for x in ("q", "k", "v")}}
    O_ref, L_ref = attention_fp64(pick["q"], pick["k"], pick["v"], inp["scale"], causal)
    compare(o_all[:, heads], l_all[:, heads], O_ref, L_ref, dtype, "paired form", src=pick)


# ------------------------------------------------------------------------------------------
# the five workloads at full size, in the launch configuration the bench times
# ------------------------------------------------------------------------------------------

def _sample(w, seed=0):
    r = np.random.default_rng(seed)
    heads = {(0, 0), (w.B - 1, w.H - 1)}
    while len(heads) < min(4, w.B * w.H):
        heads.add((int(r.integers(w.B)), int(r.integers(w.H))))
    rows = np.unique(np.concatenate([np.arange(min(32, w.Lq)), np.arange(max(0, w.Lq - 32), w.Lq),
                                     r.integers(0, w.Lq, 64)]))
    return sorted(heads), rows


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", list(ai.WORKLOADS))
def test_workload(name):
    # every row of every head against the oracle (one head per worker process), in the launch
    # configuration the bench times
    w = ai.WORKLOADS[name]
    note(f"workload {name}: generating inputs")
    inp = ai.make_inputs(w)
    note(f"workload {name}: GPU run {w.description}")
    o, lse = run_gpu(inp)
    o_c, lse_c = o.double().cpu().numpy(), lse.double().cpu().numpy()
    assert np.isfinite(o_c).all() and np.isfinite(lse_c).all(), "unwritten or non-finite output"
    note(f"workload {name}: oracle over all {w.B * w.H} heads")
    O_ref, L_ref = oracle_all_heads(inp["q"], inp["k"], inp["v"], w.scale, w.causal)
    st = compare(o_c, lse_c, O_ref, L_ref, w.dtype, f"{name} (all rows)", src=inp)
    st.update(workload=name, description=w.description, tol=TOL[w.dtype], lse_tol=LSE_TOL)
    _report(name, st)
    del O_ref, L_ref
    # properties on every row: O is a convex combination of the visible V rows
    v = inp["v"].double()
    if w.causal:
        lo = torch.cummin(v, dim=2).values.numpy()
        hi = torch.cummax(v, dim=2).values.numpy()
    else:
        lo = v.min(dim=2, keepdim=True).values.numpy()
        hi = v.max(dim=2, keepdim=True).values.numpy()
    slack = ulp(np.maximum(np.abs(lo), np.abs(hi)), w.dtype)
    assert (o_c >= lo - slack).all() and (o_c <= hi + slack).all(), "O outside the hull of visible V rows"
    if w.causal:
        # row 0 sees only key 0: its weight is exactly 1, so O equals v_0 bit for bit
        assert torch.equal(o[:, :, 0].cpu(), inp["v"][:, :, 0])
    if w.boost is not None:
        # peaked softmax: O_i ≈ v_target (|O − v_t| ≤ 2·max|V|·(n−1)·e^−Δmin + rounding)
        t = inp["targets"]
        vt = np.take_along_axis(v.numpy(), t[..., None], axis=2)
        dev_ = np.abs(o_c - vt).max()
        note(f"  {name}: max|O - v_target| = {dev_:.3e}")
        assert dev_ <= 2 * np.abs(v.numpy()).max() * (w.Lk - 1) * math.exp(-19.5) + 2 * TOL[w.dtype]


# ------------------------------------------------------------------------------------------
# GPU forms of the oracle's closed forms and invariants
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_zero_queries_give_prefix_means(dtype, causal):
    inp = ai.make_custom(2, 2, 300, 300, 128, dtype, causal, seed=501)
    inp["q"] = torch.zeros_like(inp["q"])
    note(f"Q=0 {dtype} causal={causal}")
    o, lse = run_gpu(inp)
    v = inp["v"].double().numpy()
    n = np.arange(1, 301) if causal else np.full(300, 300)
    mean = np.cumsum(v, axis=2) / n[:, None] if causal else np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
    compare(o, lse, mean, np.broadcast_to(np.log(n), lse.shape), dtype, "Q=0", src=inp)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_constant_values_are_exact(dtype):
    inp = ai.make_custom(1, 3, 333, 333, 64, dtype, True, seed=502)
    c = torch.tensor([0.75, -2.5, 1.0, 3.0] * 16).to(inp["v"].dtype)
    inp["v"] = c.expand_as(inp["v"]).contiguous()
    note(f"constant V {dtype}")
    o, _ = run_gpu(inp)
    assert torch.equal(o.cpu(), inp["v"]), "a constant V must come back exactly"


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_key_permutation_and_shift_invariance(dtype):
    inp = ai.make_custom(1, 2, 200, 500, 128, dtype, False, seed=503)
    note(f"invariance {dtype}")
    o0, l0 = run_gpu(inp)
    perm = torch.from_numpy(np.random.default_rng(5).permutation(500))
    p = dict(inp, k=inp["k"][:, :, perm].contiguous(), v=inp["v"][:, :, perm].contiguous())
    o1, l1 = run_gpu(p)
    tol = TOL[dtype]
    assert (o1.double() - o0.double()).abs().max().item() <= 2 * tol
    assert (l1 - l0).abs().max().item() <= 2 * LSE_TOL
    # a shift of every key by w moves LSE_i by scale·q_i·w and leaves O.  K is put on a
    # grid of quarters in [-4, 4] first so that K and K + w are both exact in fp16/bf16.
    kq = (inp["k"].double() * 4).round().clamp(-16, 16) / 4
    base = dict(inp, k=kq.to(inp["k"].dtype))
    w = torch.zeros(128, dtype=torch.float64)
    w[::3] = 0.5
    shifted = dict(inp, k=(kq + w).to(inp["k"].dtype))
    assert torch.equal(shifted["k"].double(), kq + w)
    o2, l2 = run_gpu(base)
    o3, l3 = run_gpu(shifted)
    shift = inp["scale"] * (inp["q"].double() @ w)
    assert (o3.double() - o2.double()).abs().max().item() <= 2 * tol
    assert (l3.double().cpu() - l2.double().cpu() - shift).abs().max().item() <= 2 * LSE_TOL


@pytest.mark.parametrize("scale", [-0.2, 0.0, 1.7, 1e-3])
def test_scale_values(scale):
    inp = ai.make_custom(1, 2, 190, 190, 64, "bf16", True, seed=504)
    inp["scale"] = scale
    note(f"scale {scale}")
    o, lse = run_gpu(inp)
    O_ref, L_ref = attention_fp64(inp["q"], inp["k"], inp["v"], scale, True)
    compare(o, lse, O_ref, L_ref, "bf16", f"scale={scale}", src=inp)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_large_logits_running_max(dtype):
    """Logits spread over hundreds of units: exercises the rescale of partial sums."""
    inp = ai.make_custom(1, 2, 400, 400, 128, dtype, False, seed=505, sigma_q=6.0, sigma_k=4.0)
    note(f"large logits {dtype}")
    o, lse = run_gpu(inp)
    O_ref, L_ref = attention_fp64(inp["q"], inp["k"], inp["v"], inp["scale"], False)
    compare(o, lse, O_ref, L_ref, dtype, "large logits", src=inp)


def test_bitwise_deterministic_and_stream():
    inp = ai.make_custom(2, 4, 1000, 1000, 128, "bf16", True, seed=506)
    note("determinism + non-default stream")
    o0, l0 = run_gpu(inp)
    for _ in range(2):
        o1, l1 = run_gpu(inp)
        assert torch.equal(o0, o1) and torch.equal(l0, l1)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o2, l2 = run_gpu(inp, stream=s)
    assert torch.equal(o0, o2) and torch.equal(l0, l2)


def test_outputs_written_into_given_buffers():
    inp = ai.make_custom(1, 1, 77, 77, 64, "fp16", False, seed=507)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    o = torch.full_like(q, float("nan"))
    lse = torch.full((1, 1, 77), float("nan"), device=DEV)
    o2, lse2 = fa.fa_fwd(q, k, v, o, lse)
    torch.cuda.synchronize()
    assert o2.data_ptr() == o.data_ptr() and lse2.data_ptr() == lse.data_ptr()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()


# ------------------------------------------------------------------------------------------
# strided and packed layouts (fa_fwd_strided): the same results on views of other layouts
# ------------------------------------------------------------------------------------------

def _views(layout, inp, pad=64):
    """GPU views of q, k, v and an output view o in the requested layout, plus a check of o's padding."""
    q, k, v = (inp[n] for n in ("q", "k", "v"))
    B, H, Lq, D = q.shape
    Lk = k.shape[2]
    blhd = lambda t: t.transpose(1, 2).contiguous().to(DEV).transpose(1, 2)   # [B,L,H,D] storage, [B,H,L,D] view
    if layout == "blhd":
        o_buf = torch.full((B, Lq, H, D), float("nan"), dtype=q.dtype, device=DEV)
        return blhd(q), blhd(k), blhd(v), o_buf.transpose(1, 2), None
    if layout == "padded":
        def padded(t):
            buf = torch.zeros(t.shape[0], t.shape[1] + 1, t.shape[2], t.shape[3] + pad, dtype=t.dtype)
            buf[:, :-1, :, :D] = t
            return buf.to(DEV)[:, :-1, :, :D]
        o_buf = torch.full((B, H + 1, Lq, D + pad), 7.0, dtype=q.dtype, device=DEV)
        o = o_buf[:, :-1, :, :D]
        def untouched():
            assert bool((o_buf[:, -1] == 7).all()) and bool((o_buf[..., D:] == 7).all()), "padding of o written"
        return padded(q), padded(k), padded(v), o, untouched
    if layout == "broadcast_kv":
        # one K/V slab shared by every batch and head: zero batch and head strides
        k1, v1 = k[:1, :1].to(DEV), v[:1, :1].to(DEV)
        return q.to(DEV), k1.expand(B, H, Lk, D), v1.expand(B, H, Lk, D), None, None
    if layout == "mixed":
        o_buf = torch.full((B, Lq, H, D + 8), float("nan"), dtype=q.dtype, device=DEV)
        return q.to(DEV), blhd(k), blhd(v), o_buf[..., :D].transpose(1, 2), None
    raise ValueError(layout)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D,dtype", [(128, "bf16"), (64, "fp16")])
@pytest.mark.parametrize("layout", ["blhd", "padded", "broadcast_kv", "mixed"])
def test_strided_layouts(layout, D, dtype, causal):
    inp = ai.make_custom(2, 3, 300, 300, D, dtype, causal, seed=700 + D + (1 if causal else 0))
    note(f"strided {layout} D{D} {dtype} causal={causal}")
    q, k, v, o, check = _views(layout, inp)
    o, lse = fa.fa_fwd(q, k, v, o, causal=causal, scale=inp["scale"])
    torch.cuda.synchronize()
    kd, vd = k.cpu().contiguous(), v.cpu().contiguous()          # the dense tensors the views show
    O_ref, L_ref = attention_fp64(q.cpu().contiguous(), kd, vd, inp["scale"], causal)
    src = dict(q=q.cpu().contiguous(), k=kd, v=vd, scale=inp["scale"], causal=causal)
    compare(o.cpu().contiguous(), lse, O_ref, L_ref, dtype, f"strided {layout}", src=src)
    if check:
        check()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D,dtype", [(128, "bf16"), (64, "fp16")])
def test_qkvpacked(D, dtype, causal):
    inp = ai.make_custom(2, 3, 333, 333, D, dtype, causal, seed=800 + D)
    note(f"qkvpacked D{D} {dtype} causal={causal}")
    qkv = torch.stack([inp[n].transpose(1, 2) for n in ("q", "k", "v")], dim=2).contiguous().to(DEV)  # [B,L,3,H,D]
    o, lse = fa.fa_fwd_qkvpacked(qkv, causal=causal, scale=inp["scale"])
    torch.cuda.synchronize()
    assert tuple(o.shape) == (2, 333, 3, D)
    O_ref, L_ref = attention_fp64(inp["q"], inp["k"], inp["v"], inp["scale"], causal)
    compare(o.transpose(1, 2).cpu().contiguous(), lse, O_ref, L_ref, dtype, "qkvpacked", src=inp)


def test_strided_matches_dense_bitwise():
    # the same values through fa_fwd (dense) and fa_fwd_strided on [B,L,H,D] storage give the same bits
    inp = ai.make_custom(1, 4, 700, 700, 128, "bf16", True, seed=901)
    o1, l1 = run_gpu(inp)
    q, k, v, o, _ = _views("blhd", inp)
    o2, l2 = fa.fa_fwd_strided(q, k, v, o, causal=True, scale=inp["scale"])
    torch.cuda.synchronize()
    assert torch.equal(o1.cpu(), o2.cpu()) and torch.equal(l1.cpu(), l2.cpu())


def test_strided_train_shape_sampled():
    # the 7B 4K training shape in [B, L, H, D] storage, sampled rows against the oracle
    w = ai.WORKLOADS["train7b_4k"]
    inp = ai.make_inputs(w)
    note("strided train7b_4k in [B,L,H,D] storage")
    q, k, v, o, _ = _views("blhd", inp)
    o, lse = fa.fa_fwd(q, k, v, o, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    heads, rows = _sample(w, seed=3)
    O_ref, L_ref = attention_fp64(inp["q"], inp["k"], inp["v"], w.scale, True, rows=rows, heads=heads)
    compare(o.cpu()[:, :, rows], lse.cpu()[:, :, rows], O_ref, L_ref, w.dtype, "strided train", src=inp,
            heads=heads, rows=rows)


# ------------------------------------------------------------------------------------------
# causal with Lq < Lk (bottom-right alignment) and key splits (fa_fwd_splitkv)
# ------------------------------------------------------------------------------------------

BR_CASES = [(1, 2, 1, 1000, 128, "bf16"), (1, 2, 100, 1000, 64, "fp16"), (2, 3, 300, 301, 128, "bf16"),
            (1, 1, 257, 4000, 128, "fp16"), (1, 2, 64, 64, 64, "bf16"), (1, 2, 700, 777, 64, "bf16")]


@pytest.mark.parametrize("B,H,Lq,Lk,D,dtype", BR_CASES,
                         ids=[f"B{b}H{h}_{lq}x{lk}_D{d}_{dt}" for b, h, lq, lk, d, dt in BR_CASES])
def test_causal_bottom_right(B, H, Lq, Lk, D, dtype):
    inp = ai.make_custom(B, H, Lq, Lk, D, dtype, True, seed=30_000 + 7 * Lq + Lk + D)
    note(f"causal bottom-right B{B} H{H} Lq{Lq} Lk{Lk} D{D} {dtype}")
    o, lse = run_gpu(inp)
    O_ref, L_ref = attention_fp64(inp["q"], inp["k"], inp["v"], inp["scale"], True)
    compare(o, lse, O_ref, L_ref, dtype, "bottom-right", src=inp)


SPLIT_CASES = [(1, 2, 300, 300, 128, "bf16", True, 2), (1, 2, 300, 300, 128, "bf16", True, 8),
               (2, 2, 200, 1000, 64, "fp16", False, 3), (1, 2, 100, 2000, 128, "fp16", True, 5),
               (1, 1, 1, 4096, 128, "bf16", False, 16), (1, 3, 513, 513, 64, "bf16", True, 4),
               (1, 2, 130, 65, 128, "fp16", False, 64),
               # few rows, many splits (the per-row merge): D = 64 with 16 lane groups and a split count that
               # is not a multiple of them; 50 splits over 11 key tiles (empty splits), 8 per lane group
               (1, 4, 3, 2000, 64, "bf16", True, 40), (2, 2, 16, 700, 128, "fp16", False, 50)]


@pytest.mark.parametrize("B,H,Lq,Lk,D,dtype,causal,splits", SPLIT_CASES,
                         ids=[f"B{b}H{h}_{lq}x{lk}_D{d}_{dt}_{'c' if c else 'nc'}_s{s}"
                              for b, h, lq, lk, d, dt, c, s in SPLIT_CASES])
def test_splitkv(B, H, Lq, Lk, D, dtype, causal, splits):
    inp = ai.make_custom(B, H, Lq, Lk, D, dtype, causal, seed=40_000 + Lq + Lk + splits)
    note(f"split-KV B{B} H{H} Lq{Lq} Lk{Lk} D{D} {dtype} causal={causal} splits={splits}")
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    o, lse = fa.fa_fwd(q, k, v, causal=causal, scale=inp["scale"], num_splits=splits)
    torch.cuda.synchronize()
    O_ref, L_ref = attention_fp64(inp["q"], inp["k"], inp["v"], inp["scale"], causal)
    compare(o, lse, O_ref, L_ref, dtype, f"split-KV x{splits}", src=inp)
    # the merge reproduces one pass up to fp32 rounding of the combination
    o1, l1 = run_gpu(inp)
    assert (lse.cpu() - l1.cpu()).abs().max().item() <= 1e-4
    assert (o.cpu().double() - o1.cpu().double()).abs().max().item() <= 2 * TOL[dtype]


def test_splitkv_workspace_reuse_and_views():
    # one workspace for two calls in a row (the second smaller), on [B, L, H, D] views
    big = ai.make_custom(2, 4, 600, 600, 128, "bf16", True, seed=41_001)
    small = ai.make_custom(1, 2, 300, 500, 128, "bf16", True, seed=41_002)
    ws = torch.empty(fa.fa_fwd_splitkv_workspace_size(2, 4, 600, 128, 4), dtype=torch.uint8, device=DEV)
    outs = []
    for inp in (big, small):
        q, k, v, o, _ = _views("blhd", inp)
        outs.append(fa.fa_fwd_splitkv(q, k, v, o, causal=True, scale=inp["scale"], num_splits=4, workspace=ws))
    torch.cuda.synchronize()
    for inp, (o, lse) in zip((big, small), outs):
        O_ref, L_ref = attention_fp64(inp["q"], inp["k"], inp["v"], inp["scale"], True)
        compare(o.cpu().contiguous(), lse, O_ref, L_ref, "bf16", "split-KV reuse", src=inp)


def test_splitkv_llama_shape_sampled():
    w = ai.WORKLOADS["llama7b_2k"]
    inp = ai.make_inputs(w)
    splits = 3  # uneven shares: 8..32 key tiles per query tile over 3 splits
    note(f"split-KV llama7b_2k with {splits} splits")
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    o, lse = fa.fa_fwd(q, k, v, causal=True, scale=w.scale, num_splits=splits)
    torch.cuda.synchronize()
    heads, rows = _sample(w, seed=5)
    O_ref, L_ref = attention_fp64(inp["q"], inp["k"], inp["v"], w.scale, True, rows=rows, heads=heads)
    compare(o.cpu()[:, :, rows], lse.cpu()[:, :, rows], O_ref, L_ref, w.dtype, "llama split", src=inp,
            heads=heads, rows=rows)


@pytest.mark.parametrize("name", list(ai.SPLIT_WORKLOADS))
def test_split_workload(name):
    # the split-KV inference shapes as timed (their own split counts), every row against the oracle
    w = ai.SPLIT_WORKLOADS[name]
    inp = ai.make_inputs(w)
    note(f"split workload {name}: {w.description}")
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
    fa.fa_fwd_splitkv(q, k, v, o, lse, causal=w.causal, scale=w.scale, num_splits=w.splits)
    torch.cuda.synchronize()
    O_ref, L_ref = attention_fp64(inp["q"], inp["k"], inp["v"], w.scale, w.causal)
    st = compare(o, lse, O_ref, L_ref, w.dtype, name, src=inp)
    _report(name, dict(st, workload=name, description=w.description, splits=w.splits))


@pytest.mark.parametrize("causal", [False, True])
def test_long_cache_decode(causal):
    # a few query rows over a million keys (ragged), 256 key splits: the rows against the oracle in full
    B, H, Lq, Lk, D = 1, 1, 4, 1_000_003, 128
    inp = ai.make_custom(B, H, Lq, Lk, D, "bf16", causal, seed=170_001)
    splits = fa.suggest_num_splits(B, H, Lq, Lk, D, causal)
    note(f"decode over {Lk} keys, causal={causal}, {splits} splits")
    assert splits == 256
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
    fa.fa_fwd(q, k, v, o, lse, causal=causal, scale=inp["scale"], num_splits=splits)
    o1, l1 = fa.fa_fwd(q, k, v, causal=causal, scale=inp["scale"])
    torch.cuda.synchronize()
    O_ref, L_ref = attention_fp64(inp["q"], inp["k"], inp["v"], inp["scale"], causal)
    compare(o, lse, O_ref, L_ref, "bf16", "long decode split", src=inp)
    compare(o1, l1, O_ref, L_ref, "bf16", "long decode one pass", src=inp)
