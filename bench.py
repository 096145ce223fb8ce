"""Throughput of the fused attention forward pass on one MI355X, as one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload train7b_4k] [--no-cpu-baseline]
    python bench.py --traffic-probe          # for rocprofv3 --pmc runs (see below)
    python bench.py --summarize-traffic DIR  # FETCH_SIZE/WRITE_SIZE CSVs -> profiles/*_traffic.md
    python bench.py --summarize-trace DIR    # kernel-trace stats CSV -> profiles/*_kernel_trace.md
    python bench.py --summarize-counters DIR # SQ counter CSVs -> profiles/*_sq_counters.md
    python bench.py --pass bwd [--workload W] # the backward pass (fa_bwd) instead of the forward
    python bench.py --microbench             # MFMA, v_exp_f32, LDS and HBM rates of this GPU (libfa355_mb.so)

One step = one ``fa_fwd`` call (the whole hot path: one kernel) over the
workload's seeded synthetic Q, K, V, which are resident in HBM before timing
starts.  The metric is attention-forward TFLOP/s with FLOP = 4·B·H·Lq·Lk·D,
halved for causal, and its fraction of MI355X's dense bf16 MFMA peak.  The
split-KV inference shapes (``--workload kvcache_16k`` and the like) step through
``fa_fwd_splitkv`` (main kernel plus merge); those below the ridge point report
an HBM roofline instead.  ``--pass bwd`` times ``fa_bwd`` (the dQ kernel, which
also forms the row statistics, then the dK/dV kernel) with o and lse from ``fa_fwd`` computed before timing and a
seeded upstream gradient; its FLOP are 2.5x the forward's (five products of the
same shape instead of two: the usual count for a recomputing backward pass).

Before the W warm-up steps the step is launched for ``--settle-s`` seconds
(default 1.0; all launches complete before timing starts): measured on MI355X,
this kernel runs ~20% slower for the first ~20 launches after the GPU idles (the
power management lowers the clock while the load ramps, then settles near
2.0 GHz), and a timed region of a few dozen launches would otherwise measure that
transient rather than the kernel.  The shader clock is sampled (amdsmi) while the
timed launches run and reported with the fraction of the MFMA peak at that clock.

Besides the contract fields the line carries:
  * ``roofline``: the kernel's algorithmic FLOP per launch divided by its mean
    launch duration, measured with HIP events recorded on the launch stream
    around every timed launch; ``traffic`` is the HBM bytes per launch from the
    committed rocprofv3 counter summary, reported only while the kernel sources
    still hash to what was profiled (else null), and ``traffic_gbs`` that over
    this run's mean launch time; ``counters``: the fractions of SIMD cycles with
    the matrix cores busy, with VALU issue, with both, and of CU cycles with LDS
    busy, from the committed SQ counter summary under the same hash rule;
  * ``timing``: median, best and mean launch time, the settle phase, the CU
    count and the sampled shader clock;
  * ``cpu_baseline``: the fp64 CPU oracle timed on this host over a bounded
    sample of the same workload (whole heads, every row, one head per worker
    process with single-threaded BLAS), as TFLOP/s-equivalent;
  * ``parity``: every row of four heads of this run's output against the oracle,
    with the parity tests' bar.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16/fp16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
PEAK_HBM_GBS = 8000.0
METRIC = "attention fwd TFLOP/s (bf16 causal, L=4096, D=128) and % of MFMA peak"
_CSRC = os.path.join(ROOT, "tiled_attention_06_amd", "csrc")
# the sources and the build script (its compiler flags shape the machine code)
_BUILD = os.path.join(ROOT, "tiled_attention_06_amd", "build.py")
KERNEL_SOURCES = {"fwd": [os.path.join(_CSRC, f) for f in ("fa_fwd_kernel.hpp", "fa355.hip")] + [_BUILD],
                  "bwd": [os.path.join(_CSRC, f) for f in ("fa_fwd_kernel.hpp", "fa_bwd_kernel.hpp", "fa355.hip")]
                  + [_BUILD]}
TRAFFIC_FILES = {"fwd": os.path.join(ROOT, "profiles", "fa_fwd_kernel_train7b_4k_traffic.md"),
                 "bwd": os.path.join(ROOT, "profiles", "fa_bwd_kernels_train7b_4k_traffic.md")}


def trace_file(workload: str, pass_: str = "fwd") -> str:
    kern = "fa_fwd_kernel" if pass_ == "fwd" else "fa_bwd_kernels"
    return os.path.join(ROOT, "profiles", f"{kern}_{workload}_kernel_trace.md")

COPY_BYTES = 1 << 30  # the plain device copy that calibrates the HBM byte counters
DROP_SEED = 2024      # Philox seed of the dropout runs


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash(pass_: str = "fwd") -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[pass_]:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def committed_traffic(workload: str, pass_: str = "fwd"):
    """HBM bytes per call from the committed counter summary, if it matches the current kernels."""
    path = TRAFFIC_FILES[pass_]
    if workload != "train7b_4k" or not os.path.exists(path):
        return None
    with open(path, encoding="utf-8") as f:
        text = f.read()
    m = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not b or m.group(1) != kernel_source_hash(pass_):
        return None
    return float(b.group(1))


def committed_sq_counters(workload: str):
    """Fractions of SIMD cycles from the committed SQ counter summary, if it matches the current kernels."""
    path = os.path.join(ROOT, "profiles", f"fa_fwd_kernel_{workload}_sq_counters.md")
    if not os.path.exists(path):
        return None
    with open(path, encoding="utf-8") as f:
        text = f.read()
    m = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    if not m or m.group(1) != kernel_source_hash("fwd"):
        return None
    keys = {"mfma_busy": r"MFMA busy, fraction of SIMD cycles\s+([0-9.]+)",
            "valu_issue": r"VALU issue \(both waves\), fraction\s+([0-9.]+)",
            "mfma_valu_overlap": r"MFMA busy while VALU issues \(co-execution\)\s+([0-9.]+)",
            "lds_busy": r"LDS busy \(indexed ops\), fraction of CU\s+([0-9.]+)"}
    out = {}
    for k, rx in keys.items():
        r = re.search(rx, text)
        if not r:
            return None
        out[k] = float(r.group(1))
    out["source"] = os.path.relpath(path, ROOT)
    return out


def _cpu_workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _oracle_head_job(args):
    """One head of the fp64 oracle (forward or gradients), unmodified, with single-threaded BLAS."""
    from threadpoolctl import threadpool_limits

    from oracle import attention_bwd_head_fp64, attention_head_fp64

    kind, q, k, v, d, scale, causal, dropout_p, seed, bh = args
    q, k, v = q.astype("float64"), k.astype("float64"), v.astype("float64")
    with threadpool_limits(1):
        if kind == "fwd":
            attention_head_fp64(q, k, v, scale, causal, dropout_p=dropout_p, seed=seed, bh=bh)
        else:
            attention_bwd_head_fp64(q, k, v, d.astype("float64"), scale, causal)
    return bh


def _cpu_baseline(inp, kind: str, flops_per_head: float, budget_s: float, dropout_p: float = 0.0,
                  do=None) -> dict:
    """The oracle over whole heads of the workload, one head per worker process, for about budget_s."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor

    w = inp["workload"]
    q, k, v = (inp[n].float().numpy() for n in ("q", "k", "v"))
    d = do.float().numpy() if do is not None else None
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    job = lambda b, h: (kind, q[b, h], k[b, h], v[b, h], None if d is None else d[b, h], w.scale, w.causal,
                        dropout_p, DROP_SEED, b * w.H + h)
    n = _cpu_workers()
    # one head alone first (its time sizes the sample), then whole rounds of n heads in parallel
    t0 = time.perf_counter()
    _oracle_head_job(job(*heads[0]))
    t1 = time.perf_counter() - t0
    rounds = max(1, min(len(heads) // n, int(budget_s / max(t1, 1e-3))))
    sample = heads[1 : 1 + rounds * n] or heads[:1]
    with ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn")) as ex:
        list(ex.map(_oracle_head_job, [job(*heads[0])] * n, timeout=600))   # start the workers untimed
        t0 = time.perf_counter()
        list(ex.map(_oracle_head_job, [job(b, h) for b, h in sample], timeout=1200))
        dt = time.perf_counter() - t0
    what = "forward" if kind == "fwd" else "dQ, dK, dV"
    return {"value": round(flops_per_head * len(sample) / dt / 1e12, 6), "unit": "TFLOP/s", "cores": n,
            "kind": "oracle",
            "sample": f"{len(sample)} of {len(heads)} heads of {w.name} ({what}, all {w.Lq} rows each), fp64 numpy "
                      f"oracle unmodified, one head per process on {n} worker processes (single-threaded BLAS), "
                      f"{dt:.1f} s wall; one head alone took {t1:.2f} s"}


def cpu_baseline(inp, budget_s: float = 15.0, dropout_p: float = 0.0) -> dict:
    w = inp["workload"]
    return _cpu_baseline(inp, "fwd", w.flops / (w.B * w.H), budget_s, dropout_p)


def cpu_baseline_bwd(inp, do, budget_s: float = 15.0) -> dict:
    w = inp["workload"]
    return _cpu_baseline(inp, "bwd", 2.5 * w.flops / (w.B * w.H), budget_s, do=do)


def sampled_parity_bwd(inp, do, grads, dropout_p: float = 0.0) -> dict:
    """Two whole heads of dQ, dK, dV against the fp64 gradient oracle, with the parity tests' bar:
    max error <= tol·max|ref| after the rounding-of-O terms of numerics.delta_bounds."""
    import numpy as np

    from numerics import delta_bounds
    from oracle import attention_bwd_fp64, attention_fp64

    w = inp["workload"]
    heads = [(0, 0), (w.B - 1, w.H - 1)]
    ref = attention_bwd_fp64(inp["q"], inp["k"], inp["v"], do, w.scale, w.causal, heads=heads,
                             dropout_p=dropout_p, seed=DROP_SEED)
    O_ref, L_ref = attention_fp64(inp["q"], inp["k"], inp["v"], w.scale, w.causal, heads=heads,
                                  dropout_p=dropout_p, seed=DROP_SEED)
    extra = delta_bounds(inp["q"], inp["k"], do, O_ref, L_ref, w.scale, w.causal, w.dtype, heads)
    tol = 2e-3 if w.dtype == "fp16" else 1e-2
    worst, worst_raw = 0.0, 0.0
    for t, (g, r) in enumerate(zip(grads, ref)):
        gc = g.double().cpu().numpy()
        for b, h in heads:
            err = np.abs(gc[b, h] - r[b, h])
            mx = np.abs(r[b, h]).max()
            worst_raw = max(worst_raw, float(err.max() / mx))
            if t < 2:
                err = np.maximum(err - extra[(b, h)][t], 0.0)
            worst = max(worst, float(err.max() / mx))
    return {"heads_checked": len(heads), "max_err_over_max_ref": worst, "raw_max_err_over_max_ref": worst_raw,
            "tol": tol, "pass": bool(worst <= tol)}


def sampled_parity(inp, o, lse, dropout_p: float = 0.0) -> dict:
    """Every row of four heads (the first, the last and two drawn ones) against the fp64 oracle, with the
    parity tests' bar: |O − O_ref| <= tol, or, only where the output format is coarser than tol, its
    rounding plus the bound of the kernel's weight rounding (numerics.fwd_allowance); LSE within 1e-3."""
    import numpy as np

    from numerics import fwd_allowance, round_to_dtype
    from numerics.bounds import fwd_check
    from oracle import attention_fp64
    from oracle.philox import dropout_keep, keep_threshold

    w = inp["workload"]
    r = np.random.default_rng(1)
    heads = [(0, 0), (w.B - 1, w.H - 1)]
    while len(set(heads)) < min(4, w.B * w.H):
        heads.append((int(r.integers(w.B)), int(r.integers(w.H))))
    heads = sorted(set(heads))
    O_ref, L_ref = attention_fp64(inp["q"], inp["k"], inp["v"], w.scale, w.causal, heads=heads,
                                  dropout_p=dropout_p, seed=DROP_SEED)
    oc, lc = o.double().cpu().numpy(), lse.double().cpu().numpy()
    tol = 2e-3 if w.dtype == "fp16" else 1e-2
    out = {"heads_checked": len(heads), "rows_checked": int(len(heads) * w.Lq), "max_abs_err_o": 0.0,
           "max_abs_err_lse": 0.0, "o_rounding_floor": 0.0, "n_over_tol": 0, "n_explained_by_format": 0,
           "tol_o": tol, "tol_lse": 1e-3, "pass": True}
    for b, h in heads:
        qh, kh, vh = (inp[n][b, h].double().numpy() for n in ("q", "k", "v"))

        def allowance(idx, b=b, h=h, qh=qh, kh=kh, vh=vh):
            keep = dropout_keep(b * w.H + h, idx, np.arange(w.Lk), dropout_p, DROP_SEED) if dropout_p else None
            return fwd_allowance(qh, kh, vh, O_ref[b, h][idx], w.scale, w.causal, w.dtype, idx, keep=keep,
                                 keep_scale=256.0 / keep_threshold(dropout_p) if dropout_p else 1.0)
        ok, info = fwd_check(oc[b, h], O_ref[b, h], w.dtype, tol, allowance)
        el = float(np.abs(lc[b, h] - L_ref[b, h]).max())
        out["max_abs_err_o"] = max(out["max_abs_err_o"], info["max_abs_err"])
        out["max_abs_err_lse"] = max(out["max_abs_err_lse"], el)
        out["o_rounding_floor"] = max(out["o_rounding_floor"],
                                      float(np.abs(round_to_dtype(O_ref[b, h], w.dtype) - O_ref[b, h]).max()))
        out["n_over_tol"] += info["n_over_tol"]
        out["n_explained_by_format"] += info["n_allowed"]
        out["pass"] = bool(out["pass"] and ok and el <= 1e-3)
    return out


def traffic_probe(w, steps: int, pass_: str = "fwd") -> None:
    """One plain device copy of COPY_BYTES (the counter calibration), then `steps` calls of fa_fwd (or, for
    pass_ == "bwd", one fa_fwd and then `steps` calls of fa_bwd)."""
    import torch

    import attn_inputs
    import tiled_attention_06_amd as fa

    dev = torch.device("cuda:0")
    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)  # a fill: writes COPY_BYTES
    dst = torch.empty_like(src)
    torch.cuda.synchronize(dev)
    torch.neg(src, out=dst)  # an elementwise kernel: reads and writes COPY_BYTES
    torch.cuda.synchronize(dev)
    del src, dst
    inp = attn_inputs.make_inputs(w)
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    if pass_ == "bwd":
        do = attn_inputs.make_dout((w.B, w.H, w.Lq, w.D), w.dtype, seed=w.seed + 100).to(dev)
        fa.fa_fwd(q, k, v, o, lse, causal=w.causal, scale=w.scale)
        grads = tuple(torch.empty_like(t) for t in (q, k, v))
        ws = torch.empty(fa.fa_bwd_workspace_size(w.B, w.H, w.Lq), dtype=torch.uint8, device=dev)
        for _ in range(steps):
            fa.fa_bwd(q, k, v, o, do, lse, *grads, causal=w.causal, scale=w.scale, workspace=ws)
    else:
        for _ in range(steps):
            fa.fa_fwd(q, k, v, o, lse, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize(dev)
    log(f"traffic probe: 1 copy of {COPY_BYTES} B, {steps} calls of fa_{pass_} on {w.name}")


def _csv_rows(directory: str, name: str):
    import csv
    import glob

    rows = []
    for path in sorted(glob.glob(os.path.join(directory, "**", name), recursive=True)):
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def summarize_traffic(directory: str, w, pass_: str = "fwd") -> str:
    """Scale FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the pass's kernels by the copy kernel's reading."""
    rows = _csv_rows(directory, "*counter_collection.csv")
    per = {}
    for r in rows:
        per.setdefault((r["Kernel_Name"], r["Dispatch_Id"]), {})[r["Counter_Name"]] = float(r["Counter_Value"])
    ours = ("fa_fwd_kernel",) if pass_ == "fwd" else ("fa_bwd_dq_kernel", "fa_bwd_dkdv")  # dkdv2 at D = 128
    mine = {name: [c for (kn, _), c in per.items() if name in kn] for name in ours}
    if not all(mine.values()):
        raise SystemExit(f"no dispatches of {[n for n, c in mine.items() if not c]} in the counter CSVs")
    # Calibration dispatches: the fill and the elementwise kernel each write
    # COPY_BYTES, and only the elementwise kernel also reads COPY_BYTES.
    other = [c for (kn, _), c in per.items() if "fa355" not in kn]
    half_kib = COPY_BYTES / 2 / 1024
    cf = [c["FETCH_SIZE"] for c in other if c.get("FETCH_SIZE", 0) > half_kib]
    cw = [c["WRITE_SIZE"] for c in other if c.get("WRITE_SIZE", 0) > half_kib]
    if not (cf and cw):
        raise SystemExit("need FETCH_SIZE and WRITE_SIZE for the copy")
    kf = COPY_BYTES / (sum(cf) / len(cf) * 1024)   # true bytes per counted byte, reads
    kw = COPY_BYTES / (sum(cw) / len(cw) * 1024)   # and writes
    detail, fetch, write = [], 0.0, 0.0
    for name, cs in mine.items():
        ff = [c["FETCH_SIZE"] for c in cs if "FETCH_SIZE" in c]
        fw = [c["WRITE_SIZE"] for c in cs if "WRITE_SIZE" in c]
        if not (ff and fw):
            raise SystemExit(f"need FETCH_SIZE and WRITE_SIZE for {name}")
        f_, w_ = sum(ff) / len(ff) * 1024 * kf, sum(fw) / len(fw) * 1024 * kw
        fetch, write = fetch + f_, write + w_
        detail.append(f"{name}: FETCH_SIZE {sum(ff) / len(ff):.1f} KiB, WRITE_SIZE {sum(fw) / len(fw):.1f} KiB per "
                      f"dispatch -> read {f_:.4g} B, write {w_:.4g} B")
    bhd = w.B * w.H * w.D
    if pass_ == "fwd":
        alg = w.hbm_bytes
        alg_what = "Q, K, V read once, O and LSE written once"
    else:
        alg = 2 * (3 * bhd * w.Lq + 2 * bhd * w.Lk) + 2 * (bhd * w.Lq + 2 * bhd * w.Lk) + 4 * w.B * w.H * w.Lq
        alg_what = "Q, O, dO, K, V and LSE read once, dQ, dK, dV written once"
    probe = "--traffic-probe" if pass_ == "fwd" else "--pass bwd --traffic-probe"
    lines = [
        f"# HBM traffic of {' + '.join(ours)} on {w.name} ({w.description})",
        "",
        f"Counters from two `rocprofv3 --pmc` runs of `bench.py {probe}`: a fill of",
        f"{COPY_BYTES} bytes, a plain elementwise copy of {COPY_BYTES} bytes to another buffer, then",
        f"calls of fa_{pass_}.  Values are KiB per dispatch.  Each counter is scaled by",
        "the calibration kernels' true bytes / counted bytes.",
        "",
        "Commands (from the repository root on the GPU box):",
        "",
        f"    rocprofv3 --pmc FETCH_SIZE --output-format csv -d {directory}/traffic_fetch -o t -- python3 bench.py {probe}",
        f"    rocprofv3 --pmc WRITE_SIZE --output-format csv -d {directory}/traffic_write -o t -- python3 bench.py {probe}",
        f"    python3 bench.py{' --pass bwd' if pass_ == 'bwd' else ''} --summarize-traffic {directory}  (reads both; "
        "nothing else under that directory)",
        "",
        f"calibration: FETCH_SIZE {sum(cf) / len(cf):.1f} KiB (mean of {len(cf)}), WRITE_SIZE "
        f"{sum(cw) / len(cw):.1f} KiB (mean of {len(cw)}) for {COPY_BYTES / 1024:.0f} KiB moved -> "
        f"read factor {kf:.4f}, write factor {kw:.4f}",
        *detail,
        f"scaled: read {fetch:.4g} B, write {write:.4g} B per call",
        f"algorithmic bytes per call ({alg_what}): {alg}",
        f"traffic / algorithmic: {(fetch + write) / alg:.3f}",
        "",
        f"kernel_source_sha256: {kernel_source_hash(pass_)}",
        f"hbm_bytes_per_launch: {fetch + write:.6g}",
        "",
    ]
    return "\n".join(lines)


# Shader-sequencer counters of the forward kernel, three rocprofv3 --pmc runs of
# `bench.py --traffic-probe` (at most 8 SQ counters per run).
SQ_PASSES = (
    "SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY SQ_ACTIVE_INST_VALU "
    "SQ_ACTIVE_INST_LDS SQ_WAIT_INST_LDS GRBM_GUI_ACTIVE",
    "SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES SQ_BUSY_CU_CYCLES SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT "
    "SQ_LDS_IDX_ACTIVE SQ_ACTIVE_INST_MISC SQ_ACTIVE_INST_VALU2 GRBM_GUI_ACTIVE",
    "SQ_THREAD_CYCLES_VALU SQ_INSTS_VALU SQ_INSTS_MFMA SQ_LDS_DATA_FIFO_FULL SQ_LDS_CMD_FIFO_FULL "
    "SQ_LDS_ADDR_CONFLICT SQ_ACTIVE_INST_SCA SQ_INSTS_SALU GRBM_GUI_ACTIVE",
)
N_CU, N_SIMD, N_XCC = 256, 1024, 8


def summarize_counters(directory: str, w) -> str:
    """Mean per fa_fwd_kernel dispatch of the SQ counters, and what they say about the SIMDs' time."""
    rows = _csv_rows(directory, "*counter_collection.csv")
    per = {}
    dur = {}
    for r in rows:
        if "fa_fwd_kernel" not in r["Kernel_Name"]:
            continue
        key = (r["Agent_Id"], r["Dispatch_Id"], r["Process_Id"])
        per.setdefault(r["Counter_Name"], {})[key] = float(r["Counter_Value"])
        dur[key] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    need = [c for p_ in SQ_PASSES for c in p_.split()]
    missing = [c for c in need if c not in per]
    if missing:
        raise SystemExit(f"counters missing for fa_fwd_kernel: {missing}")
    m = {c: sum(v.values()) / len(v) for c, v in per.items()}
    secs = sum(dur.values()) / len(dur)
    cyc = m["GRBM_GUI_ACTIVE"] / N_XCC              # GPU cycles per dispatch (summed over the XCDs)
    waves = 2 * N_SIMD                              # wave slots in use: two waves per SIMD
    q = 4.0                                         # "quad-cycle" counters count units of 4 cycles
    mfma = m["SQ_VALU_MFMA_BUSY_CYCLES"] / N_SIMD / cyc
    valu = m["SQ_ACTIVE_INST_VALU"] * q / N_SIMD / cyc
    coex = m["SQ_VALU_MFMA_COEXEC_CYCLES"] / N_SIMD / cyc
    resident = m["SQ_WAVE_CYCLES"] * q / waves / cyc
    act = m["SQ_ACTIVE_INST_ANY"] * q / waves / cyc
    wait = m["SQ_WAIT_ANY"] * q / waves / cyc
    wait_issue = m["SQ_WAIT_INST_ANY"] * q / waves / cyc
    lds = m["SQ_LDS_IDX_ACTIVE"] / N_CU / cyc
    n_mfma = m["SQ_INSTS_MFMA"]
    mfma_flop = n_mfma * 2 * 32 * 32 * 16
    lines = [
        f"# SQ counters: fa_fwd_kernel on {w.name} ({w.description})",
        "",
        "Three `rocprofv3 --pmc` runs of `bench.py --traffic-probe` (a copy, then 3 calls of fa_fwd), one per",
        "counter set; the values below are means over the fa_fwd_kernel dispatches.  Commands (from the",
        "repository root on the GPU box; rocprofv3 collects at most 8 SQ counters per run):",
        "",
    ]
    for i, p_ in enumerate(SQ_PASSES):
        lines.append(f"    rocprofv3 --pmc {p_} --output-format csv -d {directory}/sq{i} -o sq -- python3 bench.py "
                     "--traffic-probe")
    lines += [
        f"    python3 bench.py --summarize-counters {directory}  (reads the three directories)",
        "",
        "Raw means per dispatch:",
        "",
        *[f"    {c:28s} {m[c]:.6g}" for c in sorted(set(need))],
        "",
        f"Derived (MI355X: {N_CU} CUs, {N_SIMD} SIMDs, {N_XCC} XCDs; GRBM_GUI_ACTIVE counts per XCD; the kernel runs",
        "two waves per SIMD; SQ_ACTIVE_*, SQ_WAIT_* and SQ_WAVE_CYCLES count quad-cycles per wave):",
        "",
        f"    dispatch duration                          {secs * 1e6:.1f} us (counter runs, 3 cold calls)",
        f"    GPU cycles per dispatch                    {cyc:.4g}  -> shader clock {cyc / secs / 1e9:.2f} GHz",
        f"    MFMA instructions per dispatch             {n_mfma:.5g} (v_mfma_f32_32x32x16: {mfma_flop:.4g} flop;"
        f" metric FLOP {w.flops:.4g}, ratio {mfma_flop / w.flops:.3f})",
        f"    MFMA busy, fraction of SIMD cycles         {mfma:.3f}",
        f"    VALU issue (both waves), fraction          {valu:.3f}",
        f"    MFMA busy while VALU issues (co-execution) {coex:.3f}",
        f"    neither (1 - MFMA - VALU + co-execution)   {max(0.0, 1 - mfma - valu + coex):.3f}",
        f"    non-MFMA VALU instructions per MFMA        {(m['SQ_INSTS_VALU'] - n_mfma) / n_mfma:.2f}",
        f"    LDS instructions per MFMA                  {m['SQ_INSTS_LDS'] / n_mfma:.2f}",
        f"    LDS busy (indexed ops), fraction of CU     {lds:.3f}; bank conflicts {m['SQ_LDS_BANK_CONFLICT']:.0f}",
        f"    wave slots occupied                        {resident:.3f}",
        f"    per resident wave: issuing {act / resident:.3f}, waiting (waitcnt/barrier) {wait / resident:.3f}, "
        f"ready but not issued {wait_issue / resident:.3f}",
        "",
        f"kernel_source_sha256: {kernel_source_hash('fwd')}",
        "",
    ]
    return "\n".join(lines)


def summarize_trace(directory: str, w, bench_line: str | None, pass_: str = "fwd") -> str:
    rows = _csv_rows(directory, "*kernel_stats.csv")
    if not rows:
        raise SystemExit("no kernel_stats.csv under " + directory)
    keep = [r for r in rows if "fa_" in r.get("Name", "") and "fa355" in r.get("Name", "")]
    hdr = list(rows[0].keys())
    wl = "" if w.name == "train7b_4k" else f" --workload {w.name}"
    if pass_ == "bwd":
        wl += " --pass bwd"
    run_args = wl
    if bench_line:
        j = json.loads(bench_line)
        if (j.get("steps"), j.get("warmup")) != (200, 500):
            run_args += f" --steps {j['steps']} --warmup {j['warmup']}"
    what = "fa_fwd_kernel" if pass_ == "fwd" else "the fa_bwd kernels"
    lines = [
        f"# rocprofv3 kernel trace: {what} on {w.name} ({w.description})",
        "",
        "Command (from the repository root on the GPU box):",
        "",
        f"    rocprofv3 --kernel-trace --stats --output-format csv -d {directory} -o t -- python3 bench.py{run_args} --no-cpu-baseline --no-parity",
        f"    python3 bench.py{wl} --summarize-trace {directory} --bench-log <that run's stdout>",
        "",
        "(fa_fwd_kernel rows in a backward trace are the one forward call that makes o and lse.)" if pass_ == "bwd"
        else "",
        "",
        "kernel_stats.csv rows for the kernel (durations in ns):",
        "",
        "| " + " | ".join(hdr) + " |",
        "|" + "---|" * len(hdr),
    ]
    lines += ["| " + " | ".join(str(r[h]) for h in hdr) + " |" for r in keep]
    if bench_line:
        lines += ["", "bench.py JSON line of the same profiled run:", "", "    " + bench_line.strip()]
    lines += ["", f"kernel_source_sha256: {kernel_source_hash(pass_)}", ""]
    return "\n".join(lines)


def _clock_reader():
    """A function returning the shader clock (MHz, mean over the XCDs) of the GPU torch uses, from amdsmi,
    or None when amdsmi is unavailable.  The driver refreshes these readings every few hundred ms, so
    samples over a short region are few and approximate."""
    try:
        import amdsmi
        import torch

        amdsmi.amdsmi_init()
        handles = amdsmi.amdsmi_get_processor_handles()
        h = handles[0] if len(handles) == 1 else None
        if h is None:
            bus = getattr(torch.cuda.get_device_properties(0), "pci_bus_id", None)
            for cand in handles:
                bdf = str(amdsmi.amdsmi_get_gpu_device_bdf(cand)).lower()
                if bus is not None and bdf.split(":")[1:2] == [f"{int(bus):02x}"]:
                    h = cand
                    break
        if h is None:
            return None
    except Exception:
        return None

    def read():
        try:
            m = amdsmi.amdsmi_get_gpu_metrics_info(h)
            c = [float(x) for x in (m.get("current_gfxclks") or []) if isinstance(x, (int, float)) and 0 < x < 10000]
            if c:
                return sum(c) / len(c)
            c = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX).get("clk")
            return float(c) if isinstance(c, (int, float)) else None
        except Exception:
            return None
    return read


def run_timed(step, stream, steps: int, warmup: int, settle_s: float) -> dict:
    """Settle (launches for settle_s seconds), W warm-up steps, then K timed steps with a HIP event pair on
    the launch stream around each.  Returns the wall time of the K steps, per-step event times and clock
    samples taken by a thread while the timed launches run."""
    import threading

    import torch

    dev = stream.device
    clk = _clock_reader()
    clocks = {"idle": clk() if clk else None}
    t0 = time.perf_counter()
    n_settle = 0
    while settle_s > 0:
        for _ in range(10):
            step()
        n_settle += 10
        torch.cuda.synchronize(dev)
        if time.perf_counter() - t0 >= settle_s:
            break
    settle_wall = time.perf_counter() - t0
    clocks["after_settle"] = clk() if clk else None
    for _ in range(warmup):
        step()
    torch.cuda.synchronize(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    samples, stop = [], threading.Event()

    def poll():
        while not stop.is_set():
            c = clk()
            if c is not None:
                samples.append(c)
            stop.wait(0.005)

    th = threading.Thread(target=poll, daemon=True) if clk else None
    torch.cuda.synchronize(dev)
    if th:
        th.start()
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    stop.set()
    if th:
        th.join()
    clocks["after"] = clk() if clk else None
    ms = [a.elapsed_time(b) for a, b in ev]
    srt = sorted(ms)
    timing = {"mean_launch_us": round(sum(ms) / len(ms) * 1e3, 3), "median_launch_us": round(srt[len(srt) // 2] * 1e3, 3),
              "best_launch_us": round(srt[0] * 1e3, 3), "worst_launch_us": round(srt[-1] * 1e3, 3),
              "settle_s": round(settle_wall, 3), "settle_launches": n_settle,
              "cu_count": int(torch.cuda.get_device_properties(dev).multi_processor_count),
              "sclk_mhz": {**{k: (round(v) if v else None) for k, v in clocks.items()},
                           "timed_mean": round(sum(samples) / len(samples)) if samples else None,
                           "timed_min": round(min(samples)) if samples else None,
                           "timed_max": round(max(samples)) if samples else None,
                           "timed_samples": len(samples),
                           "source": ("amdsmi current_gfxclks, mean over the XCDs; the driver refreshes it about "
                                      "once a second, so after_settle and the timed samples show the clock the "
                                      "settle phase's load brought the GPU to")}}
    return {"wall": wall, "ms": ms, "timing": timing}


def at_clock(timing: dict, achieved_tflops: float) -> None:
    """Add the MFMA peak at the sampled shader clock and the fraction of it reached (in place)."""
    c = timing["sclk_mhz"].get("timed_mean") or timing["sclk_mhz"].get("after_settle")
    if c:
        peak = PEAK_BF16_TFLOPS * c / 2400.0
        timing["peak_at_clock_tflops"] = round(peak, 1)
        timing["frac_of_peak_at_clock"] = round(achieved_tflops / peak, 4)


def microbench(settle_s: float = 0.5) -> dict:
    """The units' rates on this GPU (libfa355_mb.so): bf16 MFMA, v_exp_f32, LDS reads, HBM copy.

    Each kernel is launched for settle_s seconds, then five launches of ~3-11 ms are timed with HIP events on
    the stream (the best is reported).  The MFMA, exp and LDS kernels measure the shader clock themselves (cycle
    counter against the 100 MHz real-time counter over a workgroup's lifetime); rates per CU and clock use it."""
    import ctypes

    import torch

    path = os.path.join(ROOT, "tiled_attention_06_amd", "libfa355_mb.so")
    if not os.path.exists(path):
        raise SystemExit(f"{path} missing: build with python tiled_attention_06_amd/build.py")
    lib = ctypes.CDLL(path)
    vp, i = ctypes.c_void_p, ctypes.c_int
    for name in ("mb_mfma", "mb_exp", "mb_lds"):
        getattr(lib, name).argtypes = [vp, vp, i, i, vp, vp]
        getattr(lib, name).restype = i
    lib.mb_copy.argtypes = [vp, vp, ctypes.c_size_t, i, vp]
    lib.mb_copy.restype = i
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    cu = torch.cuda.get_device_properties(dev).multi_processor_count
    g = torch.Generator(device="cpu").manual_seed(5)
    ops = (torch.randn(256 * 8, generator=g) * 0.5).to(torch.bfloat16).to(dev)          # 256 x 16 B of bf16
    fsrc = torch.rand(256, generator=g).to(dev)
    lsrc = torch.randint(0, 2 ** 31, (8192 * 4,), generator=g, dtype=torch.int32).to(dev)
    nbytes = 1 << 30
    csrc = torch.randint(0, 2 ** 31, (nbytes // 4,), dtype=torch.int32, device=dev)
    cdst = torch.empty_like(csrc)
    out = torch.empty(1024 * 512, dtype=torch.float32, device=dev)
    cyc = torch.zeros(2, dtype=torch.int64, device=dev)   # shader cycles, 100 MHz ticks (kernels that measure)

    def timed(launch, work, unit, per, measures_clock=True):
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < settle_s:
            for _ in range(4):
                assert launch() == 0
            torch.cuda.synchronize(dev)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
        mhzs = []
        for a, b in ev:
            a.record(stream)
            assert launch() == 0
            b.record(stream)
            if measures_clock:
                torch.cuda.synchronize(dev)
                c, t = (int(x) for x in cyc.tolist())
                if t > 0:
                    mhzs.append(100.0 * c / t)
        torch.cuda.synchronize(dev)
        sec = min(a.elapsed_time(b) for a, b in ev) / 1e3
        mhz = sum(mhzs) / len(mhzs) if mhzs else None
        rate = work / sec
        r = {"rate": round(rate / per, 3), "unit": unit, "best_launch_ms": round(sec * 1e3, 3),
             "sclk_mhz": round(mhz) if mhz else None}
        if mhz:
            r["per_cu_per_clock"] = round(rate / (cu * mhz * 1e6), 3)
        return r

    s_ = stream.cuda_stream
    res = {"cu_count": cu}
    it = 40000
    cp = cyc.data_ptr()
    res["mfma_bf16"] = timed(lambda: lib.mb_mfma(ops.data_ptr(), out.data_ptr(), 2 * cu, it, cp, s_),
                             2 * cu * 4 * it * 8 * 2 * 32 * 32 * 16, "TFLOP/s", 1e12)
    res["mfma_bf16"]["frac_of_spec_peak"] = round(res["mfma_bf16"]["rate"] / PEAK_BF16_TFLOPS, 4)
    if res["mfma_bf16"].get("sclk_mhz"):
        res["mfma_bf16"]["frac_of_peak_at_clock"] = round(
            res["mfma_bf16"]["rate"] / (PEAK_BF16_TFLOPS * res["mfma_bf16"]["sclk_mhz"] / 2400.0), 4)
    it = 20000
    res["v_exp_f32"] = timed(lambda: lib.mb_exp(fsrc.data_ptr(), out.data_ptr(), 4 * cu, it, cp, s_),
                             4 * cu * 256 * it * 8, "G exp/s", 1e9)
    res["lds_read_b128"] = timed(lambda: lib.mb_lds(lsrc.data_ptr(), out.data_ptr(), cu, it, cp, s_),
                                 cu * 8 * it * 8 * 1024, "TB/s", 1e12)
    res["hbm_copy"] = timed(lambda: lib.mb_copy(csrc.data_ptr(), cdst.data_ptr(), nbytes, 16 * cu, s_),
                            2 * nbytes, "GB/s", 1e9, measures_clock=False)
    res["hbm_copy"]["frac_of_spec_peak"] = round(res["hbm_copy"]["rate"] / PEAK_HBM_GBS, 4)
    assert torch.equal(csrc, cdst), "copy kernel result differs"
    return res


def bench_bwd(args, w) -> int:
    import torch

    import attn_inputs
    import tiled_attention_06_amd as fa

    log(f"bench bwd: {w.description}; generating inputs (seed {w.seed}, dO seed {w.seed + 100})")
    inp = attn_inputs.make_inputs(w)
    do_cpu = attn_inputs.make_dout((w.B, w.H, w.Lq, w.D), w.dtype, seed=w.seed + 100)
    dev = torch.device("cuda:0")
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    do = do_cpu.to(dev)
    o, lse = fa.fa_fwd(q, k, v, causal=w.causal, scale=w.scale, dropout_p=args.dropout, seed=DROP_SEED)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.fa_bwd_workspace_size(w.B, w.H, w.Lq), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, causal=w.causal, scale=w.scale, workspace=ws, stream=stream,
                  dropout_p=args.dropout, seed=DROP_SEED)

    res = run_timed(step, stream, args.steps, args.warmup, args.settle_s)
    wall = res["wall"]
    flops = 2.5 * w.flops
    step_ms = res["ms"]
    mean_s = sum(step_ms) / len(step_ms) / 1e3
    value = flops * args.steps / wall / 1e12
    achieved = flops / mean_s / 1e12
    log(f"bench bwd: {args.steps} steps in {wall * 1e3:.2f} ms; step mean {mean_s * 1e6:.1f} us; "
        f"{achieved:.1f} TFLOP/s = {100 * achieved / PEAK_BF16_TFLOPS:.2f}% of peak")
    out = {
        "metric": f"attention bwd TFLOP/s ({w.description}{f', dropout {args.dropout}' if args.dropout else ''})",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "pass": "bwd", "B": w.B, "H": w.H, "Lq": w.Lq, "Lk": w.Lk, "D": w.D,
                   "causal": w.causal, "scale": w.scale, "seed": w.seed, "dout_seed": w.seed + 100,
                   "flop_per_step": flops, "dropout_p": args.dropout},
        "pct_of_mfma_peak": round(100 * value / PEAK_BF16_TFLOPS, 3),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 5),
                     "traffic": committed_traffic(w.name, "bwd") if not args.dropout else None,
                     "kernel": "fa_bwd_dq_kernel + fa_bwd_dkdv2_kernel (fa_bwd_dkdv_kernel at D = 64; the events bracket both)", "mean_launch_us": round(mean_s * 1e6, 3)},
        "timing": res["timing"],
    }
    at_clock(out["timing"], achieved)
    if not args.no_parity:
        out["parity"] = sampled_parity_bwd(inp, do_cpu, (dq, dk, dv), dropout_p=args.dropout)
        log(f"bench bwd: parity {out['parity']}")
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_bwd(inp, do_cpu)
        log(f"bench bwd: cpu baseline {out['cpu_baseline']}")
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--settle-s", type=float, default=1.0,
                    help="seconds of launches before the warm-up steps (clock and power settle); 0 to skip")
    ap.add_argument("--workload", default="train7b_4k",
                    help="a name from attn_inputs.WORKLOADS or attn_inputs.SPLIT_WORKLOADS")
    ap.add_argument("--pass", dest="pass_", choices=["fwd", "bwd"], default="fwd",
                    help="fwd: fa_fwd (the default line); bwd: fa_bwd")
    ap.add_argument("--dropout", type=float, default=0.0,
                    help="dropout probability (fa_fwd_dropout / fa_bwd_dropout, seed 2024)")
    ap.add_argument("--splits", type=int, default=None,
                    help="key splits (fa_fwd_splitkv when > 1); default: the workload's own")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--traffic-probe", action="store_true")
    ap.add_argument("--summarize-traffic", metavar="DIR")
    ap.add_argument("--summarize-trace", metavar="DIR")
    ap.add_argument("--summarize-counters", metavar="DIR", help="SQ counter CSVs -> profiles/*_sq_counters.md")
    ap.add_argument("--bench-log", metavar="FILE", help="bench JSON line to quote in the trace summary")
    ap.add_argument("--microbench", action="store_true",
                    help="rates of the units on this GPU (MFMA, v_exp_f32, LDS, HBM copy) as one JSON line")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the attention forward pass runs on a single MI355X "
              f"(requested --gpus {args.gpus}, WORLD_SIZE={world}). Run with --gpus 1.", file=sys.stderr)
        return 2

    import attn_inputs

    w = attn_inputs.ALL_WORKLOADS[args.workload]
    if args.summarize_traffic:
        text = summarize_traffic(args.summarize_traffic, w, args.pass_)
        with open(TRAFFIC_FILES[args.pass_], "w", encoding="utf-8") as f:
            f.write(text)
        print(text)
        return 0
    if args.summarize_counters:
        text = summarize_counters(args.summarize_counters, w)
        with open(os.path.join(ROOT, "profiles", f"fa_fwd_kernel_{w.name}_sq_counters.md"), "w",
                  encoding="utf-8") as f:
            f.write(text)
        print(text)
        return 0
    if args.summarize_trace:
        line = None
        if args.bench_log and os.path.exists(args.bench_log):
            with open(args.bench_log, encoding="utf-8") as f:
                line = next((x for x in f if x.startswith("{")), None)
        text = summarize_trace(args.summarize_trace, w, line, args.pass_)
        with open(trace_file(w.name, args.pass_), "w", encoding="utf-8") as f:
            f.write(text)
        print(text)
        return 0

    import torch

    import tiled_attention_06_amd as fa

    if args.traffic_probe:
        traffic_probe(w, steps=3, pass_=args.pass_)
        return 0
    if args.microbench:
        print(json.dumps({"microbench": microbench()}), flush=True)
        return 0
    if args.pass_ == "bwd":
        return bench_bwd(args, w)
    log(f"bench: {w.description}; generating inputs (seed {w.seed})")
    inp = attn_inputs.make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    splits = w.splits if args.splits is None else args.splits
    if splits > 1:
        ws = torch.empty(fa.fa_fwd_splitkv_workspace_size(w.B, w.H, w.Lq, w.D, splits), dtype=torch.uint8,
                         device=dev)

        def step():
            fa.fa_fwd_splitkv(q, k, v, o, lse, causal=w.causal, scale=w.scale, num_splits=splits, workspace=ws,
                              stream=stream)
    elif args.dropout:
        def step():
            fa.fa_fwd_dropout(q, k, v, o, lse, causal=w.causal, scale=w.scale, dropout_p=args.dropout,
                              seed=DROP_SEED, stream=stream)
    else:
        def step():
            fa.fa_fwd(q, k, v, o, lse, causal=w.causal, scale=w.scale, stream=stream)

    res = run_timed(step, stream, args.steps, args.warmup, args.settle_s)
    wall = res["wall"]
    kernel_ms = res["ms"]
    mean_kernel_s = sum(kernel_ms) / len(kernel_ms) / 1e3
    value = w.flops * args.steps / wall / 1e12
    achieved = w.flops / mean_kernel_s / 1e12
    log(f"bench: {args.steps} steps in {wall * 1e3:.2f} ms; kernel mean {mean_kernel_s * 1e6:.1f} us "
        f"(min {min(kernel_ms) * 1e3:.1f} us); {achieved:.1f} TFLOP/s = {100 * achieved / PEAK_BF16_TFLOPS:.2f}% of peak")

    traffic = committed_traffic(w.name) if splits == 1 and not args.dropout else None
    kname = (f"fa_fwd_kernel<{w.D},{'bf16' if w.dtype == 'bf16' else 'f16'},{'causal' if w.causal else 'full'}"
             f"{',dropout' if args.dropout else ''}>")
    if splits > 1:
        kname += " + fa_merge_kernel (the events bracket both)"
    # below the ridge point (peak flop/s over peak bytes/s) the HBM roofline bounds the step
    if w.flops / w.hbm_bytes >= PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
        roof = {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 5)}
    else:
        gbs = w.hbm_bytes / mean_kernel_s / 1e9
        roof = {"bound": "hbm", "achieved": round(gbs, 3), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 5), "tflops": round(achieved, 3)}
    roof.update({"traffic": traffic, "kernel": kname, "mean_launch_us": round(mean_kernel_s * 1e6, 3),
                 "algorithmic_bytes": w.hbm_bytes})
    if traffic is not None:  # bytes beyond L2 per launch (counters) over this run's mean launch time
        roof["traffic_gbs"] = round(traffic / mean_kernel_s / 1e9, 1)
    sq = committed_sq_counters(w.name) if splits == 1 and not args.dropout else None
    if sq is not None:  # SIMD-cycle fractions from the committed SQ counter profile of this kernel
        roof["counters"] = sq
    out = {
        "metric": (METRIC if w.name == "train7b_4k" and not args.dropout
                   else f"attention fwd TFLOP/s ({w.description}{f', dropout {args.dropout}' if args.dropout else ''})"),
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Lq": w.Lq, "Lk": w.Lk, "D": w.D, "causal": w.causal,
                   "scale": w.scale, "seed": w.seed, "num_splits": splits, "flop_per_step": w.flops,
                   "dropout_p": args.dropout},
        "pct_of_mfma_peak": round(100 * value / PEAK_BF16_TFLOPS, 3),
        "roofline": roof,
        "timing": res["timing"],
    }
    at_clock(out["timing"], achieved)
    if not args.no_parity:
        out["parity"] = sampled_parity(inp, o, lse, dropout_p=args.dropout)
        log(f"bench: parity {out['parity']}")
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, dropout_p=args.dropout)
        log(f"bench: cpu baseline {out['cpu_baseline']}")
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
