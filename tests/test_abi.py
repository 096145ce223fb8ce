"""The C ABI without a GPU: exported symbols, status strings, and every argument error.

Invalid arguments are rejected on the host before any HIP call, so these run on
a machine with no GPU.  No test here makes a call that would launch a kernel.
"""

from __future__ import annotations

import ctypes
import os
import re
import shutil
import subprocess
import sys

import pytest

import tiled_attention_06_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa355.h")

# distinct, 16-byte aligned fake device addresses: never dereferenced on error paths
P = [0x10000 * (i + 1) for i in range(5)]


def declared_functions():
    with open(HEADER, encoding="utf-8") as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", src, flags=re.M)


def call(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=1, H=1, Lq=64, Lk=64, D=128, scale=0.125, causal=0,
         dtype=1):
    return fa.lib.fa_fwd(q, k, v, o, lse, B, H, Lq, Lk, D, scale, causal, dtype, None)


def call_strided(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=2, H=3, Lq=64, Lk=64, D=128, strides=None,
                 scale=0.125, causal=0, dtype=1):
    """fa_fwd_strided with per-tensor (batch, head, row) strides; default: [B, L, H, D] views."""
    dflt = {"q": (Lq * H * D, D, H * D), "k": (Lk * H * D, D, H * D), "v": (Lk * H * D, D, H * D),
            "o": (Lq * H * D, D, H * D)}
    dflt.update(strides or {})
    arr = {n: (None if s_ is None else (ctypes.c_int64 * 3)(*s_)) for n, s_ in dflt.items()}
    ptr = [None if arr[n] is None else ctypes.cast(arr[n], ctypes.c_void_p) for n in ("q", "k", "v", "o")]
    return fa.lib.fa_fwd_strided(q, k, v, o, lse, B, H, Lq, Lk, D, *ptr, scale, causal, dtype, None)


def test_header_declares_the_abi():
    assert declared_functions() == ["fa_fwd", "fa_fwd_strided", "fa_fwd_splitkv_workspace_size", "fa_fwd_splitkv",
                                    "fa_fwd_splitkv_noalloc", "fa_bwd_workspace_size", "fa_bwd", "fa_fwd_dropout", "fa_bwd_dropout",
                                    "fa_fwd_dropout_strided", "fa_bwd_strided", "fa_status_string",
                                    "fa_last_hip_error", "fa_version", "fa_fwd_launch_shape"]


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(fa.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    nm = shutil.which("nm")
    if nm:
        out = subprocess.run([nm, "-D", "--defined-only", fa.LIB_PATH], capture_output=True, text=True).stdout
        exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
        assert set(declared_functions()) <= exported


def test_version_and_strings():
    assert fa.fa_version() == 10400
    for code in range(0, -14, -1):
        s = fa.fa_status_string(code)
        assert s and "unknown" not in s
    assert "unknown" in fa.fa_status_string(5)
    assert fa.fa_last_hip_error() == 0


@pytest.mark.parametrize("which", range(5))
def test_null_pointers(which):
    args = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4])
    args[list(args)[which]] = None
    assert call(**args) == -1


@pytest.mark.parametrize("field,value", [("B", 0), ("H", 0), ("Lq", 0), ("Lk", 0), ("B", -3), ("Lk", -1),
                                         ("Lq", 1 << 24), ("Lk", 16_777_000)])
def test_shapes(field, value):
    assert call(**{field: value}) == -2


def test_workgroup_limit():
    # B*H*ceil(Lq/256) must stay below 2^22 workgroups
    assert call(B=1 << 11, H=1 << 11, Lq=256, Lk=256) == -2
    assert call(B=1 << 10, H=1 << 11, Lq=257, Lk=257) == -2


@pytest.mark.parametrize("D", [0, 32, 63, 96, 100, 127, 256])
def test_head_dim(D):
    assert call(D=D) == -3


@pytest.mark.parametrize("dtype", [-1, 2, 3, 100])
def test_dtype(dtype):
    assert call(dtype=dtype) == -4


@pytest.mark.parametrize("which,off", [("q", 8), ("k", 2), ("v", 4), ("o", 12), ("lse", 2), ("lse", 1)])
def test_alignment(which, off):
    args = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4])
    args[which] += off
    assert call(**args) == -5


def test_lse_needs_only_4_byte_alignment_but_check_order_is_stable():
    # lse at +4 is fine for alignment; make a later check fail so nothing launches
    assert call(lse=P[4] + 4, D=96) == -3


@pytest.mark.parametrize("scale", [float("nan"), float("inf"), float("-inf")])
def test_scale(scale):
    assert call(scale=scale) == -6


def test_causal_requires_no_more_queries_than_keys():
    # Lq <= Lk is accepted (bottom-right alignment); make a later check fail so nothing launches
    assert call(causal=1, Lq=64, Lk=65, D=96) == -3
    assert call(causal=1, Lq=65, Lk=64) == -7
    assert call(causal=7, Lq=3, Lk=2) == -7


@pytest.mark.parametrize("which", ["q", "k", "v", "o"])
def test_strided_null_stride_pointer(which):
    assert call_strided(strides={which: None}) == -1


@pytest.mark.parametrize("which", ["q", "k", "v", "o"])
@pytest.mark.parametrize("bad", [(-8, 128, 384), (0, -128, 384), (0, 0, 120), (0, 0, -8)])
def test_strided_bad_strides(which, bad):
    # negative strides, or a row stride below D (rows would overlap)
    assert call_strided(strides={which: bad}) == -10


@pytest.mark.parametrize("which", ["q", "k", "v", "o"])
@pytest.mark.parametrize("bad", [(12, 128, 384), (0, 4, 384), (0, 0, 129)])
def test_strided_misaligned_strides(which, bad):
    # every row must start on a 16-byte boundary: strides are multiples of 8 elements
    assert call_strided(strides={which: bad}) == -5


@pytest.mark.parametrize("which", ["q", "k", "o"])
def test_strided_row_stride_limit(which):
    # ((L + 256) * row_stride + D) * 2 must stay below 2^32
    assert call_strided(strides={which: (0, 0, 1 << 24)}) == -2


@pytest.mark.parametrize("which", ["q", "k", "v", "o"])
def test_strided_row_stride_overflow(which):
    # a row stride whose 64-bit size product ((L + 256)·s + D)·2 wraps past 2^64 to a small
    # number (L = 64 here: 640·(2^57 + 8) + 256 = 5·2^64 + 5376) is still rejected
    s = (1 << 57) + 8
    assert s % 8 == 0 and ((64 + 256) * s + 128) * 2 % (1 << 64) < (1 << 32)
    assert call_strided(strides={which: (0, 0, s)}) == -2
    assert call_strided(strides={which: (0, 0, (1 << 63) - 8)}) == -2


def test_strided_valid_strides_reach_later_checks():
    # broadcast K/V (batch and head stride 0) and padded rows are accepted; a later
    # check (head dim) fails, so nothing launches
    assert call_strided(strides={"k": (0, 0, 136), "v": (0, 0, 256)}, D=96) == -3
    assert call_strided(causal=1, Lq=65, Lk=64) == -7
    assert call_strided(scale=float("nan")) == -6


def test_dense_call_matches_the_strided_checks():
    # fa_fwd is fa_fwd_strided with dense strides: same codes for the same faults
    assert call(Lk=16_776_960) == call_strided(Lk=16_776_960, strides={"k": (0, 0, 128), "v": (0, 0, 128)}) == -2


def test_python_binding_rejects_bad_tensors():
    import torch

    q = torch.zeros(1, 1, 4, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        fa.fa_fwd(q, q, q)                      # CPU tensors
    with pytest.raises(ValueError):
        fa.fa_fwd(q.float(), q.float(), q.float())
    with pytest.raises(ValueError):
        fa.fa_fwd(q[0], q[0], q[0])             # not 4-D
    with pytest.raises(ValueError):
        fa.fa_fwd(q, q[:, :, :2], q)            # k/v mismatch
    qt = torch.zeros(1, 1, 64, 4, dtype=torch.float16).transpose(2, 3)
    with pytest.raises(ValueError):
        fa.fa_fwd(qt, qt, qt)                   # head dim not contiguous
    with pytest.raises(ValueError):
        fa.fa_fwd_qkvpacked(torch.zeros(1, 4, 2, 1, 64, dtype=torch.float16))  # not [B, L, 3, H, D]


def test_missing_library_fails_loudly(tmp_path):
    """The binding has no fallback: without libfa355.so the import raises ImportError."""
    pkg = tmp_path / "tiled_attention_06_amd"
    pkg.mkdir()
    src = os.path.join(ROOT, "tiled_attention_06_amd")
    for name in os.listdir(src):
        if name.endswith(".py"):
            shutil.copy(os.path.join(src, name), pkg / name)
    res = subprocess.run([sys.executable, "-c", "import tiled_attention_06_amd"], cwd=tmp_path,
                         capture_output=True, text=True, env={**os.environ, "PYTHONPATH": str(tmp_path)})
    assert res.returncode != 0
    assert "ImportError" in res.stderr and "not built" in res.stderr


def test_product_path_does_not_touch_the_oracle():
    """Nothing in the package imports the oracle or falls back to a CPU path."""
    src = os.path.join(ROOT, "tiled_attention_06_amd")
    for dirpath, _, files in os.walk(src):
        for name in files:
            if name.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                with open(os.path.join(dirpath, name), encoding="utf-8") as f:
                    text = f.read()
                assert "oracle" not in text.lower(), name
                assert "scaled_dot_product_attention" not in text, name


def call_split(splits=2, ws=P[4] * 16, ws_bytes=None, B=1, H=2, Lq=300, Lk=500, D=128, **kw):
    if ws_bytes is None:
        ws_bytes = fa.fa_fwd_splitkv_workspace_size(B, H, Lq, D, splits)
    st = {"q": (H * Lq * D, Lq * D, D), "k": (H * Lk * D, Lk * D, D), "v": (H * Lk * D, Lk * D, D),
          "o": (H * Lq * D, Lq * D, D)}
    arr = [(ctypes.c_int64 * 3)(*st[n]) for n in ("q", "k", "v", "o")]
    ptr = [ctypes.cast(a, ctypes.c_void_p) for a in arr]
    args = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], scale=0.125, causal=0, dtype=1)
    args.update(kw)
    return fa.lib.fa_fwd_splitkv(args["q"], args["k"], args["v"], args["o"], args["lse"], B, H, Lq, Lk, D, *ptr,
                                 args["scale"], args["causal"], args["dtype"], splits, ws, ws_bytes, None)


def call_noalloc(splits=2, B=1, H=2, Lq=300, Lk=500, D=128, **kw):
    st = {"q": (H * Lq * D, Lq * D, D), "k": (H * Lk * D, Lk * D, D), "v": (H * Lk * D, Lk * D, D),
          "o": (H * Lq * D, Lq * D, D)}
    st.update(kw.pop("strides", {}))
    arr = [None if st[n] is None else (ctypes.c_int64 * 3)(*st[n]) for n in ("q", "k", "v", "o")]
    ptr = [None if a is None else ctypes.cast(a, ctypes.c_void_p) for a in arr]
    args = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], scale=0.125, causal=0, dtype=1)
    args.update(kw)
    return fa.lib.fa_fwd_splitkv_noalloc(args["q"], args["k"], args["v"], args["o"], args["lse"], B, H, Lq, Lk, D,
                                         *ptr, args["scale"], args["causal"], args["dtype"], splits, None)


def test_noalloc_argument_checks():
    # every argument fault is reported before the call touches HIP (no GPU here)
    for which in ("q", "k", "v", "o", "lse"):
        assert call_noalloc(**{which: None}) == -1
    assert call_noalloc(strides={"k": None}) == -1
    assert call_noalloc(splits=0) == -11 and call_noalloc(splits=257) == -11
    assert call_noalloc(D=96) == -3 and call_noalloc(dtype=2) == -4
    assert call_noalloc(scale=float("nan")) == -6
    assert call_noalloc(causal=1, Lq=501, Lk=500) == -7
    assert call_noalloc(strides={"o": (0, 0, 28_823_037_615_171_176)}) == -2
    # partials beyond the scratch array: FA_ERR_WORKSPACE, nothing enqueued
    cap = fa.FA_NOALLOC_SCRATCH_BYTES
    assert fa.fa_fwd_splitkv_workspace_size(1, 32, 256, 128, 16) > cap      # 16 splits of 32 x 256 rows
    assert call_noalloc(splits=16, B=1, H=32, Lq=256, Lk=16384) == -12
    assert fa.fa_fwd_splitkv_workspace_size(1, 32, 256, 128, 8) <= cap      # 8 of them fit
    assert call_noalloc(splits=8, B=1, H=32, Lq=256, Lk=16384, scale=float("inf")) == -6


def test_noalloc_scratch_size_in_header():
    with open(HEADER, encoding="utf-8") as f:
        m = re.search(r"#define FA_NOALLOC_SCRATCH_BYTES \((\d+)u \* (\d+)u \* (\d+)u\)", f.read())
    assert m and int(m.group(1)) * int(m.group(2)) * int(m.group(3)) == fa.FA_NOALLOC_SCRATCH_BYTES


def test_splitkv_workspace_size():
    # partial outputs (fp32 [splits, B*H, Lq, D]) then row statistics (fp32 [splits, B*H, Lq, 4])
    assert fa.fa_fwd_splitkv_workspace_size(2, 3, 100, 128, 4) == 4 * 6 * 100 * (128 + 4) * 4
    assert fa.fa_fwd_splitkv_workspace_size(1, 1, 7, 64, 3) == 3 * 7 * (64 + 4) * 4
    assert fa.fa_fwd_splitkv_workspace_size(1, 1, 7, 64, 1) == 0
    for bad in [(0, 1, 7, 64, 2), (1, 1, 7, 96, 2), (1, 1, 7, 64, 0), (1, 1, 7, 64, 257), (1, 0, 7, 64, 2)]:
        assert fa.fa_fwd_splitkv_workspace_size(*bad) == 0


@pytest.mark.parametrize("splits", [0, -1, 257, 1000])
def test_splitkv_split_count(splits):
    assert call_split(splits=splits, ws_bytes=1 << 40) == -11


def test_splitkv_workspace_errors():
    assert call_split(ws=None) == -1                         # no workspace
    assert call_split(ws=P[4] * 16 + 16) == -5                # not 256-byte aligned
    need = fa.fa_fwd_splitkv_workspace_size(1, 2, 300, 128, 2)
    assert call_split(ws_bytes=need - 1) == -12               # too small
    # enough workspace: a later check fails so nothing launches
    assert call_split(ws_bytes=need, scale=float("nan")) == -6
    assert call_split(ws_bytes=need, causal=1, Lq=501, Lk=500) == -7


def test_splitkv_partial_slab_limit():
    # (Lq + 256) * D * 4 must stay below 2^32 for the fp32 partials
    assert call_split(Lq=8_388_352, Lk=8_388_352, ws_bytes=1 << 62) == -2


def test_suggest_num_splits():
    assert fa.suggest_num_splits(4, 32, 4096, 4096, 128, True) == 1        # 2,048 workgroups fill 256 CUs
    assert fa.suggest_num_splits(1, 32, 2048, 2048, 128, True) == 1        # 256 workgroups already
    assert fa.suggest_num_splits(1, 8, 1, 32768, 128, False) == 32         # decode: 8 workgroups
    assert fa.suggest_num_splits(1, 32, 256, 16384, 128, False) == 8       # 32 workgroups
    assert fa.suggest_num_splits(2, 32, 512, 8192, 128, True) == 2         # 128 workgroups
    assert fa.suggest_num_splits(1, 32, 1024, 1024, 64, True) == 1         # 8 tiles on average
    assert fa.suggest_num_splits(1, 1, 128, 128, 64, False) == 1           # too few keys to split
    assert 1 <= fa.suggest_num_splits(1, 2, 256, 65536, 128, False) <= 256
    assert fa.suggest_num_splits(1, 1, 4, 1_000_003, 128, False) == 256      # one query tile, long cache


# ------------------------------------------------------------------------------------------
# fa_bwd: argument checks (nothing is launched on these paths)
# ------------------------------------------------------------------------------------------

PB = [0x100000 * (i + 1) for i in range(10)]  # q k v o dout lse dq dk dv workspace (256-byte aligned)


def call_bwd(B=1, H=2, Lq=300, Lk=500, D=128, scale=0.125, causal=0, dtype=1, ws_bytes=None, ptrs=None):
    p = dict(zip(["q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv", "ws"], PB))
    p.update(ptrs or {})
    if ws_bytes is None:
        ws_bytes = fa.fa_bwd_workspace_size(B, H, Lq)
    return fa.lib.fa_bwd(p["q"], p["k"], p["v"], p["o"], p["dout"], p["lse"], p["dq"], p["dk"], p["dv"],
                         B, H, Lq, Lk, D, scale, causal, dtype, p["ws"], ws_bytes, None)


def test_bwd_workspace_size():
    # LSE·log2(e), then Δ: fp32 per query row each, the second array 256-byte aligned
    assert fa.fa_bwd_workspace_size(2, 3, 100) == 2560 + 2400
    assert fa.fa_bwd_workspace_size(1, 1, 64) == 256 + 256
    assert fa.fa_bwd_workspace_size(1, 1, 5) == 256 + 8 * 4          # rows padded to a multiple of 4
    assert fa.fa_bwd_workspace_size(0, 1, 64) == 0 and fa.fa_bwd_workspace_size(1, 1, 0) == 0


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv", "ws"])
def test_bwd_null_pointers(which):
    assert call_bwd(ptrs={which: None}) == -1


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "dout", "dq", "dk", "dv"])
def test_bwd_alignment(which):
    base = dict(zip(["q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv", "ws"], PB))
    assert call_bwd(ptrs={which: base[which] + 8}) == -5
    assert call_bwd(ptrs={which: base[which] + 16}, scale=float("inf")) == -6  # 16 bytes is enough


def test_bwd_argument_checks():
    assert call_bwd(ptrs={"lse": PB[5] + 2}) == -5
    assert call_bwd(ptrs={"ws": PB[9] + 16}) == -5       # workspace needs 256-byte alignment
    assert call_bwd(B=0) == -2 and call_bwd(Lk=0) == -2
    assert call_bwd(D=96) == -3
    assert call_bwd(dtype=2) == -4
    assert call_bwd(scale=float("nan")) == -6
    assert call_bwd(causal=1, Lq=501, Lk=500) == -7
    need = fa.fa_bwd_workspace_size(1, 2, 300)
    assert call_bwd(ws_bytes=need - 1) == -12
    assert call_bwd(Lk=16_776_960) == -2                 # slab beyond 32-bit offsets
    # enough of everything: a later check fails, so nothing launches
    assert call_bwd(ws_bytes=need, causal=1, Lq=600, Lk=500) == -7


# ------------------------------------------------------------------------------------------
# dropout entry points: argument checks (nothing is launched on these paths)
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("p", [-0.1, 1.0, 1.5, float("nan"), float("inf"), 0.999])
def test_dropout_probability_checked(p):
    assert fa.lib.fa_fwd_dropout(*P, 1, 2, 64, 64, 128, 0.125, 0, 1, p, 7, None) == -13
    args = dict(zip(["q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv", "ws"], PB))
    need = fa.fa_bwd_workspace_size(1, 2, 64)
    assert fa.lib.fa_bwd_dropout(args["q"], args["k"], args["v"], args["o"], args["dout"], args["lse"], args["dq"],
                                 args["dk"], args["dv"], 1, 2, 64, 64, 128, 0.125, 0, 1, p, 7, args["ws"], need,
                                 None) == -13


def test_dropout_entry_points_run_the_common_checks():
    assert fa.lib.fa_fwd_dropout(None, *P[1:], 1, 2, 64, 64, 128, 0.125, 0, 1, 0.1, 7, None) == -1
    assert fa.lib.fa_fwd_dropout(*P, 1, 2, 64, 64, 96, 0.125, 0, 1, 0.1, 7, None) == -3
    assert fa.lib.fa_fwd_dropout(*P, 1, 2, 65, 64, 128, 0.125, 1, 1, 0.1, 7, None) == -7
    assert fa.lib.fa_fwd_dropout(*P, 1, 2, 64, 64, 128, float("nan"), 0, 1, 0.1, 2 ** 64 - 1, None) == -6


def call_bwd_strided(strides="blhd", B=1, H=2, Lq=300, Lk=500, D=128, ws_bytes=None, **kw):
    """fa_bwd_strided with [B, L, H, D] strides for all eight tensors unless `strides` is a list."""
    if strides == "blhd":
        rows = [Lq, Lk, Lk, Lq, Lq, Lq, Lk, Lk]
        strides = [x for L in rows for x in (L * H * D, D, H * D)]
    arr = None if strides is None else (ctypes.c_int64 * 24)(*strides)
    p = dict(zip(["q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv", "ws"], PB))
    if ws_bytes is None:
        ws_bytes = fa.fa_bwd_workspace_size(B, H, Lq)
    a = dict(scale=0.125, causal=0, dtype=1, p=0.0)
    a.update(kw)
    return fa.lib.fa_bwd_strided(p["q"], p["k"], p["v"], p["o"], p["dout"], p["lse"], p["dq"], p["dk"], p["dv"],
                                 B, H, Lq, Lk, D, None if arr is None else ctypes.cast(arr, ctypes.c_void_p),
                                 a["scale"], a["causal"], a["dtype"], a["p"], 7, p["ws"], ws_bytes, None)


def test_bwd_strided_checks():
    good = [x for L in [300, 500, 500, 300, 300, 300, 500, 500] for x in (L * 2 * 128, 128, 2 * 128)]
    assert call_bwd_strided(strides=None) == -1
    assert call_bwd_strided(scale=float("nan")) == -6                 # valid strides reach later checks
    for t in range(8):
        bad = list(good)
        bad[3 * t + 2] = 64                                           # row stride < D
        assert call_bwd_strided(strides=bad) == -10
        bad = list(good)
        bad[3 * t] = -8                                               # negative batch stride
        assert call_bwd_strided(strides=bad) == -10
        bad = list(good)
        bad[3 * t + 1] = 132                                          # head stride not a multiple of 8
        assert call_bwd_strided(strides=bad) == -5
    big = list(good)
    big[3 * 1 + 2] = 1 << 22                                          # k rows beyond 32-bit offsets
    assert call_bwd_strided(strides=big) == -2
    for t in range(8):                                                # a row stride whose size product wraps
        big = list(good)
        big[3 * t + 2] = 28_823_037_615_171_176
        assert call_bwd_strided(strides=big) == -2
    assert call_bwd_strided(p=1.0) == -13


def test_launch_shape_query():
    # fa_fwd_launch_shape: argument statuses as fa_fwd's, checked before any device query; for valid sizes a
    # grid that covers every query row once (256-row items, or 128-row items one or two to a workgroup)
    ref = (ctypes.c_int(), ctypes.c_int(), ctypes.c_int())
    out = [ctypes.byref(x) for x in ref]
    q = fa.lib.fa_fwd_launch_shape
    assert q(1, 1, 64, 64, 128, 0, 0.0, 1, None, out[1], out[2]) == -1
    assert q(0, 1, 64, 64, 128, 0, 0.0, 1, *out) == -2
    assert q(1, 1, 64, 64, 96, 0, 0.0, 1, *out) == -3
    assert q(1, 1, 65, 64, 128, 1, 0.0, 1, *out) == -7
    assert q(1, 1, 64, 64, 128, 0, 0.0, 0, *out) == -11
    assert q(1, 1, 64, 64, 128, 0, 0.0, 257, *out) == -11
    assert q(1, 1, 64, 64, 128, 0, 0.1, 2, *out) == -11
    assert q(1, 1, 64, 64, 128, 0, 1.5, 1, *out) == -13
    for B, H, Lq, Lk, D, causal, p, splits in [(4, 32, 4096, 4096, 128, True, 0.0, 1), (1, 32, 2048, 2048, 128, True, 0.0, 1),
                                              (1, 19, 1900, 1900, 64, False, 0.0, 1), (1, 8, 1, 32768, 128, True, 0.0, 32),
                                              (2, 3, 300, 300, 128, True, 0.2, 1)]:
        wg, rows, items = fa.fa_fwd_launch_shape(B, H, Lq, Lk, D, causal, p, splits)
        assert rows in (128, 256) and items in (1, 2)
        n_items = B * H * -(-Lq // rows)
        if rows == 256:
            assert items == 1 and wg == n_items * splits
        else:
            assert splits == 1 and wg == -(-n_items // items)
        if p > 0:
            assert items == 1
