"""Python binding of libfa355, the gfx950 fused attention forward and backward passes.

Argument marshalling only: every step of the computation runs in the HIP
kernel behind the C ABI declared in ``include/fa355.h``.  PyTorch supplies
device memory and the current stream.  There is no fallback: if the compiled
library is missing, importing this package raises ImportError.

Names follow the C ABI: ``fa_fwd``, ``fa_fwd_strided``, ``fa_fwd_splitkv``,
``fa_fwd_splitkv_workspace_size``, ``fa_status_string``, ``fa_last_hip_error``,
``fa_version``, ``fa_bwd``, ``fa_bwd_workspace_size``, ``fa_fwd_dropout``,
``fa_bwd_dropout``, ``fa_fwd_dropout_strided``, ``fa_bwd_strided`` (reached through ``fa_fwd`` /
``fa_bwd`` with views and ``dropout_p``), ``fa_fwd_splitkv_noalloc``, ``fa_fwd_launch_shape``;
``fa_fwd_qkvpacked`` is a
view helper over ``fa_fwd_strided`` for a packed [B, L, 3, H, D] qkv buffer,
``suggest_num_splits`` a host heuristic, and ``flash_attention`` an autograd
function whose forward is ``fa_fwd`` and whose backward is ``fa_bwd``.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = ["fa_fwd", "fa_fwd_strided", "fa_fwd_splitkv", "fa_fwd_splitkv_workspace_size", "fa_fwd_qkvpacked",
           "fa_fwd_splitkv_noalloc", "FA_NOALLOC_SCRATCH_BYTES",
           "suggest_num_splits", "fa_bwd", "fa_bwd_workspace_size", "fa_fwd_dropout", "fa_bwd_dropout",
           "flash_attention", "fa_status_string",
           "fa_last_hip_error", "fa_version", "fa_fwd_launch_shape", "FaError", "lib", "LIB_PATH", "FA_DTYPE_F16", "FA_DTYPE_BF16"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa355.so")

FA_DTYPE_F16 = 0
FA_DTYPE_BF16 = 1
_DTYPES = {torch.float16: FA_DTYPE_F16, torch.bfloat16: FA_DTYPE_BF16}


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libfa355.so is not built ({LIB_PATH} missing); build it with "
            "`python tiled_attention_06_amd/build.py` or `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i = ctypes.c_void_p, ctypes.c_int
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, ctypes.c_float, i, i, vp]
    lib.fa_fwd.restype = i
    lib.fa_fwd_strided.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, vp, vp, vp, vp, ctypes.c_float, i, i, vp]
    lib.fa_fwd_strided.restype = i
    lib.fa_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, vp, vp, vp, vp, ctypes.c_float, i, i, i, vp,
                                   ctypes.c_size_t, vp]
    lib.fa_fwd_splitkv.restype = i
    lib.fa_fwd_splitkv_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, vp, vp, vp, vp, ctypes.c_float, i, i,
                                           i, vp]
    lib.fa_fwd_splitkv_noalloc.restype = i
    lib.fa_fwd_splitkv_workspace_size.argtypes = [i, i, i, i, i]
    lib.fa_fwd_splitkv_workspace_size.restype = ctypes.c_size_t
    lib.fa_bwd.argtypes = [vp] * 9 + [i] * 5 + [ctypes.c_float, i, i, vp, ctypes.c_size_t, vp]
    lib.fa_bwd.restype = i
    lib.fa_fwd_dropout.argtypes = [vp] * 5 + [i] * 5 + [ctypes.c_float, i, i, ctypes.c_float, ctypes.c_uint64, vp]
    lib.fa_fwd_dropout.restype = i
    lib.fa_bwd_dropout.argtypes = [vp] * 9 + [i] * 5 + [ctypes.c_float, i, i, ctypes.c_float, ctypes.c_uint64, vp,
                                                       ctypes.c_size_t, vp]
    lib.fa_bwd_dropout.restype = i
    lib.fa_fwd_dropout_strided.argtypes = ([vp] * 5 + [i] * 5 + [vp] * 4 +
                                           [ctypes.c_float, i, i, ctypes.c_float, ctypes.c_uint64, vp])
    lib.fa_fwd_dropout_strided.restype = i
    lib.fa_bwd_strided.argtypes = ([vp] * 9 + [i] * 5 + [vp, ctypes.c_float, i, i, ctypes.c_float, ctypes.c_uint64,
                                                         vp, ctypes.c_size_t, vp])
    lib.fa_bwd_strided.restype = i
    lib.fa_bwd_workspace_size.argtypes = [i, i, i]
    lib.fa_bwd_workspace_size.restype = ctypes.c_size_t
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_last_hip_error.argtypes = []
    lib.fa_last_hip_error.restype = i
    lib.fa_version.argtypes = []
    lib.fa_version.restype = i
    lib.fa_fwd_launch_shape.argtypes = [i, i, i, i, i, i, ctypes.c_float, i, ctypes.POINTER(i), ctypes.POINTER(i),
                                        ctypes.POINTER(i)]
    lib.fa_fwd_launch_shape.restype = i
    return lib


lib = _load()


class FaError(RuntimeError):
    def __init__(self, code: int):
        self.code = code
        super().__init__(f"{fa_status_string(code)} (status {code})")


def fa_status_string(status: int) -> str:
    return lib.fa_status_string(int(status)).decode()


def fa_last_hip_error() -> int:
    return int(lib.fa_last_hip_error())


def fa_version() -> int:
    return int(lib.fa_version())


def _check(q, k, v, o, lse):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, L, D] (views of any strides)")
    B, H, Lq, D = q.shape
    Lk = k.shape[2]
    if tuple(k.shape) != (B, H, Lk, D) or tuple(v.shape) != (B, H, Lk, D):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype, float16 or bfloat16")
    dev = q.device
    if dev.type != "cuda" or k.device != dev or v.device != dev:
        raise ValueError("q, k, v must be on the same GPU")
    if o is None:
        o = torch.empty_like(q, memory_format=torch.contiguous_format)
    elif tuple(o.shape) != tuple(q.shape) or o.dtype != q.dtype or o.device != dev:
        raise ValueError("o must be a tensor of q's shape, dtype and device")
    if lse is None:
        lse = torch.empty((B, H, Lq), dtype=torch.float32, device=dev)
    elif tuple(lse.shape) != (B, H, Lq) or lse.dtype != torch.float32 or lse.device != dev or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor [B, H, Lq]")
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        if t.stride(3) != 1:
            raise ValueError(f"{name}: the head dim must be contiguous (stride 1)")
    return B, H, Lq, Lk, D, o, lse


def _launch(strided, q, k, v, o, lse, B, H, Lq, Lk, D, causal, scale, stream, splits=1, workspace=None):
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    if splits != 1:
        need = fa_fwd_splitkv_workspace_size(B, H, Lq, D, splits)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        st = [(ctypes.c_int64 * 3)(*t.stride()[:3]) for t in (q, k, v, o)]
        code = lib.fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                  B, H, Lq, Lk, D, *[ctypes.cast(s_, ctypes.c_void_p) for s_ in st],
                                  float(scale), 1 if causal else 0, _DTYPES[q.dtype], int(splits),
                                  workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                  stream.cuda_stream)
    elif not strided:
        code = lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                          B, H, Lq, Lk, D, float(scale), 1 if causal else 0, _DTYPES[q.dtype], stream.cuda_stream)
    else:
        st = [(ctypes.c_int64 * 3)(*t.stride()[:3]) for t in (q, k, v, o)]
        code = lib.fa_fwd_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                  B, H, Lq, Lk, D, *[ctypes.cast(s_, ctypes.c_void_p) for s_ in st],
                                  float(scale), 1 if causal else 0, _DTYPES[q.dtype], stream.cuda_stream)
    if code != 0:
        raise FaError(code)
    return o, lse


def fa_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor | None = None,
           lse: torch.Tensor | None = None, *, causal: bool = False, scale: float | None = None,
           stream: torch.cuda.Stream | None = None, num_splits: int = 1, dropout_p: float = 0.0, seed: int = 0):
    """Enqueue the attention forward pass on ``stream`` (default: torch's current stream of q's device).

    q: [B, H, Lq, D]; k, v: [B, H, Lk, D]; fp16/bf16 tensors on one GPU, dense or
    any strided views with a contiguous head dim (a [B, L, H, D] tensor passed as
    ``x.transpose(1, 2)`` is used in place).  o (q's shape and dtype, dense or a
    view) and lse ([B, H, Lq], float32, dense) are allocated when not given.
    ``scale`` defaults to 1/sqrt(D).  Causal with Lq < Lk aligns the queries with
    the last Lq keys.  Dense inputs go through the C ``fa_fwd``, others through
    ``fa_fwd_strided``; ``num_splits`` > 1 goes through ``fa_fwd_splitkv`` with a
    workspace allocated here (see ``suggest_num_splits``).  Returns (o, lse).
    """
    if dropout_p:
        if num_splits != 1:
            raise ValueError("dropout is served by the single-pass call only (num_splits=1)")
        return fa_fwd_dropout(q, k, v, o, lse, causal=causal, scale=scale, dropout_p=dropout_p, seed=seed,
                              stream=stream)
    B, H, Lq, Lk, D, o, lse = _check(q, k, v, o, lse)
    dense = all(t.is_contiguous() for t in (q, k, v, o))
    return _launch(not dense, q, k, v, o, lse, B, H, Lq, Lk, D, causal, scale, stream, num_splits)


def fa_fwd_dropout(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor | None = None,
                   lse: torch.Tensor | None = None, *, causal: bool = False, scale: float | None = None,
                   dropout_p: float = 0.0, seed: int = 0, stream: torch.cuda.Stream | None = None):
    """The C ``fa_fwd_dropout`` (dense tensors) or ``fa_fwd_dropout_strided`` (views): dropout probability
    and 64-bit seed."""
    B, H, Lq, Lk, D, o, lse = _check(q, k, v, o, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    if all(t.is_contiguous() for t in (q, k, v, o)):
        code = lib.fa_fwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, Lq,
                                  Lk, D, float(scale), 1 if causal else 0, _DTYPES[q.dtype], float(dropout_p), seed,
                                  stream.cuda_stream)
    else:
        st = [(ctypes.c_int64 * 3)(*t.stride()[:3]) for t in (q, k, v, o)]
        code = lib.fa_fwd_dropout_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                          B, H, Lq, Lk, D, *[ctypes.cast(s_, ctypes.c_void_p) for s_ in st],
                                          float(scale), 1 if causal else 0, _DTYPES[q.dtype], float(dropout_p),
                                          seed, stream.cuda_stream)
    if code != 0:
        raise FaError(code)
    return o, lse


def fa_fwd_strided(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor | None = None,
                   lse: torch.Tensor | None = None, *, causal: bool = False, scale: float | None = None,
                   stream: torch.cuda.Stream | None = None):
    """Like ``fa_fwd``, always through the C ``fa_fwd_strided`` (the tensors' own strides)."""
    B, H, Lq, Lk, D, o, lse = _check(q, k, v, o, lse)
    return _launch(True, q, k, v, o, lse, B, H, Lq, Lk, D, causal, scale, stream)


def fa_fwd_splitkv_workspace_size(B: int, H: int, Lq: int, D: int, num_splits: int) -> int:
    """Bytes of workspace ``fa_fwd_splitkv`` needs (0 for num_splits == 1 or invalid arguments)."""
    return int(lib.fa_fwd_splitkv_workspace_size(B, H, Lq, D, num_splits))


def fa_fwd_splitkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor | None = None,
                   lse: torch.Tensor | None = None, *, causal: bool = False, scale: float | None = None,
                   num_splits: int = 2, workspace: torch.Tensor | None = None,
                   stream: torch.cuda.Stream | None = None):
    """Like ``fa_fwd`` through the C ``fa_fwd_splitkv``: the keys of each query tile are divided into
    ``num_splits`` ranges and merged exactly.  ``workspace`` (a device tensor of at least
    ``fa_fwd_splitkv_workspace_size`` bytes) is allocated when not given."""
    B, H, Lq, Lk, D, o, lse = _check(q, k, v, o, lse)
    if num_splits == 1:
        return _launch(True, q, k, v, o, lse, B, H, Lq, Lk, D, causal, scale, stream)
    return _launch(True, q, k, v, o, lse, B, H, Lq, Lk, D, causal, scale, stream, num_splits, workspace)


FA_NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024  # the scratch array of fa_fwd_splitkv_noalloc (include/fa355.h)


def fa_fwd_splitkv_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
                           *, causal: bool = False, scale: float | None = None, num_splits: int = 2,
                           stream: torch.cuda.Stream | None = None):
    """The C ``fa_fwd_splitkv_noalloc``: ``fa_fwd_splitkv`` with its partials in the library's own device
    array (at most FA_NOALLOC_SCRATCH_BYTES), so that neither this call nor the library allocates.  o and
    lse must be given (this wrapper allocates nothing either).  Calls that may overlap on one GPU race on
    the shared array."""
    if o is None or lse is None:
        raise ValueError("fa_fwd_splitkv_noalloc allocates nothing: pass o and lse")
    B, H, Lq, Lk, D, o, lse = _check(q, k, v, o, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = [(ctypes.c_int64 * 3)(*t.stride()[:3]) for t in (q, k, v, o)]
    code = lib.fa_fwd_splitkv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                      B, H, Lq, Lk, D, *[ctypes.cast(s_, ctypes.c_void_p) for s_ in st],
                                      float(scale), 1 if causal else 0, _DTYPES[q.dtype], int(num_splits),
                                      stream.cuda_stream)
    if code != 0:
        raise FaError(code)
    return o, lse


def fa_fwd_launch_shape(B: int, H: int, Lq: int, Lk: int, D: int, causal: bool, dropout_p: float = 0.0,
                        num_splits: int = 1) -> tuple[int, int, int]:
    """(workgroups, rows per work item, work items per workgroup) of the forward kernel for these sizes on the
    current device (``fa_fwd_launch_shape``)."""
    wg, rows, items = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0)
    code = lib.fa_fwd_launch_shape(B, H, Lq, Lk, D, int(bool(causal)), float(dropout_p), num_splits,
                                   ctypes.byref(wg), ctypes.byref(rows), ctypes.byref(items))
    if code != 0:
        raise FaError(code)
    return wg.value, rows.value, items.value


def suggest_num_splits(B: int, H: int, Lq: int, Lk: int, D: int, causal: bool, num_cu: int = 256) -> int:
    """Key splits for ``fa_fwd_splitkv``: 1 unless the query tiles leave most CUs idle.

    One workgroup covers 256 query rows and occupies one CU.  With at most half as
    many workgroups as CUs, the keys are split so that about one workgroup per CU
    results, keeping at least eight 64-key tiles per split (causal: counted over the
    keys an average query row sees).  With more workgroups the merge costs more than
    the balance gains (measured: 7B 2K causal, 256 workgroups, is slower split).
    """
    wgs = B * H * ((Lq + 255) // 256)
    if 2 * wgs > num_cu:
        return 1
    keys = Lk - Lq / 2 if causal else Lk  # causal: visible keys of the average row (Lq <= Lk)
    tiles = int(-(-keys // 64))
    return int(max(1, min(256, num_cu // wgs, tiles // 8)))


def fa_fwd_qkvpacked(qkv: torch.Tensor, o: torch.Tensor | None = None, lse: torch.Tensor | None = None, *,
                     causal: bool = False, scale: float | None = None, stream: torch.cuda.Stream | None = None):
    """Attention on a packed qkv buffer [B, L, 3, H, D] (q, k, v interleaved per position).

    Runs in place on strided views of qkv.  o, when not given, is allocated as
    [B, L, H, D] (the packed call's output layout); lse is [B, H, L].  Returns
    (o, lse) with o in [B, L, H, D].
    """
    if qkv.dim() != 5 or qkv.shape[2] != 3:
        raise ValueError("qkv must be [B, L, 3, H, D]")
    B, L, _, H, D = qkv.shape
    q, k, v = (qkv[:, :, i].transpose(1, 2) for i in range(3))
    if o is None:
        o = torch.empty((B, L, H, D), dtype=qkv.dtype, device=qkv.device)
    elif tuple(o.shape) != (B, L, H, D):
        raise ValueError("o must be [B, L, H, D]")
    _, lse = fa_fwd_strided(q, k, v, o.transpose(1, 2), lse, causal=causal, scale=scale, stream=stream)
    return o, lse


def fa_bwd_workspace_size(B: int, H: int, Lq: int) -> int:
    """Bytes of workspace ``fa_bwd`` needs (0 for invalid arguments)."""
    return int(lib.fa_bwd_workspace_size(B, H, Lq))


def fa_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, dout: torch.Tensor,
           lse: torch.Tensor, dq: torch.Tensor | None = None, dk: torch.Tensor | None = None,
           dv: torch.Tensor | None = None, *, causal: bool = False, scale: float | None = None,
           workspace: torch.Tensor | None = None, stream: torch.cuda.Stream | None = None, dropout_p: float = 0.0,
           seed: int = 0):
    """Enqueue the attention backward pass (the C ``fa_bwd``): gradients of o = fa_fwd(q, k, v) for dout.

    q, o, dout: [B, H, Lq, D]; k, v: [B, H, Lk, D]; lse: [B, H, Lq] float32 dense (fa_fwd's outputs o and
    lse for the same q, k, v, scale and causal flag).  Tensors may be views of any strides with a
    contiguous head dim (dense ones go through ``fa_bwd`` / ``fa_bwd_dropout``, others through
    ``fa_bwd_strided``).  dq, dk, dv (q's, k's, v's shapes; views allowed) are allocated dense when not
    given; ``workspace`` (at least ``fa_bwd_workspace_size`` bytes) likewise.  ``dropout_p`` and ``seed``
    must be those of the forward pass.  Returns (dq, dk, dv).
    """
    B, H, Lq, Lk, D, o, lse = _check(q, k, v, o, lse)
    if tuple(dout.shape) != tuple(q.shape) or dout.dtype != q.dtype or dout.device != q.device:
        raise ValueError("dout must be a tensor of q's shape, dtype and device")
    dq = torch.empty_like(q, memory_format=torch.contiguous_format) if dq is None else dq
    dk = torch.empty_like(k, memory_format=torch.contiguous_format) if dk is None else dk
    dv = torch.empty_like(v, memory_format=torch.contiguous_format) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if tuple(t.shape) != tuple(ref.shape) or t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{name} must be a tensor of {name[1:]}'s shape, dtype and device")
    tensors = (q, k, v, o, dout, dq, dk, dv)
    for name, t in zip(("q", "k", "v", "o", "dout", "dq", "dk", "dv"), tensors):
        if t.stride(3) != 1:
            raise ValueError(f"{name}: the head dim must be contiguous (stride 1)")
    dense = all(t.is_contiguous() for t in tensors)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    need = fa_bwd_workspace_size(B, H, Lq)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if not dense:
        st = (ctypes.c_int64 * 24)(*[x for t in tensors for x in t.stride()[:3]])
        code = lib.fa_bwd_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                                  lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Lq, Lk, D,
                                  ctypes.cast(st, ctypes.c_void_p), float(scale), 1 if causal else 0,
                                  _DTYPES[q.dtype], float(dropout_p), int(seed) & 0xFFFFFFFFFFFFFFFF,
                                  workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                  stream.cuda_stream)
    elif dropout_p:
        code = lib.fa_bwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                                  lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Lq, Lk, D,
                                  float(scale), 1 if causal else 0, _DTYPES[q.dtype], float(dropout_p),
                                  int(seed) & 0xFFFFFFFFFFFFFFFF, workspace.data_ptr(),
                                  workspace.numel() * workspace.element_size(), stream.cuda_stream)
    else:
        code = lib.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                          dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Lq, Lk, D, float(scale),
                          1 if causal else 0, _DTYPES[q.dtype], workspace.data_ptr(),
                          workspace.numel() * workspace.element_size(), stream.cuda_stream)
    if code != 0:
        raise FaError(code)
    return dq, dk, dv


class _FlashAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, causal, scale, dropout_p, seed):
        # views are used in place (a contiguous head dim is all the kernels need)
        o, lse = fa_fwd(q, k, v, causal=causal, scale=scale, dropout_p=dropout_p, seed=seed)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.causal, ctx.scale, ctx.dropout_p, ctx.seed = causal, scale, dropout_p, seed
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        if do.stride(3) != 1:
            do = do.contiguous()
        dq, dk, dv = fa_bwd(q, k, v, o, do, lse, causal=ctx.causal, scale=ctx.scale, dropout_p=ctx.dropout_p,
                            seed=ctx.seed)
        return dq, dk, dv, None, None, None, None


def flash_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
                    scale: float | None = None, dropout_p: float = 0.0, seed: int | None = None) -> torch.Tensor:
    """o = dropout(softmax(scale·q·kᵀ [causal])) · v on [B, H, L, D] tensors, differentiable in q, k and v.

    The forward pass is ``fa_fwd`` (o and the per-row LSE are kept), the backward pass ``fa_bwd``; with
    ``dropout_p`` > 0 the dropout bits come from ``seed`` (drawn from torch's CPU generator when None) and
    are recomputed, not stored, for the backward pass.
    """
    if dropout_p and seed is None:
        seed = int(torch.randint(0, 2 ** 62, (1,)).item())
    return _FlashAttention.apply(q, k, v, causal, scale, dropout_p, 0 if seed is None else seed)
