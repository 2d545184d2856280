"""Python binding of the MI355X exact-attention library (``libattn_mi355x.so``).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/attn_mi355x.h``.  PyTorch is
used for device memory and the current stream.  There is no fallback: if the
shared library is missing or fails to load, importing this package raises.

The library is loaded after ``import torch`` so that it binds to the HIP
runtime PyTorch already loaded (same soname), giving one runtime per process.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = [
    "attn_fwd", "attn_bwd_preprocess", "attn_bwd", "attn_bwd_workspace_bytes",
    "attn_fwd_gqa", "attn_bwd_gqa", "attn_bwd_gqa_workspace_bytes",
    "attention_backward", "attn_sparse_fwd", "attn_sparse_bwd", "attn_sparse_bwd_workspace_bytes",
    "attn_bwd_noalloc", "attn_bwd_noalloc_max_workspace_bytes", "attn_bwd_workspace_bytes",
    "lib_path", "AttnError", "version",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libattn_mi355x.so")


class AttnError(RuntimeError):
    """A non-OK status returned by the C ABI."""

    def __init__(self, status: int, msg: str):
        super().__init__(f"attn status {status}: {msg}")
        self.status = status


def _load():
    if not os.path.exists(lib_path):
        raise ImportError(
            f"{lib_path} is missing: build it first (python exact_attention_bwd_amd/build.py)")
    lib = ctypes.CDLL(lib_path, mode=ctypes.RTLD_GLOBAL)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
    lib.attn_fwd.restype = i
    lib.attn_bwd_preprocess.argtypes = [vp, vp, vp, i, i, i, i, vp]
    lib.attn_bwd_preprocess.restype = i
    lib.attn_bwd_workspace_bytes.argtypes = [i, i, i, i]
    lib.attn_bwd_workspace_bytes.restype = sz
    lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, f, vp]
    lib.attn_bwd.restype = i
    lib.attn_bwd_timed.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, f, vp, vp, vp]
    lib.attn_bwd_timed.restype = i
    lib.attn_fwd_gqa.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    lib.attn_fwd_gqa.restype = i
    lib.attn_bwd_workspace_bytes_ex.argtypes = [i, i, i, i, i, i]
    lib.attn_bwd_workspace_bytes_ex.restype = sz
    lib.attn_bwd_gqa_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.attn_bwd_gqa_workspace_bytes.restype = sz
    lib.attn_bwd_gqa.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, f, vp]
    lib.attn_bwd_gqa.restype = i
    lib.attn_bwd_gqa_timed.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, f, vp, vp, vp]
    lib.attn_bwd_gqa_timed.restype = i
    lib.attn_sparse_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    lib.attn_sparse_fwd.restype = i
    lib.attn_sparse_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.attn_sparse_bwd_workspace_bytes.restype = sz
    lib.attn_sparse_bwd.argtypes = [vp] * 12 + [sz, i, i, i, i, i, i, f, vp]
    lib.attn_sparse_bwd.restype = i
    lib.attn_sparse_bwd_timed.argtypes = [vp] * 12 + [sz, i, i, i, i, i, i, f, vp, vp, vp]
    lib.attn_sparse_bwd_timed.restype = i
    lib.attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
    lib.attn_bwd_noalloc.restype = i
    lib.attn_bwd_noalloc_max_workspace_bytes.argtypes = []
    lib.attn_bwd_noalloc_max_workspace_bytes.restype = sz
    lib.attn_last_error.argtypes = []
    lib.attn_last_error.restype = ctypes.c_char_p
    lib.attn_version.argtypes = []
    lib.attn_version.restype = ctypes.c_char_p
    return lib


_lib = _load()


def version() -> str:
    return _lib.attn_version().decode()


def _check(status: int):
    if status != 0:
        raise AttnError(status, _lib.attn_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _shape4(x: torch.Tensor, name: str):
    if x.dim() != 4:
        raise ValueError(f"{name} must be [B, H, N, d], got {tuple(x.shape)}")
    if x.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {x.dtype}")
    if not x.is_cuda or not x.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    return tuple(x.shape)


def _same(shape, x: torch.Tensor, name: str):
    if _shape4(x, name) != shape:
        raise ValueError(f"{name} has shape {tuple(x.shape)}, expected {shape}")


def _workspace(workspace, need: int, like: torch.Tensor):
    """The caller's workspace (any dtype) or a new one; it must be a contiguous
    tensor on the same device as the inputs.  Returns (tensor, size in bytes)."""
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=like.device)
    if not workspace.is_cuda or workspace.device != like.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    return workspace, workspace.numel() * workspace.element_size()


def _stat(x: torch.Tensor, shape3, name: str):
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous() or tuple(x.shape) != shape3:
        raise ValueError(f"{name} must be a contiguous float32 device tensor of shape {shape3}")


def attn_fwd(q, k, v, causal: bool, scale: float | None = None, o=None, lse=None, stream=None):
    """Forward pass.  q, k, v: bf16 [B, H, N, d].  Returns (o bf16, lse fp32 [B, H, N])."""
    shape = _shape4(q, "q")
    _same(shape, k, "k")
    _same(shape, v, "v")
    B, H, N, d = shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty_like(q)
    _same(shape, o, "o")
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _stat(lse, (B, H, N), "lse")
    _check(_lib.attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                         int(bool(causal)), float(scale), _stream(stream)))
    return o, lse


def attn_bwd_preprocess(o, do, D=None, stream=None):
    """D = rowsum(dO o O) in fp32, shape [B, H, N]."""
    shape = _shape4(o, "o")
    _same(shape, do, "dO")
    B, H, N, d = shape
    if D is None:
        D = torch.empty((B, H, N), dtype=torch.float32, device=o.device)
    _stat(D, (B, H, N), "D")
    _check(_lib.attn_bwd_preprocess(_ptr(o), _ptr(do), _ptr(D), B, H, N, d, _stream(stream)))
    return D


def attn_bwd_workspace_bytes(B: int, H: int, N: int, d: int, causal: bool | None = None,
                             Hkv: int | None = None) -> int:
    """Workspace bytes of attn_bwd (attn_bwd_gqa with Hkv): the exact size for
    `causal`, or with causal=None a size that serves both."""
    hkv = H if Hkv is None else Hkv
    if causal is None:
        return int(_lib.attn_bwd_gqa_workspace_bytes(B, H, hkv, N, d))
    return int(_lib.attn_bwd_workspace_bytes_ex(B, H, hkv, N, d, int(bool(causal))))


def attn_bwd(q, k, v, do, lse, D, causal: bool, scale: float | None = None,
             dq=None, dk=None, dv=None, workspace=None, stream=None, main_events=None):
    """Fused backward.  Returns (dq, dk, dv), bf16 [B, H, N, d].

    ``main_events``: optional pair of raw hipEvent_t handles (ints) recorded on
    the stream around the fused main kernel (profiling; see attn_bwd_timed)."""
    shape = _shape4(q, "q")
    for t, n in ((k, "k"), (v, "v"), (do, "dO")):
        _same(shape, t, n)
    B, H, N, d = shape
    _stat(lse, (B, H, N), "lse")
    _stat(D, (B, H, N), "D")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _same(shape, t, n)
    workspace, ws_bytes = _workspace(workspace, attn_bwd_workspace_bytes(B, H, N, d, causal), q)
    if main_events is None:
        _check(_lib.attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse), _ptr(D), _ptr(dq),
                             _ptr(dk), _ptr(dv), _ptr(workspace), ws_bytes, B, H, N, d,
                             int(bool(causal)), float(scale), _stream(stream)))
    else:
        ev0, ev1 = (ctypes.c_void_p(e) for e in main_events)
        _check(_lib.attn_bwd_timed(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse), _ptr(D), _ptr(dq),
                                   _ptr(dk), _ptr(dv), _ptr(workspace), ws_bytes, B, H, N, d,
                                   int(bool(causal)), float(scale), _stream(stream), ev0, ev1))
    return dq, dk, dv


def _gqa_shapes(q, k, v):
    B, H, N, d = _shape4(q, "q")
    kshape = _shape4(k, "k")
    _same(kshape, v, "v")
    if kshape[0] != B or kshape[2:] != (N, d) or kshape[1] < 1 or H % kshape[1] != 0:
        raise ValueError(f"k / v shape {kshape} does not fit q {tuple(q.shape)} (Hkv must divide H)")
    return B, H, kshape[1], N, d


def attn_fwd_gqa(q, k, v, causal: bool, scale: float | None = None, o=None, lse=None, stream=None):
    """Grouped-query forward.  q: bf16 [B, H, N, d]; k, v: bf16 [B, Hkv, N, d]
    with Hkv dividing H.  Returns (o bf16 [B, H, N, d], lse fp32 [B, H, N])."""
    B, H, Hkv, N, d = _gqa_shapes(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty_like(q)
    _same((B, H, N, d), o, "o")
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _stat(lse, (B, H, N), "lse")
    _check(_lib.attn_fwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, N, d,
                             int(bool(causal)), float(scale), _stream(stream)))
    return o, lse


def attn_bwd_gqa_workspace_bytes(B: int, H: int, Hkv: int, N: int, d: int) -> int:
    return int(_lib.attn_bwd_gqa_workspace_bytes(B, H, Hkv, N, d))


def attn_bwd_gqa(q, k, v, do, lse, D, causal: bool, scale: float | None = None,
                 dq=None, dk=None, dv=None, workspace=None, stream=None, main_events=None):
    """Grouped-query backward.  Returns (dq [B, H, N, d], dk, dv [B, Hkv, N, d]);
    dk and dv are summed over the query heads that share each K / V head."""
    B, H, Hkv, N, d = _gqa_shapes(q, k, v)
    _same((B, H, N, d), do, "dO")
    _stat(lse, (B, H, N), "lse")
    _stat(D, (B, H, N), "D")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _same((B, H, N, d), dq, "dq")
    _same((B, Hkv, N, d), dk, "dk")
    _same((B, Hkv, N, d), dv, "dv")
    workspace, ws_bytes = _workspace(workspace, attn_bwd_workspace_bytes(B, H, N, d, causal, Hkv), q)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse), _ptr(D), _ptr(dq), _ptr(dk), _ptr(dv),
            _ptr(workspace), ws_bytes, B, H, Hkv, N, d, int(bool(causal)), float(scale), _stream(stream))
    if main_events is None:
        _check(_lib.attn_bwd_gqa(*args))
    else:
        _check(_lib.attn_bwd_gqa_timed(*args, *(ctypes.c_void_p(e) for e in main_events)))
    return dq, dk, dv


def attn_bwd_noalloc(q, k, v, do, lse, D, causal: bool, dq, dk, dv, scale: float | None = None,
                     stream=None):
    """attn_bwd with the library's static scratch as workspace: the C call
    allocates nothing (the caller passes dq, dk, dv).  Shapes whose workspace
    exceeds attn_bwd_noalloc_max_workspace_bytes() raise AttnError; calls that
    overlap on one device race."""
    shape = _shape4(q, "q")
    for t, n in ((k, "k"), (v, "v"), (do, "dO"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        _same(shape, t, n)
    B, H, N, d = shape
    _stat(lse, (B, H, N), "lse")
    _stat(D, (B, H, N), "D")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check(_lib.attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse), _ptr(D), _ptr(dq), _ptr(dk),
                                 _ptr(dv), B, H, N, d, int(bool(causal)), float(scale), _stream(stream)))
    return dq, dk, dv


def attn_bwd_noalloc_max_workspace_bytes() -> int:
    return int(_lib.attn_bwd_noalloc_max_workspace_bytes())


def attention_backward(q, k, v, do, o, lse, causal: bool, scale: float | None = None,
                       workspace=None, stream=None):
    """The whole backward of the method: preprocess (D) then the fused backward."""
    D = attn_bwd_preprocess(o, do, stream=stream)
    return attn_bwd(q, k, v, do, lse, D, causal, scale, workspace=workspace, stream=stream)


# ---------------------------------------------------------------------------
# Top-k sparse attention (d_qk = 576, d_v = 512, heads in groups of 64)
# ---------------------------------------------------------------------------
def _dev(x, dtype, shape, name):
    if x.dtype != dtype or not x.is_cuda or not x.is_contiguous() or tuple(x.shape) != tuple(shape):
        raise ValueError(f"{name} must be a contiguous {dtype} device tensor of shape {tuple(shape)}, "
                         f"got {x.dtype} {tuple(x.shape)}")


def _sparse_dims(q, k, v, idx):
    if q.dim() != 3 or k.dim() != 2 or v.dim() != 2 or idx.dim() != 2:
        raise ValueError("expected q [Hq, Nq, dqk], k [Nkv, dqk], v [Nkv, dv], idx [Nq, topk]")
    Hq, Nq, dqk = q.shape
    Nkv, dvd = v.shape
    topk = idx.shape[1]
    _dev(q, torch.bfloat16, (Hq, Nq, dqk), "q")
    _dev(k, torch.bfloat16, (Nkv, dqk), "k")
    _dev(v, torch.bfloat16, (Nkv, dvd), "v")
    _dev(idx, torch.int32, (Nq, topk), "idx")
    return Hq, Nq, Nkv, dqk, dvd, topk


def attn_sparse_fwd(q, k, v, idx, topk_len=None, scale: float | None = None, o=None, lse=None,
                    stream=None):
    """Sparse forward.  Returns (o bf16 [Hq, Nq, dv], lse fp32 [Hq, Nq])."""
    Hq, Nq, Nkv, dqk, dvd, topk = _sparse_dims(q, k, v, idx)
    if topk_len is not None:
        _dev(topk_len, torch.int32, (Nq,), "topk_len")
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    o = torch.empty((Hq, Nq, dvd), dtype=torch.bfloat16, device=q.device) if o is None else o
    lse = torch.empty((Hq, Nq), dtype=torch.float32, device=q.device) if lse is None else lse
    _dev(o, torch.bfloat16, (Hq, Nq, dvd), "o")
    _dev(lse, torch.float32, (Hq, Nq), "lse")
    _check(_lib.attn_sparse_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(topk_len), _ptr(o),
                                _ptr(lse), Hq, Nq, Nkv, dqk, dvd, topk, float(scale), _stream(stream)))
    return o, lse


def attn_sparse_bwd_workspace_bytes(Hq: int, Nq: int, Nkv: int, topk: int, dqk: int = 576,
                                    dv: int = 512) -> int:
    return int(_lib.attn_sparse_bwd_workspace_bytes(Hq, Nq, Nkv, dqk, dv, topk))


def attn_sparse_bwd(q, k, v, do, lse, D, idx, topk_len=None, scale: float | None = None,
                    dq=None, dk=None, dv=None, workspace=None, stream=None, main_events=None):
    """Sparse backward.  Returns (dq [Hq, Nq, dqk], dk [Nkv, dqk], dv [Nkv, dv]), bf16."""
    Hq, Nq, Nkv, dqk, dvd, topk = _sparse_dims(q, k, v, idx)
    _dev(do, torch.bfloat16, (Hq, Nq, dvd), "dO")
    _dev(lse, torch.float32, (Hq, Nq), "lse")
    _dev(D, torch.float32, (Hq, Nq), "D")
    if topk_len is not None:
        _dev(topk_len, torch.int32, (Nq,), "topk_len")
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _dev(dq, torch.bfloat16, (Hq, Nq, dqk), "dq")
    _dev(dk, torch.bfloat16, (Nkv, dqk), "dk")
    _dev(dv, torch.bfloat16, (Nkv, dvd), "dv")
    workspace, ws_bytes = _workspace(workspace, attn_sparse_bwd_workspace_bytes(Hq, Nq, Nkv, topk, dqk, dvd), q)
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse), _ptr(D), _ptr(idx), _ptr(topk_len),
            _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), ws_bytes, Hq, Nq, Nkv, dqk, dvd, topk,
            float(scale), _stream(stream)]
    if main_events is None:
        _check(_lib.attn_sparse_bwd(*args))
    else:
        _check(_lib.attn_sparse_bwd_timed(*args, *(ctypes.c_void_p(e) for e in main_events)))
    return dq, dk, dv
