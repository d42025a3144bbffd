"""osattn: fused online-softmax attention for AMD MI355X (gfx950), Python binding.

A thin ctypes layer over the C ABI in ``include/osattn.h`` (``libosattn.so`` next
to this file).  It only checks tensors and marshals pointers, sizes and the
current HIP stream: every step of the computation runs in the library's HIP
kernels.  There is no fallback: if the library is missing or a call fails, an
exception is raised.

    o, lse = attn_fwd(q, k, v, causal=False)          # q [B,H,N,d], k/v [B,Hkv,N,d]
    dq, dk, dv = attn_bwd(q, k, v, o, lse, do, causal=False)

Row softmax, log-softmax and cross-entropy with logits over the last dimension:

    y = rowsoftmax_fwd(x, log_softmax=False)          # any shape, rows = numel / cols
    dx = rowsoftmax_bwd(y, dy, log_softmax=False)
    loss, lse = rowxent_fwd(logits, targets)          # logits [..., C], targets int32
    dlogits = rowxent_bwd(logits, targets, lse, dloss)

The backward's three kernels can also be enqueued one at a time with
``attn_bwd_preprocess``, ``attn_bwd_dkdv`` and ``attn_bwd_dq`` on a shared
workspace (``new_bwd_workspace``).

Tensors must be contiguous ROCm-device tensors of one dtype (float32, float16 or
bfloat16); ``lse`` is float32 [B,H,N].  ``scale`` defaults to 1/sqrt(d).
"""

from __future__ import annotations

import ctypes
import functools
import math
import os

import torch

__all__ = [
    "attn_fwd",
    "attn_bwd",
    "attn_bwd_workspace_bytes",
    "attn_bwd_preprocess",
    "attn_bwd_dkdv",
    "attn_bwd_dq",
    "attn_bwd_noalloc",
    "new_bwd_workspace",
    "attn_fwd_splitkv",
    "attn_fwd_splitkv_workspace_bytes",
    "attn_fwd_masked",
    "attn_bwd_masked",
    "attn_bwd_masked_workspace_bytes",
    "attn_fwd_fp8",
    "attn_fwd_fp8_workspace_bytes",
    "rowsoftmax_fwd",
    "rowsoftmax_bwd",
    "rowxent_fwd",
    "rowxent_bwd",
    "status_string",
    "library",
    "library_path",
    "AttnError",
    "DTYPE_CODES",
    "STATUS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libosattn.so")

STATUS = {
    "ATTN_OK": 0,
    "ATTN_ERR_NULL": -1,
    "ATTN_ERR_SHAPE": -2,
    "ATTN_ERR_HEAD_DIM": -3,
    "ATTN_ERR_GQA": -4,
    "ATTN_ERR_DTYPE": -5,
    "ATTN_ERR_SCALE": -6,
    "ATTN_ERR_ALIGN": -7,
    "ATTN_ERR_WORKSPACE": -8,
    "ATTN_ERR_LAUNCH": -9,
    "ATTN_ERR_SCRATCH": -10,
}
DTYPE_CODES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}

EXPORTED = ("attn_fwd", "attn_bwd", "attn_bwd_workspace_bytes", "attn_bwd_preprocess",
            "attn_bwd_dkdv", "attn_bwd_dq", "attn_fwd_splitkv", "attn_fwd_splitkv_workspace_bytes",
            "attn_fwd_masked", "attn_bwd_masked", "attn_bwd_masked_workspace_bytes",
            "attn_fwd_fp8", "attn_fwd_fp8_workspace_bytes",
            "rowsoftmax_fwd", "rowsoftmax_bwd", "rowxent_fwd", "rowxent_bwd",
            "attn_bwd_noalloc", "attn_status_string")

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def library_path() -> str:
    return _LIB_PATH


def library() -> ctypes.CDLL:
    """Load libosattn.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m online_softmax_attn_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp]
    lib.attn_fwd.restype = i
    lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp,
                             ctypes.c_size_t, vp]
    lib.attn_bwd.restype = i
    lib.attn_bwd_noalloc.argtypes = [vp] * 9 + [i, i, i, i, i, f, i, i, vp]
    lib.attn_bwd_noalloc.restype = i
    sz = ctypes.c_size_t
    lib.attn_bwd_preprocess.argtypes = [vp, vp, vp, i, i, i, i, i, i, vp, sz, vp]
    lib.attn_bwd_preprocess.restype = i
    lib.attn_bwd_dkdv.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp, sz, vp]
    lib.attn_bwd_dkdv.restype = i
    lib.attn_bwd_dq.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp, sz, vp]
    lib.attn_bwd_dq.restype = i
    lib.attn_fwd_masked.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, vp, i, vp]
    lib.attn_fwd_masked.restype = i
    lib.attn_bwd_masked.argtypes = [vp] * 9 + [i, i, i, i, i, i, f, vp, vp, i, vp, sz, vp]
    lib.attn_bwd_masked.restype = i
    lib.attn_bwd_masked_workspace_bytes.argtypes = [i] * 7
    lib.attn_bwd_masked_workspace_bytes.restype = sz
    lib.attn_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, i, vp, sz, vp]
    lib.attn_fwd_splitkv.restype = i
    lib.attn_fwd_splitkv_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i, i]
    lib.attn_fwd_splitkv_workspace_bytes.restype = sz
    lib.attn_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_fwd_fp8.argtypes = [vp] * 5 + [i] * 5 + [f, f, f, f, i, vp, sz, vp]
    lib.attn_fwd_fp8.restype = i
    lib.attn_fwd_fp8_workspace_bytes.argtypes = [i] * 4
    lib.attn_fwd_fp8_workspace_bytes.restype = sz
    ll = ctypes.c_longlong
    lib.rowsoftmax_fwd.argtypes = [vp, vp, ll, i, i, i, vp]
    lib.rowsoftmax_fwd.restype = i
    lib.rowsoftmax_bwd.argtypes = [vp, vp, vp, ll, i, i, i, vp]
    lib.rowsoftmax_bwd.restype = i
    lib.rowxent_fwd.argtypes = [vp, vp, vp, vp, ll, i, i, vp]
    lib.rowxent_fwd.restype = i
    lib.rowxent_bwd.argtypes = [vp, vp, vp, vp, vp, ll, i, i, vp]
    lib.rowxent_bwd.restype = i
    lib.attn_status_string.argtypes = [i]
    lib.attn_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return library().attn_status_string(int(status)).decode()


def _common_device(tensors):
    """The one device the CUDA (ROCm) tensors among `tensors` share, or None if none is."""
    devs = {t.device for t in tensors if t.device.type == "cuda"}
    if len(devs) > 1:
        raise ValueError(f"tensors on more than one device: {sorted(str(d) for d in devs)}")
    return next(iter(devs), None)


def _one_device(fn):
    """Run fn with the device of its tensor arguments current: the library launches on
    the current device, into the stream passed to it, and both must be the tensors'
    device.  Tensors on two devices are refused before anything is enqueued."""
    @functools.wraps(fn)
    def call(*args, **kwargs):
        dev = _common_device([a for a in (*args, *kwargs.values()) if isinstance(a, torch.Tensor)])
        if dev is None:
            return fn(*args, **kwargs)
        with torch.cuda.device(dev):
            return fn(*args, **kwargs)
    return call


def _check_dev(name, t, dtype=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the ROCm device, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _dims(q, k):
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B,H,N,d] and k, v [B,Hkv,N,d]")
    B, H, N, d = q.shape
    if k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError(f"k shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    return B, H, k.shape[1], N, d


def _stream_handle(dev) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def attn_bwd_workspace_bytes(B, H, Hkv, N, d, dtype) -> int:
    code = DTYPE_CODES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(library().attn_bwd_workspace_bytes(B, H, Hkv, N, d, code))


@_one_device
def attn_fwd(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None):
    """O and LSE for q [B,H,N,d], k/v [B,Hkv,N,d]; enqueued on the current stream."""
    lib = library()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(name, t, q.dtype)
    if q.dtype not in DTYPE_CODES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    B, H, Hkv, N, d = _dims(q, k)
    if v.shape != k.shape:
        raise ValueError("v must have the shape of k")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), device=q.device, dtype=torch.float32)
    _check_dev("out", out, q.dtype)
    _check_dev("lse", lse, torch.float32)
    if out.shape != q.shape or lse.shape != (B, H, N):
        raise ValueError("out / lse have the wrong shape")
    st = lib.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                      B, H, Hkv, N, d, float(scale), int(bool(causal)), DTYPE_CODES[q.dtype],
                      _stream_handle(q.device))
    if st != 0:
        raise AttnError(st, "attn_fwd")
    return out, lse


def _bwd_checked(q, k, v, o, lse, do, scale, dq, dk, dv, workspace):
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check_dev(name, t, q.dtype)
    _check_dev("lse", lse, torch.float32)
    B, H, Hkv, N, d = _dims(q, k)
    if v.shape != k.shape or o.shape != q.shape or do.shape != q.shape or lse.shape != (B, H, N):
        raise ValueError("inconsistent shapes")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _check_dev(name, t, q.dtype)
        if t.shape != ref.shape:
            raise ValueError(f"{name} has the wrong shape")
    if workspace is False:  # no workspace taken (the allocation-free call)
        return (B, H, Hkv, N, d), float(scale), dq, dk, dv, None
    if workspace is None:
        workspace = new_bwd_workspace(q, k)
    _check_dev("workspace", workspace)
    return (B, H, Hkv, N, d), float(scale), dq, dk, dv, workspace


@_one_device
def new_bwd_workspace(q, k):
    """An uninitialised device buffer of attn_bwd_workspace_bytes() for these tensors."""
    B, H, Hkv, N, d = _dims(q, k)
    need = attn_bwd_workspace_bytes(B, H, Hkv, N, d, q.dtype)
    return torch.empty(need, device=q.device, dtype=torch.uint8)


def _ws_bytes(ws):
    return ws.numel() * ws.element_size()


@_one_device
def attn_bwd(q, k, v, o, lse, do, causal: bool = False, scale: float | None = None,
             dq=None, dk=None, dv=None, workspace=None):
    """dQ, dK, dV from the forward's O and LSE; enqueued on the current stream."""
    lib = library()
    (B, H, Hkv, N, d), scale, dq, dk, dv, ws = _bwd_checked(q, k, v, o, lse, do, scale, dq, dk,
                                                            dv, workspace)
    st = lib.attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                      do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                      B, H, Hkv, N, d, scale, int(bool(causal)), DTYPE_CODES[q.dtype],
                      ws.data_ptr(), _ws_bytes(ws), _stream_handle(q.device))
    if st != 0:
        raise AttnError(st, "attn_bwd")
    return dq, dk, dv


@_one_device
def attn_bwd_noalloc(q, k, v, o, lse, do, causal: bool = False, scale: float | None = None,
                     dq=None, dk=None, dv=None):
    """attn_bwd without a workspace: the library keeps it in a fixed device array per
    GPU (B*H*N up to 4194304 query rows).  Pass dq, dk, dv to have nothing allocated
    here either.  Calls that may overlap in time on one GPU race on that array."""
    lib = library()
    (B, H, Hkv, N, d), scale, dq, dk, dv, _ = _bwd_checked(q, k, v, o, lse, do, scale, dq, dk,
                                                           dv, False)
    st = lib.attn_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              lse.data_ptr(), do.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                              dv.data_ptr(), B, H, Hkv, N, d, scale, int(bool(causal)),
                              DTYPE_CODES[q.dtype], _stream_handle(q.device))
    if st != 0:
        raise AttnError(st, "attn_bwd_noalloc")
    return dq, dk, dv


@_one_device
def attn_bwd_preprocess(q, k, o, lse, do, workspace):
    """First backward kernel alone: D and LSE*log2(e) into ``workspace``.

    q and k only supply the shapes (nothing is read from them)."""
    lib = library()
    for name, t in (("o", o), ("do", do)):
        _check_dev(name, t, q.dtype)
    _check_dev("lse", lse, torch.float32)
    _check_dev("workspace", workspace)
    B, H, Hkv, N, d = _dims(q, k)
    if o.shape != q.shape or do.shape != q.shape or lse.shape != (B, H, N):
        raise ValueError("inconsistent shapes")
    st = lib.attn_bwd_preprocess(o.data_ptr(), lse.data_ptr(), do.data_ptr(), B, H, Hkv, N, d,
                                 DTYPE_CODES[q.dtype], workspace.data_ptr(), _ws_bytes(workspace),
                                 _stream_handle(q.device))
    if st != 0:
        raise AttnError(st, "attn_bwd_preprocess")
    return workspace


@_one_device
def attn_bwd_dkdv(q, k, v, o, lse, do, workspace, causal: bool = False,
                  scale: float | None = None, dk=None, dv=None):
    """dK/dV kernel alone, after attn_bwd_preprocess filled ``workspace``."""
    lib = library()
    (B, H, Hkv, N, d), scale, _, dk, dv, ws = _bwd_checked(q, k, v, o, lse, do, scale, q, dk, dv,
                                                           workspace)
    st = lib.attn_bwd_dkdv(q.data_ptr(), k.data_ptr(), v.data_ptr(), lse.data_ptr(),
                           do.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Hkv, N, d, scale,
                           int(bool(causal)), DTYPE_CODES[q.dtype], ws.data_ptr(), _ws_bytes(ws),
                           _stream_handle(q.device))
    if st != 0:
        raise AttnError(st, "attn_bwd_dkdv")
    return dk, dv


@_one_device
def attn_bwd_dq(q, k, v, o, lse, do, workspace, causal: bool = False,
                scale: float | None = None, dq=None):
    """dQ kernel alone, after attn_bwd_preprocess filled ``workspace``."""
    lib = library()
    (B, H, Hkv, N, d), scale, dq, _, _, ws = _bwd_checked(q, k, v, o, lse, do, scale, dq, k, v,
                                                          workspace)
    st = lib.attn_bwd_dq(q.data_ptr(), k.data_ptr(), v.data_ptr(), lse.data_ptr(), do.data_ptr(),
                         dq.data_ptr(), B, H, Hkv, N, d, scale, int(bool(causal)),
                         DTYPE_CODES[q.dtype], ws.data_ptr(), _ws_bytes(ws),
                         _stream_handle(q.device))
    if st != 0:
        raise AttnError(st, "attn_bwd_dq")
    return dq


def attn_fwd_splitkv_workspace_bytes(B, H, Hkv, Nq, Nk, d, causal, dtype, n_splits=0) -> int:
    code = DTYPE_CODES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(library().attn_fwd_splitkv_workspace_bytes(B, H, Hkv, Nq, Nk, d, int(bool(causal)),
                                                          code, int(n_splits)))


@_one_device
def attn_fwd_splitkv(q, k, v, causal: bool = False, scale: float | None = None, n_splits: int = 0,
                     out=None, lse=None, workspace=None):
    """Split-KV forward: q [B,H,Nq,d] against k/v [B,Hkv,Nk,d] (Nq may be much smaller
    than Nk; the causal mask is aligned bottom-right).  fp16/bf16 only."""
    lib = library()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(name, t, q.dtype)
    if q.dtype not in DTYPE_CODES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q must be [B,H,Nq,d] and k, v [B,Hkv,Nk,d]")
    B, H, Nq, d = q.shape
    if k.shape[0] != B or k.shape[3] != d:
        raise ValueError(f"k shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    Hkv, Nk = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, Nq), device=q.device, dtype=torch.float32) if lse is None else lse
    _check_dev("out", out, q.dtype)
    _check_dev("lse", lse, torch.float32)
    if out.shape != q.shape or lse.shape != (B, H, Nq):
        raise ValueError("out / lse have the wrong shape")
    if workspace is None:
        need = attn_fwd_splitkv_workspace_bytes(B, H, Hkv, Nq, Nk, d, causal, q.dtype, n_splits)
        workspace = torch.empty(max(need, 1), device=q.device, dtype=torch.uint8)
    _check_dev("workspace", workspace)
    st = lib.attn_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                              lse.data_ptr(), B, H, Hkv, Nq, Nk, d, float(scale), int(bool(causal)),
                              DTYPE_CODES[q.dtype], int(n_splits), workspace.data_ptr(),
                              _ws_bytes(workspace), _stream_handle(q.device))
    if st != 0:
        raise AttnError(st, "attn_fwd_splitkv")
    return out, lse


def _check_intervals(kv_lo, kv_hi, B, Nq):
    for name, t in (("kv_lo", kv_lo), ("kv_hi", kv_hi)):
        _check_dev(name, t, torch.int32)
        if tuple(t.shape) != (B, Nq):
            raise ValueError(f"{name} must be int32 [B, Nq] = {(B, Nq)}, got {tuple(t.shape)}")


@_one_device
def attn_fwd_masked(q, k, v, kv_lo, kv_hi, scale: float | None = None, out=None, lse=None):
    """Forward under per-row visible key intervals: query i of batch b sees keys
    kv_lo[b, i] .. kv_hi[b, i] (int32 [B, Nq] device tensors); k/v may be longer than q."""
    lib = library()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(name, t, q.dtype)
    if q.dtype not in DTYPE_CODES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q must be [B,H,Nq,d] and k, v [B,Hkv,Nk,d]")
    B, H, Nq, d = q.shape
    if k.shape[0] != B or k.shape[3] != d:
        raise ValueError(f"k shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    Hkv, Nk = k.shape[1], k.shape[2]
    _check_intervals(kv_lo, kv_hi, B, Nq)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, Nq), device=q.device, dtype=torch.float32) if lse is None else lse
    _check_dev("out", out, q.dtype)
    _check_dev("lse", lse, torch.float32)
    if out.shape != q.shape or lse.shape != (B, H, Nq):
        raise ValueError("out / lse have the wrong shape")
    st = lib.attn_fwd_masked(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                             lse.data_ptr(), B, H, Hkv, Nq, Nk, d, float(scale), kv_lo.data_ptr(),
                             kv_hi.data_ptr(), DTYPE_CODES[q.dtype], _stream_handle(q.device))
    if st != 0:
        raise AttnError(st, "attn_fwd_masked")
    return out, lse


def attn_bwd_masked_workspace_bytes(B, H, Hkv, Nq, Nk, d, dtype) -> int:
    code = DTYPE_CODES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(library().attn_bwd_masked_workspace_bytes(B, H, Hkv, Nq, Nk, d, code))


@_one_device
def attn_bwd_masked(q, k, v, o, lse, do, kv_lo, kv_hi, scale: float | None = None,
                    dq=None, dk=None, dv=None, workspace=None):
    """dQ, dK, dV under the same per-row key intervals as attn_fwd_masked."""
    lib = library()
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check_dev(name, t, q.dtype)
    _check_dev("lse", lse, torch.float32)
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q must be [B,H,Nq,d] and k, v [B,Hkv,Nk,d]")
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != d or o.shape != q.shape or do.shape != q.shape \
            or lse.shape != (B, H, Nq):
        raise ValueError("inconsistent shapes")
    _check_intervals(kv_lo, kv_hi, B, Nq)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _check_dev(name, t, q.dtype)
        if t.shape != ref.shape:
            raise ValueError(f"{name} has the wrong shape")
    if workspace is None:
        need = attn_bwd_masked_workspace_bytes(B, H, Hkv, Nq, Nk, d, q.dtype)
        workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
    _check_dev("workspace", workspace)
    st = lib.attn_bwd_masked(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                             lse.data_ptr(), do.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                             dv.data_ptr(), B, H, Hkv, Nq, Nk, d, float(scale), kv_lo.data_ptr(),
                             kv_hi.data_ptr(), DTYPE_CODES[q.dtype], workspace.data_ptr(),
                             _ws_bytes(workspace), _stream_handle(q.device))
    if st != 0:
        raise AttnError(st, "attn_bwd_masked")
    return dq, dk, dv


def _rows_of(x):
    if x.dim() < 1 or x.shape[-1] < 1 or x.numel() == 0:
        raise ValueError("need at least one row of at least one element")
    cols = x.shape[-1]
    return x.numel() // cols, cols


@_one_device
def rowsoftmax_fwd(x, log_softmax: bool = False, out=None):
    """Softmax (or log-softmax) of every row of x over its last dimension."""
    lib = library()
    _check_dev("x", x)
    if x.dtype not in DTYPE_CODES:
        raise ValueError(f"unsupported dtype {x.dtype}")
    rows, cols = _rows_of(x)
    out = torch.empty_like(x) if out is None else out
    _check_dev("out", out, x.dtype)
    if out.shape != x.shape:
        raise ValueError("out has the wrong shape")
    st = lib.rowsoftmax_fwd(x.data_ptr(), out.data_ptr(), rows, cols, int(bool(log_softmax)),
                            DTYPE_CODES[x.dtype], _stream_handle(x.device))
    if st != 0:
        raise AttnError(st, "rowsoftmax_fwd")
    return out


@_one_device
def rowsoftmax_bwd(y, dy, log_softmax: bool = False, out=None):
    """Gradient with respect to the rows' input, from the forward's output y and dy."""
    lib = library()
    _check_dev("y", y)
    _check_dev("dy", dy, y.dtype)
    if y.dtype not in DTYPE_CODES:
        raise ValueError(f"unsupported dtype {y.dtype}")
    if dy.shape != y.shape:
        raise ValueError("dy must have y's shape")
    rows, cols = _rows_of(y)
    out = torch.empty_like(y) if out is None else out
    _check_dev("out", out, y.dtype)
    if out.shape != y.shape:
        raise ValueError("out has the wrong shape")
    st = lib.rowsoftmax_bwd(y.data_ptr(), dy.data_ptr(), out.data_ptr(), rows, cols,
                            int(bool(log_softmax)), DTYPE_CODES[y.dtype],
                            _stream_handle(y.device))
    if st != 0:
        raise AttnError(st, "rowsoftmax_bwd")
    return out


def _check_targets(targets, rows):
    _check_dev("targets", targets, torch.int32)
    if targets.numel() != rows:
        raise ValueError(f"targets must hold one int32 per row ({rows}), got {targets.numel()}")


@_one_device
def rowxent_fwd(logits, targets, loss=None, lse=None):
    """Per-row cross-entropy logsumexp(x) - x[target] (0 where the target is outside
    0 .. C-1) and the row logsumexp, both float32 with the rows' shape."""
    lib = library()
    _check_dev("logits", logits)
    if logits.dtype not in DTYPE_CODES:
        raise ValueError(f"unsupported dtype {logits.dtype}")
    rows, cols = _rows_of(logits)
    _check_targets(targets, rows)
    shape = logits.shape[:-1]
    loss = torch.empty(shape, device=logits.device, dtype=torch.float32) if loss is None else loss
    lse = torch.empty(shape, device=logits.device, dtype=torch.float32) if lse is None else lse
    for name, t in (("loss", loss), ("lse", lse)):
        _check_dev(name, t, torch.float32)
        if t.numel() != rows:
            raise ValueError(f"{name} must hold one float32 per row")
    st = lib.rowxent_fwd(logits.data_ptr(), targets.data_ptr(), loss.data_ptr(), lse.data_ptr(),
                         rows, cols, DTYPE_CODES[logits.dtype], _stream_handle(logits.device))
    if st != 0:
        raise AttnError(st, "rowxent_fwd")
    return loss, lse


@_one_device
def rowxent_bwd(logits, targets, lse, dloss, out=None):
    """dlogits = dloss[row] * (softmax(logits) - onehot(target)); zero for ignored rows."""
    lib = library()
    _check_dev("logits", logits)
    if logits.dtype not in DTYPE_CODES:
        raise ValueError(f"unsupported dtype {logits.dtype}")
    rows, cols = _rows_of(logits)
    _check_targets(targets, rows)
    for name, t in (("lse", lse), ("dloss", dloss)):
        _check_dev(name, t, torch.float32)
        if t.numel() != rows:
            raise ValueError(f"{name} must hold one float32 per row")
    out = torch.empty_like(logits) if out is None else out
    _check_dev("out", out, logits.dtype)
    if out.shape != logits.shape:
        raise ValueError("out has the wrong shape")
    st = lib.rowxent_bwd(logits.data_ptr(), targets.data_ptr(), lse.data_ptr(), dloss.data_ptr(),
                         out.data_ptr(), rows, cols, DTYPE_CODES[logits.dtype],
                         _stream_handle(logits.device))
    if st != 0:
        raise AttnError(st, "rowxent_bwd")
    return out


def attn_fwd_fp8_workspace_bytes(B, Hkv, N, d=128) -> int:
    return int(library().attn_fwd_fp8_workspace_bytes(B, Hkv, N, d))


@_one_device
def attn_fwd_fp8(q8, k8, v8, descale_q: float, descale_k: float, descale_v: float,
                 causal: bool = False, scale: float | None = None, out=None, lse=None,
                 workspace=None):
    """Forward over e4m3 codes (uint8 tensors q8 [B,H,N,d], k8/v8 [B,Hkv,N,d], d = 64 or
    128) with per-tensor dequantisation factors; returns O (bf16) and LSE (fp32)."""
    lib = library()
    for name, t in (("q8", q8), ("k8", k8), ("v8", v8)):
        _check_dev(name, t, torch.uint8)
    B, H, Hkv, N, d = _dims(q8, k8)
    if v8.shape != k8.shape:
        raise ValueError("v8 must have k8's shape")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = torch.empty(q8.shape, device=q8.device, dtype=torch.bfloat16) if out is None else out
    lse = torch.empty((B, H, N), device=q8.device, dtype=torch.float32) if lse is None else lse
    _check_dev("out", out, torch.bfloat16)
    _check_dev("lse", lse, torch.float32)
    if out.shape != q8.shape or lse.shape != (B, H, N):
        raise ValueError("out / lse have the wrong shape")
    if workspace is None:
        need = attn_fwd_fp8_workspace_bytes(B, Hkv, N, d)
        workspace = torch.empty(max(need, 1), device=q8.device, dtype=torch.uint8)
    _check_dev("workspace", workspace)
    st = lib.attn_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), out.data_ptr(),
                          lse.data_ptr(), B, H, Hkv, N, d, float(scale), float(descale_q),
                          float(descale_k), float(descale_v), int(bool(causal)),
                          workspace.data_ptr(), _ws_bytes(workspace), _stream_handle(q8.device))
    if st != 0:
        raise AttnError(st, "attn_fwd_fp8")
    return out, lse
