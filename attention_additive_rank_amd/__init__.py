"""Python binding of libflashbias (ctypes): the same entry points as ``include/fb.h``.

Attention with an additive bias on AMD Instinct MI355X (gfx950),
O = softmax(s Q K^T + b) V, with b given as low-rank factors (FlashBias) or as a
dense tensor.  This module only marshals arguments: PyTorch provides device
memory and the current HIP stream, every step of the computation runs in the
library's HIP kernels (or, for ``fb_svd_factors``, its host C++ code).  There is
no fallback: if ``libflashbias.so`` is missing or fails to load, every call
raises ``RuntimeError``.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading
from typing import Optional, Tuple

import numpy as np

__all__ = [
    "FbError", "load", "library_path", "fb_status_str", "fb_last_error",
    "fb_make_factors", "fb_make_factors_log2", "fb_make_dense_bias", "fb_svd_factors",
    "fb_attn_fwd_lowrank", "fb_attn_fwd_lowrank_log2", "fb_attn_fwd_densebias",
    "FB_ALIBI", "FB_SANDWICH", "factor_columns",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libflashbias.so")

FB_OK, FB_EINVAL, FB_EUNSUPPORTED, FB_EHIP, FB_ENOMEM = range(5)
FB_F32, FB_BF16, FB_F16 = 0, 1, 2
FB_ALIBI, FB_SANDWICH = 0, 1

_lib = None
_lock = threading.Lock()


class FbError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class _AttnArgs(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int), ("H", ctypes.c_int), ("N", ctypes.c_int), ("D", ctypes.c_int),
        ("dt", ctypes.c_int), ("causal", ctypes.c_int), ("scale", ctypes.c_float),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("o", ctypes.c_void_p),
        ("sq", ctypes.c_int64 * 3), ("sk", ctypes.c_int64 * 3), ("sv", ctypes.c_int64 * 3),
        ("so", ctypes.c_int64 * 3), ("lse", ctypes.c_void_p),
    ]


_I64x3 = ctypes.c_int64 * 3
_DP = ctypes.POINTER(ctypes.c_double)


class _BwdArgs(ctypes.Structure):
    _fields_ = [
        ("dout", ctypes.c_void_p), ("sdo", _I64x3),
        ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
        ("sdq", _I64x3), ("sdk", _I64x3), ("sdv", _I64x3),
        ("dphi_q", ctypes.c_void_p), ("dphi_k", ctypes.c_void_p), ("sdphi_q", _I64x3), ("sdphi_k", _I64x3),
        ("work", ctypes.c_void_p), ("work_bytes", ctypes.c_size_t),
    ]


def load():
    """Load libflashbias.so (once).  Raises RuntimeError if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(library_path):
            raise RuntimeError(f"{library_path} is not built; run `python -m attention_additive_rank_amd.build` "
                               "or __graft_entry__.build()")
        lib = ctypes.CDLL(library_path)
        lib.fb_status_str.restype = ctypes.c_char_p
        lib.fb_status_str.argtypes = [ctypes.c_int]
        lib.fb_last_error.restype = ctypes.c_char_p
        lib.fb_last_error.argtypes = []
        for fn in (lib.fb_make_factors, lib.fb_make_factors_log2):
            fn.restype = ctypes.c_int
            fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, _DP, ctypes.c_int,
                           ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                           ctypes.POINTER(ctypes.c_int), ctypes.c_void_p]
        lib.fb_make_dense_bias.restype = ctypes.c_int
        lib.fb_make_dense_bias.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, _DP,
                                           ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                           ctypes.c_void_p]
        for fn in (lib.fb_svd_factors, lib.fb_svd_factors_log2):
            fn.restype = ctypes.c_int
            fn.argtypes = [_DP, ctypes.c_int, ctypes.c_int, ctypes.c_uint64, _DP, _DP, _DP, _DP]
        lib.fb_svd_rank_for_energy.restype = ctypes.c_int
        lib.fb_svd_rank_for_energy.argtypes = [_DP, ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_uint64,
                                               ctypes.POINTER(ctypes.c_int), _DP, ctypes.POINTER(ctypes.c_int)]
        for fn in (lib.fb_attn_fwd_lowrank, lib.fb_attn_fwd_lowrank_log2):
            fn.restype = ctypes.c_int
            fn.argtypes = [ctypes.POINTER(_AttnArgs), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                           ctypes.POINTER(_I64x3), ctypes.POINTER(_I64x3), ctypes.c_void_p]
        for fn in (lib.fb_attn_bwd_lowrank, lib.fb_attn_bwd_lowrank_log2, lib.fb_attn_bwd_lowrank_noalloc):
            fn.restype = ctypes.c_int
            fn.argtypes = [ctypes.POINTER(_AttnArgs), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                           ctypes.POINTER(_I64x3), ctypes.POINTER(_I64x3), ctypes.POINTER(_BwdArgs), ctypes.c_void_p]
        lib.fb_attn_fwd_alibi.restype = ctypes.c_int
        lib.fb_attn_fwd_alibi.argtypes = [ctypes.POINTER(_AttnArgs), _DP, ctypes.c_void_p]
        lib.fb_attn_fwd_sandwich.restype = ctypes.c_int
        lib.fb_attn_fwd_sandwich.argtypes = [ctypes.POINTER(_AttnArgs), ctypes.c_int, ctypes.c_void_p]
        lib.fb_attn_fwd_mulbias.restype = ctypes.c_int
        lib.fb_attn_fwd_mulbias.argtypes = [ctypes.POINTER(_AttnArgs), ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_int, ctypes.c_int, ctypes.POINTER(_I64x3),
                                            ctypes.POINTER(_I64x3), ctypes.c_void_p, ctypes.c_size_t,
                                            ctypes.c_void_p]
        lib.fb_mulbias_expand.restype = ctypes.c_int
        lib.fb_mulbias_expand.argtypes = lib.fb_attn_fwd_mulbias.argtypes
        lib.fb_attn_bwd_workspace_bytes.restype = ctypes.c_size_t
        lib.fb_attn_bwd_workspace_bytes.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                    ctypes.POINTER(_I64x3), ctypes.POINTER(_I64x3)]
        lib.fb_mulbias_workspace_bytes.restype = ctypes.c_size_t
        lib.fb_mulbias_workspace_bytes.argtypes = [ctypes.POINTER(_AttnArgs), ctypes.c_int]
        lib.fb_attn_fwd_densebias.restype = ctypes.c_int
        lib.fb_attn_fwd_densebias.argtypes = [ctypes.POINTER(_AttnArgs), ctypes.c_void_p, ctypes.c_int,
                                              ctypes.POINTER(_I64x3), ctypes.c_void_p]
        _lib = lib
    return _lib


def fb_status_str(status: int) -> str:
    return load().fb_status_str(status).decode()


def fb_last_error() -> str:
    return load().fb_last_error().decode()


def _check(status: int):
    if status != FB_OK:
        raise FbError(status, f"{fb_status_str(status)}: {fb_last_error()}")


# ------------------------------------------------------------ torch glue ----
def _torch():
    import torch
    return torch


def _dt_code(dtype) -> int:
    torch = _torch()
    m = {torch.float32: FB_F32, torch.bfloat16: FB_BF16, torch.float16: FB_F16}
    if dtype not in m:
        raise TypeError(f"unsupported dtype {dtype}")
    return m[dtype]


def _stream_ptr(device, stream=None) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return s.cuda_stream


def _kind_code(kind) -> int:
    if isinstance(kind, str):
        return {"alibi": FB_ALIBI, "sandwich": FB_SANDWICH}[kind.lower()]
    return int(kind)


def factor_columns(kind, C: int = 0, split: int = 1) -> int:
    """Number of factor columns fb_make_factors writes (natural rank x split(split+1)/2)."""
    r = 2 if _kind_code(kind) == FB_ALIBI else C
    return r * split * (split + 1) // 2


def _slopes_ptr(slopes):
    if slopes is None:
        return None, None
    arr = np.ascontiguousarray(np.asarray(slopes, dtype=np.float64))
    return arr, arr.ctypes.data_as(_DP)


def fb_make_factors(kind, H: int, N: int, C: int = 0, slopes=None, dtype=None, split: int = 1,
                    R_pad: Optional[int] = None, phi_q=None, phi_k=None, device="cuda", stream=None):
    """Exact ALiBi / Sandwich factors on the GPU.  Returns ``(phi_q, phi_k, R_used)`` with
    ``phi_*`` of shape ``[H, N, R_pad]`` (allocated here if not given).  R_pad defaults to
    R_used rounded up to whole 16-byte rows (zero columns past R_used), the width with
    which the attention kernels copy phi_k rows straight into on-chip memory."""
    return _make_factors("fb_make_factors", kind, H, N, C, slopes, dtype, split, R_pad, phi_q, phi_k, device, stream)


def fb_make_factors_log2(kind, H: int, N: int, C: int = 0, slopes=None, dtype=None, split: int = 1,
                         R_pad: Optional[int] = None, phi_q=None, phi_k=None, device="cuda", stream=None):
    """As :func:`fb_make_factors` with ``phi_q`` in exp2 units (times log2(e) before rounding),
    the factors :func:`fb_attn_fwd_lowrank_log2` takes."""
    return _make_factors("fb_make_factors_log2", kind, H, N, C, slopes, dtype, split, R_pad, phi_q, phi_k, device,
                         stream)


def _make_factors(entry, kind, H, N, C, slopes, dtype, split, R_pad, phi_q, phi_k, device, stream):
    torch = _torch()
    dtype = dtype or torch.bfloat16
    used = factor_columns(kind, C, split)
    if phi_q is None or phi_k is None:
        if R_pad is None:
            ce = 16 // torch.empty((), dtype=dtype).element_size()
            R_pad = (used + ce - 1) // ce * ce
        phi_q = torch.empty((H, N, R_pad), dtype=dtype, device=device)
        phi_k = torch.empty((H, N, R_pad), dtype=dtype, device=device)
    else:
        R_pad = phi_q.shape[-1]
        if phi_q.shape != (H, N, R_pad) or phi_k.shape != (H, N, R_pad) or not (phi_q.is_contiguous() and phi_k.is_contiguous()):
            raise ValueError("phi_q / phi_k must be contiguous [H, N, R_pad]")
    keep, sp = _slopes_ptr(slopes)
    r_used = ctypes.c_int(0)
    st = getattr(load(), entry)(_kind_code(kind), H, N, C, sp, _dt_code(phi_q.dtype), split, phi_q.data_ptr(),
                                phi_k.data_ptr(), R_pad, ctypes.byref(r_used), _stream_ptr(phi_q.device, stream))
    _check(st)
    return phi_q, phi_k, r_used.value


def fb_make_dense_bias(kind, H: int, N: int, C: int = 0, slopes=None, dtype=None, out=None, device="cuda",
                       stream=None):
    """Dense closed-form bias ``[H, N, N]`` on the GPU (fp64 arithmetic, rounded once)."""
    torch = _torch()
    if out is None:
        out = torch.empty((H, N, N), dtype=dtype or torch.bfloat16, device=device)
    if out.dim() != 3 or out.shape[0] != H or out.shape[1] != N or out.shape[2] != N or out.stride(2) != 1:
        raise ValueError("out must be [H, N, N] with a contiguous last axis")
    keep, sp = _slopes_ptr(slopes)
    st = load().fb_make_dense_bias(_kind_code(kind), H, N, C, sp, _dt_code(out.dtype), out.data_ptr(),
                                   out.stride(0), out.stride(1), _stream_ptr(out.device, stream))
    _check(st)
    return out


def fb_svd_factors(bias: np.ndarray, R: int, seed: int = 0, log2: bool = False):
    """Host truncated SVD of one ``[N, N]`` bias.  Returns a dict with ``phi_q``, ``phi_k``
    (``[N, R]`` fp64), ``sigma`` (``[R]``) and ``energy`` (retained energy).  ``log2``:
    ``phi_q`` in exp2 units (fb_svd_factors_log2), the factors fb_attn_fwd_lowrank_log2 takes."""
    a = np.ascontiguousarray(np.asarray(bias, dtype=np.float64))
    if a.ndim != 2 or a.shape[0] != a.shape[1]:
        raise ValueError("bias must be a square [N, N] matrix")
    N = a.shape[0]
    pq = np.empty((N, R))
    pk = np.empty((N, R))
    sig = np.empty(R)
    en = ctypes.c_double(0.0)
    fn = load().fb_svd_factors_log2 if log2 else load().fb_svd_factors
    st = fn(a.ctypes.data_as(_DP), N, R, seed, pq.ctypes.data_as(_DP), pk.ctypes.data_as(_DP),
            sig.ctypes.data_as(_DP), ctypes.byref(en))
    _check(st)
    return {"phi_q": pq, "phi_k": pk, "sigma": sig, "energy": en.value}


def fb_svd_rank_for_energy(bias: np.ndarray, target: float = 0.95, R_max: Optional[int] = None, seed: int = 0):
    """Smallest rank whose truncated SVD keeps ``target`` of the bias energy (host).
    Returns a dict with ``R``, ``energy`` (kept by ``R``) and ``reached`` (bool)."""
    a = np.ascontiguousarray(np.asarray(bias, dtype=np.float64))
    if a.ndim != 2 or a.shape[0] != a.shape[1]:
        raise ValueError("bias must be a square [N, N] matrix")
    N = a.shape[0]
    R_max = min(N, 64) if R_max is None else int(R_max)
    r = ctypes.c_int(0)
    en = ctypes.c_double(0.0)
    ok = ctypes.c_int(0)
    st = load().fb_svd_rank_for_energy(a.ctypes.data_as(_DP), N, R_max, float(target), seed, ctypes.byref(r),
                                       ctypes.byref(en), ctypes.byref(ok))
    _check(st)
    return {"R": r.value, "energy": en.value, "reached": bool(ok.value)}


def _attn_args(q, k, v, out, lse, causal, scale):
    B, H, N, D = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if t.dim() != 4 or tuple(t.shape) != (B, H, N, D):
            raise ValueError(f"{name} must have shape {(B, H, N, D)}")
        if t.stride(3) != 1 and N * B * H > 0:
            raise ValueError(f"{name} must have a contiguous last axis")
        if t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{name} dtype/device differs from q")
    a = _AttnArgs()
    a.B, a.H, a.N, a.D = B, H, N, D
    a.dt = _dt_code(q.dtype)
    a.causal = 1 if causal else 0
    a.scale = float(1.0 / math.sqrt(D) if scale is None else scale)
    a.q, a.k, a.v, a.o = q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr()
    a.sq = _I64x3(*q.stride()[:3])
    a.sk = _I64x3(*k.stride()[:3])
    a.sv = _I64x3(*v.stride()[:3])
    a.so = _I64x3(*out.stride()[:3])
    if lse is not None:
        if tuple(lse.shape) != (B, H, N) or not lse.is_contiguous() or lse.dtype != _torch().float32:
            raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")
        a.lse = lse.data_ptr()
    else:
        a.lse = None
    return a


def _bhn_strides(t, B, H, N, name):
    """Element strides (b, h, n) of a factor / bias tensor broadcastable to [B, H, N, X]."""
    if t.dim() == 2:
        t = t.unsqueeze(0).unsqueeze(0)
    elif t.dim() == 3:
        t = t.unsqueeze(0)
    if t.dim() != 4:
        raise ValueError(f"{name} must have 2, 3 or 4 dims")
    e = t.expand(B, H, N, t.shape[-1])
    if e.stride(3) != 1 and t.shape[-1] > 1:
        raise ValueError(f"{name} must have a contiguous last axis")
    return e, _I64x3(*e.stride()[:3])


def fb_attn_fwd_lowrank(q, k, v, phi_q=None, phi_k=None, *, causal: bool = False, scale: Optional[float] = None,
                        out=None, lse=None, stream=None):
    """O = softmax(scale * Q K^T + phi_q phi_k^T) V (fused; no N x N bias formed).

    ``q, k, v``: ``[B, H, N, D]`` device tensors (fp32 / bf16 / fp16, contiguous last axis).
    ``phi_q, phi_k``: ``[..., N, R]`` broadcastable to ``[B, H, N, R]`` (or None for R = 0).
    ``scale`` defaults to 1/sqrt(D).  ``lse``: optional float32 ``[B, H, N]`` output."""
    return _lowrank("fb_attn_fwd_lowrank", q, k, v, phi_q, phi_k, causal, scale, out, lse, stream)


def fb_attn_fwd_lowrank_log2(q, k, v, phi_q=None, phi_k=None, *, causal: bool = False,
                             scale: Optional[float] = None, out=None, lse=None, stream=None):
    """O = softmax(scale * Q K^T + ln(2) phi_q phi_k^T) V: ``phi_q`` in exp2 units (as
    :func:`fb_make_factors_log2` writes it); bf16 / fp16 only.  Otherwise as
    :func:`fb_attn_fwd_lowrank`."""
    return _lowrank("fb_attn_fwd_lowrank_log2", q, k, v, phi_q, phi_k, causal, scale, out, lse, stream)


def _lowrank(entry, q, k, v, phi_q, phi_k, causal, scale, out, lse, stream):
    torch = _torch()
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    a = _attn_args(q, k, v, out, lse, causal, scale)
    B, H, N, _ = q.shape
    if phi_q is None or phi_k is None or phi_q.shape[-1] == 0:
        st = getattr(load(), entry)(ctypes.byref(a), None, None, a.dt, 0, None, None, _stream_ptr(q.device, stream))
    else:
        if phi_q.shape[-1] != phi_k.shape[-1]:
            raise ValueError("phi_q and phi_k need the same rank")
        if phi_q.dtype != phi_k.dtype or phi_q.device != q.device or phi_k.device != q.device:
            raise ValueError("phi_q / phi_k dtype or device mismatch")
        eq, sq = _bhn_strides(phi_q, B, H, N, "phi_q")
        ek, sk = _bhn_strides(phi_k, B, H, N, "phi_k")
        st = getattr(load(), entry)(ctypes.byref(a), eq.data_ptr(), ek.data_ptr(), _dt_code(phi_q.dtype),
                                    phi_q.shape[-1], ctypes.byref(sq), ctypes.byref(sk), _stream_ptr(q.device, stream))
    _check(st)
    return out


def fb_attn_fwd_densebias(q, k, v, bias, *, causal: bool = False, scale: Optional[float] = None, out=None,
                          lse=None, stream=None):
    """O = softmax(scale * Q K^T + bias) V with the bias streamed from HBM (the baseline).

    ``bias``: ``[..., N, N]`` broadcastable to ``[B, H, N, N]``, dtype of q, contiguous last axis."""
    torch = _torch()
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    a = _attn_args(q, k, v, out, lse, causal, scale)
    B, H, N, _ = q.shape
    if bias.shape[-1] != N or bias.shape[-2] != N:
        raise ValueError("bias must end in [N, N]")
    if bias.device != q.device:
        raise ValueError("bias device differs from q")
    eb, sb = _bhn_strides(bias, B, H, N, "bias")
    st = load().fb_attn_fwd_densebias(ctypes.byref(a), eb.data_ptr(), _dt_code(bias.dtype), ctypes.byref(sb),
                                      _stream_ptr(q.device, stream))
    _check(st)
    return out


def fb_mulbias_workspace_bytes(q, R: int) -> int:
    """Device workspace (bytes) that fb_attn_fwd_mulbias needs for q's shape and rank R."""
    a = _AttnArgs()
    a.B, a.H, a.N, a.D = q.shape
    a.dt = _dt_code(q.dtype)
    return int(load().fb_mulbias_workspace_bytes(ctypes.byref(a), int(R)))


def fb_attn_fwd_mulbias(q, k, v, phi_q, phi_k, *, causal: bool = False, scale: Optional[float] = None, out=None,
                        lse=None, workspace=None, stream=None):
    """O = softmax((scale * Q K^T) * (phi_q phi_k^T)) V: attention with a multiplicative
    rank-R bias, through operand expansion to width D R and the fused low-rank kernel.

    ``phi_q, phi_k``: ``[..., N, R]`` broadcastable to ``[B, H, N, R]`` (fp32 / bf16 / fp16).
    ``workspace``: optional uint8 device tensor of at least fb_mulbias_workspace_bytes(q, R)
    bytes (allocated here when None)."""
    torch = _torch()
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    a = _attn_args(q, k, v, out, lse, causal, scale)
    B, H, N, _ = q.shape
    if phi_q.shape[-1] != phi_k.shape[-1]:
        raise ValueError("phi_q and phi_k need the same rank")
    if phi_q.dtype != phi_k.dtype or phi_q.device != q.device or phi_k.device != q.device:
        raise ValueError("phi_q / phi_k dtype or device mismatch")
    R = phi_q.shape[-1]
    need = fb_mulbias_workspace_bytes(q, R)
    if workspace is None:
        workspace = torch.empty(max(need, 1) + 256, dtype=torch.uint8, device=q.device)
    base = workspace.data_ptr()
    off = (-base) % 256
    eq, sq = _bhn_strides(phi_q, B, H, N, "phi_q")
    ek, sk = _bhn_strides(phi_k, B, H, N, "phi_k")
    st = load().fb_attn_fwd_mulbias(ctypes.byref(a), eq.data_ptr(), ek.data_ptr(), _dt_code(phi_q.dtype), R,
                                    ctypes.byref(sq), ctypes.byref(sk), base + off, workspace.numel() - off,
                                    _stream_ptr(q.device, stream))
    _check(st)
    return out


def fb_mulbias_expand(q, k, phi_q, phi_k, *, scale: Optional[float] = None, workspace=None, stream=None):
    """The expansion stage of fb_attn_fwd_mulbias alone.  Returns a dict of views into the
    workspace: ``q1`` (= scale * q * phi_q[..., 0]) and ``k1`` (``[B, H, N, D]``), ``phi_q`` and
    ``phi_k`` (``[B, H, N, (R - 1) D]``, the remaining expanded columns, None for R = 1), and the
    ``workspace`` tensor; fb_attn_fwd_lowrank(q1, k1, v, phi_q, phi_k, scale=1) then gives the
    same output as fb_attn_fwd_mulbias."""
    torch = _torch()
    B, H, N, D = q.shape
    R = phi_q.shape[-1]
    need = fb_mulbias_workspace_bytes(q, R)
    if workspace is None:
        workspace = torch.empty(max(need, 1) + 256, dtype=torch.uint8, device=q.device)
    off = (-workspace.data_ptr()) % 256
    dummy_out = q  # never written by the expansion
    a = _attn_args(q, k, k, dummy_out, None, False, scale)
    eq, sq = _bhn_strides(phi_q, B, H, N, "phi_q")
    ek, sk = _bhn_strides(phi_k, B, H, N, "phi_k")
    st = load().fb_mulbias_expand(ctypes.byref(a), eq.data_ptr(), ek.data_ptr(), _dt_code(phi_q.dtype), R,
                                  ctypes.byref(sq), ctypes.byref(sk), workspace.data_ptr() + off,
                                  workspace.numel() - off, _stream_ptr(q.device, stream))
    _check(st)
    es = q.element_size()
    up = lambda x: (x + 255) // 256 * 256
    E = B * H * N
    A = up(E * D * es)
    W = (R - 1) * D

    def view(byte_off, cols):
        if cols == 0:
            return None
        n = E * cols
        return workspace[off + byte_off: off + byte_off + n * es].view(q.dtype).view(B, H, N, cols)
    return {"q1": view(0, D), "k1": view(A, D), "phi_q": view(2 * A, W), "phi_k": view(2 * A + up(E * W * es), W),
            "workspace": workspace}


def fb_attn_bwd_lowrank(q, k, v, out, lse, dout, phi_q=None, phi_k=None, *, causal: bool = False,
                        scale: Optional[float] = None, dq=None, dk=None, dv=None, dphi_q=None, dphi_k=None,
                        stream=None, noalloc: bool = False, log2: bool = False):
    """Gradients of fb_attn_fwd_lowrank's output for the upstream gradient ``dout``.

    ``out`` and ``lse`` are the forward's output and LSE (float32 ``[B, H, N]``).  Returns
    ``(dq, dk, dv, dphi_q, dphi_k)``; the factor gradients are float32 with the factors'
    own shapes (summed over the axes a factor is broadcast on), None for R = 0.
    ``noalloc``: call fb_attn_bwd_lowrank_noalloc, whose workspace is the library's device
    scratch (with every output passed in, this wrapper then allocates nothing either).
    ``log2``: the factors are fb_attn_fwd_lowrank_log2's (phi_q in exp2 units; the gradients
    are with respect to them): fb_attn_bwd_lowrank_log2."""
    torch = _torch()
    B, H, N, D = q.shape
    dq = torch.empty_like(q, memory_format=torch.contiguous_format) if dq is None else dq
    dk = torch.empty_like(k, memory_format=torch.contiguous_format) if dk is None else dk
    dv = torch.empty_like(v, memory_format=torch.contiguous_format) if dv is None else dv
    a = _attn_args(q, k, v, out, lse, causal, scale)
    if lse is None:
        raise ValueError("the forward LSE is required")
    g = _BwdArgs()
    for name, t in (("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{name} must match q in shape, dtype and device")
        setattr(g, name, t.data_ptr())
        setattr(g, "s" + ("do" if name == "dout" else name), _I64x3(*t.stride()[:3]))
    dpq = dpk = None
    R = 0 if (phi_q is None or phi_k is None) else phi_q.shape[-1]
    if R > 0:
        if phi_q.shape[-1] != phi_k.shape[-1] or phi_q.dtype != phi_k.dtype:
            raise ValueError("phi_q / phi_k rank or dtype mismatch")
        eq, sq = _bhn_strides(phi_q, B, H, N, "phi_q")
        ek, sk = _bhn_strides(phi_k, B, H, N, "phi_k")
        dpq = torch.empty(phi_q.shape, dtype=torch.float32, device=q.device) if dphi_q is None else dphi_q
        dpk = torch.empty(phi_k.shape, dtype=torch.float32, device=q.device) if dphi_k is None else dphi_k
        for name, t, f in (("dphi_q", dpq, phi_q), ("dphi_k", dpk, phi_k)):
            if tuple(t.shape) != tuple(f.shape) or t.dtype != torch.float32 or t.device != q.device:
                raise ValueError(f"{name} must be float32 with the factor's shape, on q's device")
        _, gsq = _bhn_strides(dpq, B, H, N, "dphi_q")
        _, gsk = _bhn_strides(dpk, B, H, N, "dphi_k")
        g.dphi_q, g.dphi_k, g.sdphi_q, g.sdphi_k = dpq.data_ptr(), dpk.data_ptr(), gsq, gsk
    work = None
    if noalloc:
        if log2:
            raise ValueError("the no-alloc backward takes natural-unit factors")
        entry = load().fb_attn_bwd_lowrank_noalloc
        g.work, g.work_bytes = None, 0
    else:
        # workspace (Delta and per-(b, h) partials of summed factor gradients), 256-byte aligned
        entry = load().fb_attn_bwd_lowrank_log2 if log2 else load().fb_attn_bwd_lowrank
        nbytes = int(load().fb_attn_bwd_workspace_bytes(B, H, N, R, ctypes.byref(g.sdphi_q), ctypes.byref(g.sdphi_k)))
        work = torch.empty(nbytes + 256, dtype=torch.uint8, device=q.device)
        g.work = (work.data_ptr() + 255) // 256 * 256
        g.work_bytes = nbytes
    if R > 0:
        st = entry(ctypes.byref(a), eq.data_ptr(), ek.data_ptr(), _dt_code(phi_q.dtype), R, ctypes.byref(sq),
                   ctypes.byref(sk), ctypes.byref(g), _stream_ptr(q.device, stream))
    else:
        st = entry(ctypes.byref(a), None, None, a.dt, 0, None, None, ctypes.byref(g), _stream_ptr(q.device, stream))
    _check(st)
    if stream is not None and work is not None:
        work.record_stream(stream)   # the workspace outlives this call on a caller's stream
    return dq, dk, dv, dpq, dpk


def fb_attn_bwd_workspace_bytes(B: int, H: int, N: int, R: int, sdphi_q=(0, 0, 0), sdphi_k=(0, 0, 0)) -> int:
    """Device workspace (bytes) that fb_attn_bwd_lowrank needs; strides of the fp32 factor
    gradients in (batch, head, row) order (a 0 stride sums over that axis)."""
    return int(load().fb_attn_bwd_workspace_bytes(int(B), int(H), int(N), int(R), ctypes.byref(_I64x3(*sdphi_q)),
                                                  ctypes.byref(_I64x3(*sdphi_k))))


def fb_attn_fwd_alibi(q, k, v, slopes=None, *, causal: bool = False, scale: Optional[float] = None, out=None,
                      lse=None, stream=None):
    """O = softmax(scale * Q K^T + m_h (j - i)) V with the ALiBi factors formed inside the
    kernel (no factor tensors).  ``slopes``: H host values or None for 2^(-8(h+1)/H)."""
    torch = _torch()
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    a = _attn_args(q, k, v, out, lse, causal, scale)
    if slopes is not None and len(np.asarray(slopes).reshape(-1)) != q.shape[1]:
        raise ValueError("one slope per head")
    keep, sp = _slopes_ptr(slopes)
    st = load().fb_attn_fwd_alibi(ctypes.byref(a), sp, _stream_ptr(q.device, stream))
    del keep
    _check(st)
    return out


def fb_attn_fwd_sandwich(q, k, v, C: int = 64, *, causal: bool = False, scale: Optional[float] = None, out=None,
                         lse=None, stream=None):
    """O = softmax(scale * Q K^T + b) V for the Sandwich bias b_ij = sum_k cos((i - j) w_k) with
    its cos / sin factors formed inside the kernel (no factor tensors).  ``C``: even channel
    count, 2..64; bf16 / fp16, head dim <= 64."""
    torch = _torch()
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    a = _attn_args(q, k, v, out, lse, causal, scale)
    st = load().fb_attn_fwd_sandwich(ctypes.byref(a), int(C), _stream_ptr(q.device, stream))
    _check(st)
    return out
