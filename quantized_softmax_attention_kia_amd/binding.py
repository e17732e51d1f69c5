"""Python binding of libkia (include/kia.h): argument marshalling only.

Every step of the operator runs in the HIP kernels of libkia.so; this module
checks tensors, turns them into device pointers and passes the caller's
current HIP stream.  PyTorch is used for device memory and streams.  If the
library is not built this module fails at import.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkia.so")

KIA_OK = 0
STATUS = {0: "KIA_OK", -1: "KIA_ERR_INVALID_ARG", -2: "KIA_ERR_UNSUPPORTED", -3: "KIA_ERR_WORKSPACE",
          -4: "KIA_ERR_HIP"}
CALIB = {"minmax": 0, "fwm": 1}
RECON = {"lerp": 0, "nearest": 1, "softmax": 2, "exp_bf16": 3, "exp_fp8": 4, "binmean": 5, "nearest_binmean": 6}
STE = {"weight": 0, "prob": 1}
GRAD = {"full": 0, "detached": 1, "max_only": 2, "min_only": 3, "p1": 4}
DTYPE = {torch.float32: 0, torch.bfloat16: 1}
TAIL = {"zero": 0, "floor": 1, "resolved": 2}


class KiaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


class Params(ctypes.Structure):
    """Mirror of kia_params_t."""
    _fields_ = [("B", ctypes.c_int64), ("H", ctypes.c_int64), ("T", ctypes.c_int64), ("D", ctypes.c_int64),
                ("causal", ctypes.c_int32), ("K", ctypes.c_int32), ("tau", ctypes.c_float),
                ("scale", ctypes.c_float), ("calib", ctypes.c_int32), ("recon", ctypes.c_int32),
                ("ste", ctypes.c_int32), ("grad", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("tail", ctypes.c_int32)]


EXPORTS = ("kia_workspace_size", "kia_forward", "kia_forward_scores", "kia_forward_weights", "kia_backward", "kia_backward_dq", "kia_backward_dkdv",
           "kia_backward_noalloc", "kia_flash_forward", "kia_flash_backward", "kia_debug_bins",
           "kia_status_string", "kia_last_error")
NOALLOC_WS_BYTES = 64 << 20  # KIA_NOALLOC_WS_BYTES


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"libkia.so is not built ({path}); run python -m quantized_softmax_attention_kia_amd.build")
    lib = ctypes.CDLL(path)
    vp, sz = ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t)
    P = ctypes.POINTER(Params)
    lib.kia_workspace_size.argtypes = [P, sz, sz]
    lib.kia_forward.argtypes = [P, vp, vp, vp, vp, vp, vp]
    lib.kia_forward_scores.argtypes = [P, vp, vp, vp, vp, vp]
    lib.kia_forward_weights.argtypes = [P, vp, vp, vp, vp, vp, vp]
    lib.kia_backward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.kia_backward_dq.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.kia_backward_dkdv.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.kia_backward_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.kia_flash_forward.argtypes = [P, vp, vp, vp, vp, vp, vp]
    lib.kia_flash_backward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.kia_debug_bins.argtypes = [P, vp, vp, vp]
    for f in ("kia_workspace_size", "kia_forward", "kia_forward_scores", "kia_forward_weights", "kia_backward",
              "kia_backward_dq", "kia_backward_dkdv", "kia_backward_noalloc", "kia_flash_forward",
              "kia_flash_backward", "kia_debug_bins"):
        getattr(lib, f).restype = ctypes.c_int
    lib.kia_status_string.argtypes = [ctypes.c_int]
    lib.kia_status_string.restype = ctypes.c_char_p
    lib.kia_last_error.argtypes = []
    lib.kia_last_error.restype = ctypes.c_char_p
    return lib


_lib = load_library()


def _check(status: int) -> None:
    if status != KIA_OK:
        raise KiaError(status, _lib.kia_last_error().decode())


@dataclass(frozen=True)
class Config:
    """Operator variant: calibration x reconstruction x surrogate x gradient mode."""
    calib: str = "minmax"
    recon: str = "lerp"
    ste: str = "prob"
    grad: str = "full"
    K: int = 4
    tau: float = 8.0
    causal: bool = True
    scale: float = 0.0     # 0 selects 1/sqrt(D)
    tail: str = "zero"     # FWM tail policy: zero, floor or resolved

    @classmethod
    def of(cls, v, causal=True, scale=0.0):
        return cls(v.calib, v.recon, v.ste, v.grad, int(v.K), float(v.tau), causal, scale, getattr(v, "tail", "zero"))


def make_params(cfg: Config, shape, dtype) -> Params:
    B, H, T, D = (int(x) for x in shape)
    return Params(B, H, T, D, int(bool(cfg.causal)), int(cfg.K), float(cfg.tau), float(cfg.scale),
                  CALIB[cfg.calib], RECON[cfg.recon], STE[cfg.ste], GRAD[cfg.grad], DTYPE[dtype], TAIL[cfg.tail])


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr() if t is not None and t.numel() > 0 else 0)


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


_DTYPE_OF = {v: k for k, v in DTYPE.items()}


def _check_inputs(p: Params, *tensors, outputs=(), rowrec=None, workspace=None):
    """Every input [B,H,T,D], contiguous, of the params' dtype, on one GPU; every output the same
    shape in float32 on that GPU; the record and workspace at least the sizes the library asks for.
    The kernels read buffers through raw pointers: a mismatch here would be an out-of-bounds access."""
    shape = (p.B, p.H, p.T, p.D)
    want = _DTYPE_OF.get(p.dtype)
    dev = tensors[0].device if tensors else None
    for t in tensors:
        if tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"expected contiguous [B,H,T,D]={shape}, got {tuple(t.shape)}")
        if t.dtype != want:
            raise ValueError(f"expected {want} inputs (params dtype), got {t.dtype}")
    for t in outputs:
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != shape or not t.is_contiguous()):
            raise ValueError(f"outputs must be contiguous float32 [B,H,T,D]={shape}, got {t.dtype} {tuple(t.shape)}")
    bufs = []
    if rowrec is not None or workspace is not None:
        rr, ws = kia_workspace_size(p)
        for name, buf, need in (("rowrec", rowrec, rr), ("workspace", workspace, ws)):
            if buf is None:
                continue
            if buf.numel() * buf.element_size() < need or not buf.is_contiguous():
                raise ValueError(f"{name} holds {buf.numel() * buf.element_size()} bytes; {need} needed")
            bufs.append(buf)
    for t in list(tensors) + [x for x in outputs if x is not None] + bufs:
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if t.device != dev:
            raise ValueError(f"tensors on different devices: {dev} and {t.device}")


def kia_workspace_size(p: Params):
    """(rowrec_bytes, bwd_ws_bytes) for params p."""
    a, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(_lib.kia_workspace_size(ctypes.byref(p), ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def kia_forward(p: Params, q, k, v, o, rowrec, stream=None) -> None:
    _check_inputs(p, q, k, v, outputs=(o,), rowrec=rowrec)
    _check(_lib.kia_forward(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(rowrec), _stream(stream)))


def kia_forward_scores(p: Params, q, k, v, rowrec, stream=None) -> None:
    _check_inputs(p, q, k, v, rowrec=rowrec)
    _check(_lib.kia_forward_scores(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(rowrec), _stream(stream)))


def kia_forward_weights(p: Params, q, k, v, o, rowrec, stream=None) -> None:
    _check_inputs(p, q, k, v, outputs=(o,), rowrec=rowrec)
    _check(_lib.kia_forward_weights(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(rowrec),
                                    _stream(stream)))


def kia_backward(p: Params, q, k, v, o, d_o, rowrec, dq, dk, dv, workspace, stream=None) -> None:
    _check_inputs(p, q, k, v, d_o, outputs=(o, dq, dk, dv), rowrec=rowrec, workspace=workspace)
    _check(_lib.kia_backward(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(d_o), _ptr(rowrec),
                             _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), _stream(stream)))


def kia_backward_dq(p: Params, q, k, v, o, d_o, rowrec, dq, workspace, stream=None) -> None:
    _check_inputs(p, q, k, v, d_o, outputs=(o, dq), rowrec=rowrec, workspace=workspace)
    _check(_lib.kia_backward_dq(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(d_o), _ptr(rowrec),
                                _ptr(dq), _ptr(workspace), _stream(stream)))


def kia_backward_dkdv(p: Params, q, k, v, d_o, rowrec, dk, dv, workspace, stream=None) -> None:
    _check_inputs(p, q, k, v, d_o, outputs=(dk, dv), rowrec=rowrec, workspace=workspace)
    _check(_lib.kia_backward_dkdv(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(d_o), _ptr(rowrec),
                                  _ptr(dk), _ptr(dv), _ptr(workspace), _stream(stream)))


def kia_backward_noalloc(p: Params, q, k, v, o, d_o, rowrec, dq, dk, dv, stream=None) -> None:
    """kia_backward on the library's built-in workspace (no allocation; params whose workspace
    exceeds NOALLOC_WS_BYTES raise KIA_ERR_WORKSPACE)."""
    _check_inputs(p, q, k, v, d_o, outputs=(o, dq, dk, dv), rowrec=rowrec)
    _check(_lib.kia_backward_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(d_o), _ptr(rowrec),
                                     _ptr(dq), _ptr(dk), _ptr(dv), _stream(stream)))


def _check_rowstats(p: Params, rowstats):
    need = 3 * p.B * p.H * p.T
    if rowstats.dtype != torch.float32 or rowstats.numel() < need or not rowstats.is_contiguous():
        raise ValueError(f"rowstats must be contiguous float32 with at least {need} elements")


def kia_flash_forward(p: Params, q, k, v, o, rowstats, stream=None) -> None:
    """The one-pass exact-softmax forward (p.recon must be softmax)."""
    _check_inputs(p, q, k, v, outputs=(o,))
    _check_rowstats(p, rowstats)
    if rowstats.device != q.device:
        raise ValueError("rowstats on another device")
    _check(_lib.kia_flash_forward(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(rowstats),
                                  _stream(stream)))


def kia_flash_backward(p: Params, q, k, v, o, d_o, rowstats, dq, dk, dv, stream=None) -> None:
    _check_inputs(p, q, k, v, d_o, outputs=(o, dq, dk, dv))
    _check_rowstats(p, rowstats)
    if rowstats.device != q.device:
        raise ValueError("rowstats on another device")
    _check(_lib.kia_flash_backward(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(d_o), _ptr(rowstats),
                                   _ptr(dq), _ptr(dk), _ptr(dv), _stream(stream)))


def flash_forward(cfg: Config, q, k, v, stream=None):
    """Allocate O and the row statistics with torch and run kia_flash_forward.  Returns (o, rowstats, params)."""
    p = make_params(cfg, q.shape, q.dtype)
    o = torch.empty(q.shape, device=q.device, dtype=torch.float32)
    rowstats = torch.empty(max(3 * p.B * p.H * p.T, 1), device=q.device, dtype=torch.float32)
    kia_flash_forward(p, q, k, v, o, rowstats, stream)
    return o, rowstats, p


def flash_backward(p: Params, q, k, v, o, d_o, rowstats, stream=None):
    dq = torch.empty(q.shape, device=q.device, dtype=torch.float32)
    dk = torch.empty_like(dq)
    dv = torch.empty_like(dq)
    kia_flash_backward(p, q, k, v, o, d_o, rowstats, dq, dk, dv, stream)
    return dq, dk, dv


def kia_debug_bins(p: Params, rowrec, bins, stream=None) -> None:
    rr, _ = kia_workspace_size(p)
    if rowrec.numel() * rowrec.element_size() < rr:
        raise ValueError(f"rowrec holds {rowrec.numel() * rowrec.element_size()} bytes; {rr} needed")
    if bins.dtype != torch.uint8 or bins.numel() < p.B * p.H * p.T * p.T or bins.device != rowrec.device:
        raise ValueError("bins must be uint8 [B,H,T,T] on the record's GPU")
    _check(_lib.kia_debug_bins(ctypes.byref(p), _ptr(rowrec), _ptr(bins), _stream(stream)))


# ------------------------------------------------------------------ tensor-level convenience

def forward(cfg: Config, q, k, v, stream=None):
    """Allocate O and the row record with torch and run kia_forward.  Returns (o, rowrec, params)."""
    p = make_params(cfg, q.shape, q.dtype)
    rr, _ = kia_workspace_size(p)
    o = torch.empty(q.shape, device=q.device, dtype=torch.float32)
    rowrec = torch.empty(max(rr, 1), device=q.device, dtype=torch.uint8)
    kia_forward(p, q, k, v, o, rowrec, stream)
    return o, rowrec, p


def backward(p: Params, q, k, v, o, d_o, rowrec, stream=None):
    """Allocate dQ, dK, dV and the workspace with torch and run kia_backward."""
    _, ws = kia_workspace_size(p)
    dq = torch.empty(q.shape, device=q.device, dtype=torch.float32)
    dk = torch.empty_like(dq)
    dv = torch.empty_like(dq)
    work = torch.empty(max(ws, 1), device=q.device, dtype=torch.uint8)
    kia_backward(p, q, k, v, o, d_o, rowrec, dq, dk, dv, work, stream)
    return dq, dk, dv


def debug_bins(p: Params, rowrec, stream=None):
    bins = torch.empty((p.B, p.H, p.T, p.T), device=rowrec.device, dtype=torch.uint8)
    kia_debug_bins(p, rowrec, bins, stream)
    return bins


class KIAttention(torch.autograd.Function):
    """Autograd wrapper: forward and backward both run in libkia."""

    @staticmethod
    def forward(ctx, q, k, v, cfg: Config):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        o, rowrec, p = forward(cfg, q, k, v)
        ctx.save_for_backward(q, k, v, o, rowrec)
        ctx.p = p
        return o

    @staticmethod
    def backward(ctx, grad_o):
        q, k, v, o, rowrec = ctx.saved_tensors
        d_o = grad_o.to(q.dtype).contiguous()
        dq, dk, dv = backward(ctx.p, q, k, v, o, d_o, rowrec)
        return dq.to(q.dtype), dk.to(k.dtype), dv.to(v.dtype), None


def kia_attention(q, k, v, cfg: Config = Config()):
    """K-interval attention on [B, H, T, D] tensors (float32 or bfloat16); returns float32 O."""
    return KIAttention.apply(q, k, v, cfg)
