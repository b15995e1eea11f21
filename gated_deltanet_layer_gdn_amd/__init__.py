"""Gated DeltaNet (GDN) token-mixing layer for AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``libgdn.so`` (declared in
``include/gdn.h``): every function here only checks tensor shapes, dtypes and
devices and passes raw pointers and the current HIP stream.  Every step of
the layer runs in the library's HIP kernels.  PyTorch provides device memory
and streams.

Entry points (same names as the C ABI without the ``gdn_`` prefix):
``conv1d``, ``prefill_chunked``, ``decode_step``, ``state_save``,
``state_restore``, plus the size queries.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import numpy as np

from . import _lib
from ._lib import BF16, F32, GdnError

__all__ = [
    "Dims", "GdnError", "conv1d", "prefill_chunked", "decode_step", "state_save",
    "state_restore", "state_check", "prefill_workspace_bytes", "decode_workspace_bytes",
    "rec_state_bytes", "conv_state_bytes", "state_blob_bytes", "F32", "BF16",
]


@dataclass(frozen=True)
class Dims:
    """Layer geometry (mirrors ``gdn_dims``)."""
    B: int
    H_k: int
    H_v: int
    d_k: int
    d_v: int
    W: int = 4
    in_dtype: int = BF16
    out_dtype: int = F32
    l2_eps: float = 1e-6
    q_scale: float = 1.0

    @property
    def C_ch(self) -> int:
        return 2 * self.H_k * self.d_k + self.H_v * self.d_v

    def c(self) -> _lib.GdnDims:
        return _lib.GdnDims(_lib.ABI_VERSION, self.B, self.H_k, self.H_v, self.d_k, self.d_v,
                            self.W, self.in_dtype, self.out_dtype, self.l2_eps, self.q_scale)


def _torch():
    import torch
    return torch


def _dt(code: int):
    torch = _torch()
    return torch.float32 if code == F32 else torch.bfloat16


def _stream():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, name, shape, dtype):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype} != {dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def rec_state_bytes(d: Dims) -> int:
    return _lib.load().gdn_rec_state_bytes(ctypes.byref(d.c()))


def conv_state_bytes(d: Dims) -> int:
    return _lib.load().gdn_conv_state_bytes(ctypes.byref(d.c()))


def state_blob_bytes(d: Dims) -> int:
    return _lib.load().gdn_state_blob_bytes(ctypes.byref(d.c()))


def prefill_workspace_bytes(d: Dims, T: int, chunk: int) -> int:
    return _lib.load().gdn_prefill_workspace_bytes(ctypes.byref(d.c()), T, chunk)


def decode_workspace_bytes(d: Dims) -> int:
    return _lib.load().gdn_decode_workspace_bytes(ctypes.byref(d.c()))


def _workspace(nbytes: int, ref, ws):
    torch = _torch()
    if ws is None:
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=ref.device)
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError("workspace too small")
    return ws


def conv1d(d: Dims, x, conv_w, conv_state, out=None):
    """Conv1D + SiLU + L2 norm (steps 1-2) over x [B,T,C_ch]; returns fp32
    [B,T,C_ch] and updates conv_state in place."""
    torch = _torch()
    L = _lib.load()
    B, T = x.shape[0], x.shape[1]
    dt = _dt(d.in_dtype)
    px = _need(x, "x", (d.B, T, d.C_ch), dt)
    pw = _need(conv_w, "conv_w", (d.C_ch, d.W), dt)
    ph = _need(conv_state, "conv_state", (d.B, d.W - 1, d.C_ch), dt)
    if out is None:
        out = torch.empty((B, T, d.C_ch), dtype=torch.float32, device=x.device)
    po = _need(out, "out", (d.B, T, d.C_ch), torch.float32)
    _lib.check(L.gdn_conv1d(ctypes.byref(d.c()), T, px, pw, ph, po, _stream()), "gdn_conv1d")
    return out


def prefill_chunked(d: Dims, x, z, g, beta, conv_w, conv_state, rec_state, chunk: int = 64,
                    y=None, ws=None, kernel_ms=None):
    """Whole layer over T tokens; updates conv_state and rec_state in place and
    returns y [B,T,H_v,d_v].  With ``kernel_ms`` (a list), calls the timed
    entry point and appends the 3 per-kernel durations in ms (conv, prep with the history
    roll, state)."""
    torch = _torch()
    L = _lib.load()
    T = x.shape[1]
    dt = _dt(d.in_dtype)
    args = [
        _need(x, "x", (d.B, T, d.C_ch), dt),
        _need(z, "z", (d.B, T, d.H_v, d.d_v), dt),
        _need(g, "g", (d.B, T, d.H_v), torch.float32),
        _need(beta, "beta", (d.B, T, d.H_v), torch.float32),
        _need(conv_w, "conv_w", (d.C_ch, d.W), dt),
        _need(conv_state, "conv_state", (d.B, d.W - 1, d.C_ch), dt),
        _need(rec_state, "rec_state", (d.B, d.H_v, d.d_v, d.d_k), torch.float32),
    ]
    if y is None:
        y = torch.empty((d.B, T, d.H_v, d.d_v), dtype=_dt(d.out_dtype), device=x.device)
    args.append(_need(y, "y", (d.B, T, d.H_v, d.d_v), _dt(d.out_dtype)))
    need = L.gdn_prefill_workspace_bytes(ctypes.byref(d.c()), T, chunk)
    if need == 0:
        raise GdnError(-2, "gdn_prefill_chunked", f"no workspace size for T={T} chunk={chunk}")
    ws = _workspace(need, x, ws)
    tail = [ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(), _stream()]
    if kernel_ms is None:
        rc = L.gdn_prefill_chunked(ctypes.byref(d.c()), T, chunk, *args, *tail)
    else:
        ms = (ctypes.c_float * 3)()
        rc = L.gdn_prefill_chunked_timed(ctypes.byref(d.c()), T, chunk, *args, *tail, ms)
        kernel_ms.extend(float(v) for v in ms)
    _lib.check(rc, "gdn_prefill_chunked")
    return y


def decode_step(d: Dims, x, z, g, beta, conv_w, conv_state, rec_state, y=None, ws=None,
                kernel_ms=None):
    """One token per sequence: x [B,1,C_ch] (or [B,C_ch]), z [B,1,H_v,d_v] (or
    [B,H_v,d_v]), g/beta [B,1,H_v] (or [B,H_v]); returns y shaped like z.
    With ``kernel_ms`` (a list), appends the 2 per-kernel durations in ms."""
    torch = _torch()
    L = _lib.load()
    dt = _dt(d.in_dtype)
    zshape = tuple(z.shape)
    args = [
        _need(x.reshape(d.B, d.C_ch), "x", (d.B, d.C_ch), dt),
        _need(z.reshape(d.B, d.H_v, d.d_v), "z", (d.B, d.H_v, d.d_v), dt),
        _need(g.reshape(d.B, d.H_v), "g", (d.B, d.H_v), torch.float32),
        _need(beta.reshape(d.B, d.H_v), "beta", (d.B, d.H_v), torch.float32),
        _need(conv_w, "conv_w", (d.C_ch, d.W), dt),
        _need(conv_state, "conv_state", (d.B, d.W - 1, d.C_ch), dt),
        _need(rec_state, "rec_state", (d.B, d.H_v, d.d_v, d.d_k), torch.float32),
    ]
    if y is None:
        y = torch.empty(zshape, dtype=_dt(d.out_dtype), device=x.device)
    args.append(_need(y.reshape(d.B, d.H_v, d.d_v), "y", (d.B, d.H_v, d.d_v), _dt(d.out_dtype)))
    need = L.gdn_decode_workspace_bytes(ctypes.byref(d.c()))
    ws = _workspace(need, x, ws)
    tail = [ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(), _stream()]
    if kernel_ms is None:
        rc = L.gdn_decode_step(ctypes.byref(d.c()), *args, *tail)
    else:
        ms = (ctypes.c_float * 2)()
        rc = L.gdn_decode_step_timed(ctypes.byref(d.c()), *args, *tail, ms)
        kernel_ms.extend(float(v) for v in ms)
    _lib.check(rc, "gdn_decode_step")
    return y


def state_save(d: Dims, conv_state, rec_state) -> np.ndarray:
    """Checkpoint blob (uint8 numpy array) of the conv and recurrent state."""
    torch = _torch()
    L = _lib.load()
    pc = _need(conv_state, "conv_state", (d.B, d.W - 1, d.C_ch), _dt(d.in_dtype))
    pr = _need(rec_state, "rec_state", (d.B, d.H_v, d.d_v, d.d_k), torch.float32)
    n = L.gdn_state_blob_bytes(ctypes.byref(d.c()))
    blob = np.empty(n, np.uint8)
    rc = L.gdn_state_save(ctypes.byref(d.c()), pc, pr, blob.ctypes.data_as(ctypes.c_void_p), n,
                          _stream())
    _lib.check(rc, "gdn_state_save")
    return blob


def state_restore(d: Dims, blob, conv_state, rec_state) -> None:
    """Validate ``blob`` and copy it into conv_state and rec_state."""
    torch = _torch()
    L = _lib.load()
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    pc = _need(conv_state, "conv_state", (d.B, d.W - 1, d.C_ch), _dt(d.in_dtype))
    pr = _need(rec_state, "rec_state", (d.B, d.H_v, d.d_v, d.d_k), torch.float32)
    rc = L.gdn_state_restore(ctypes.byref(d.c()), blob.ctypes.data_as(ctypes.c_void_p),
                             blob.size, pc, pr, _stream())
    _lib.check(rc, "gdn_state_restore")


def state_check(d: Dims, blob) -> int:
    """Host-only blob validation; returns the status code."""
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    return _lib.load().gdn_state_check(ctypes.byref(d.c()), blob.ctypes.data_as(ctypes.c_void_p),
                                       blob.size)
