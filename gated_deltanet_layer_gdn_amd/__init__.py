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
from ._lib import BF16, F16, F32, GdnError

__all__ = [
    "Dims", "GdnError", "conv1d", "prefill_chunked", "decode_step", "decode_step_noalloc",
    "decode_multi", "prefill_varlen", "prefill_varlen_workspace_bytes", "gated_rmsnorm", "in_proj",
    "AttnDims", "attn_prefill", "attn_workspace_bytes",
    "state_save",
    "state_restore", "state_check", "prefill_workspace_bytes", "decode_workspace_bytes",
    "rec_state_bytes", "conv_state_bytes", "state_blob_bytes", "F32", "BF16", "F16",
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


@dataclass(frozen=True)
class AttnDims:
    """Full-attention geometry (mirrors ``gdn_attn_dims``)."""
    B: int
    H_q: int = 24
    H_kv: int = 2
    d_h: int = 256
    rot_dim: int = 64
    out_dtype: int = BF16
    rope_base: float = 1e7
    scale: float | None = None

    def c(self) -> _lib.GdnAttnDims:
        sc = self.d_h ** -0.5 if self.scale is None else self.scale
        return _lib.GdnAttnDims(_lib.ABI_VERSION, self.B, self.H_q, self.H_kv, self.d_h,
                                self.rot_dim, BF16, self.out_dtype, self.rope_base, sc)


def _torch():
    import torch
    return torch


def _dt(code: int):
    torch = _torch()
    return {F32: torch.float32, BF16: torch.bfloat16, F16: torch.float16}[code]


def _stream():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need_opt(t, name, shape, dtype):
    """_need for an optional tensor (None passes a null pointer)."""
    return ctypes.c_void_p(None) if t is None else _need(t, name, shape, dtype)


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
    """A new workspace when ``ws`` is None, else ``ws`` after a size check."""
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
        _need_opt(z, "z", (d.B, T, d.H_v, d.d_v), dt),
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
    zshape = tuple(z.shape) if z is not None else (
        (d.B, d.H_v, d.d_v) if x.dim() == 2 else (d.B, 1, d.H_v, d.d_v))
    args = [
        _need(x.reshape(d.B, d.C_ch), "x", (d.B, d.C_ch), dt),
        _need_opt(None if z is None else z.reshape(d.B, d.H_v, d.d_v), "z", (d.B, d.H_v, d.d_v),
                  dt),
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


def decode_multi(d: Dims, x, z, g, beta, conv_w, conv_pool, rec_pool, in_slots, out_slots=None,
                 y=None, ws=None):
    """T (1..4) tokens per sequence from slot-indexed states: x [B,T,C_ch],
    z [B,T,H_v,d_v], g/beta [B,T,H_v]; conv_pool [n_slots,W-1,C_ch], rec_pool
    [n_slots,H_v,d_v,d_k]; in_slots int32 [B] and out_slots int32 [B,T] (or
    None) on the device.  Returns y [B,T,H_v,d_v]."""
    torch = _torch()
    L = _lib.load()
    T = x.shape[1]
    n_slots = rec_pool.shape[0]
    dt = _dt(d.in_dtype)
    args = [
        _need(x, "x", (d.B, T, d.C_ch), dt),
        _need_opt(z, "z", (d.B, T, d.H_v, d.d_v), dt),
        _need(g, "g", (d.B, T, d.H_v), torch.float32),
        _need(beta, "beta", (d.B, T, d.H_v), torch.float32),
        _need(conv_w, "conv_w", (d.C_ch, d.W), dt),
        _need(conv_pool, "conv_pool", (n_slots, d.W - 1, d.C_ch), dt),
        _need(rec_pool, "rec_pool", (n_slots, d.H_v, d.d_v, d.d_k), torch.float32),
    ]
    pin = _need(in_slots, "in_slots", (d.B,), torch.int32)
    pout = (ctypes.c_void_p(None) if out_slots is None
            else _need(out_slots, "out_slots", (d.B, T), torch.int32))
    if y is None:
        y = torch.empty((d.B, T, d.H_v, d.d_v), dtype=_dt(d.out_dtype), device=x.device)
    py = _need(y, "y", (d.B, T, d.H_v, d.d_v), _dt(d.out_dtype))
    need = T * L.gdn_decode_workspace_bytes(ctypes.byref(d.c()))
    ws = _workspace(need, x, ws)
    rc = L.gdn_decode_multi(ctypes.byref(d.c()), T, *args[:5], args[5], args[6], n_slots, pin,
                            pout, py, ctypes.c_void_p(ws.data_ptr()),
                            ws.numel() * ws.element_size(), _stream())
    _lib.check(rc, "gdn_decode_multi")
    return y


def _cu_array(cu_seqlens):
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    return cu, cu.ctypes.data_as(ctypes.c_void_p)


def prefill_varlen_workspace_bytes(d: Dims, cu_seqlens, chunk: int) -> int:
    cu, pcu = _cu_array(cu_seqlens)
    return _lib.load().gdn_prefill_varlen_workspace_bytes(ctypes.byref(d.c()), pcu, chunk)


def prefill_varlen(d: Dims, cu_seqlens, x, z, g, beta, conv_w, conv_pool, rec_pool, slots,
                   chunk: int = 64, y=None, ws=None):
    """Packed variable-length prefill of d.B sequences: cu_seqlens (host,
    B+1 offsets), x [T_total,C_ch], z [T_total,H_v,d_v], g/beta [T_total,H_v];
    slots (host, B) index conv_pool / rec_pool.  Returns y [T_total,H_v,d_v]."""
    torch = _torch()
    L = _lib.load()
    cu, pcu = _cu_array(cu_seqlens)
    sl = np.ascontiguousarray(np.asarray(slots, dtype=np.int32))
    T_total = x.shape[0]
    n_slots = rec_pool.shape[0]
    dt = _dt(d.in_dtype)
    args = [
        _need(x, "x", (T_total, d.C_ch), dt),
        _need_opt(z, "z", (T_total, d.H_v, d.d_v), dt),
        _need(g, "g", (T_total, d.H_v), torch.float32),
        _need(beta, "beta", (T_total, d.H_v), torch.float32),
        _need(conv_w, "conv_w", (d.C_ch, d.W), dt),
        _need(conv_pool, "conv_pool", (n_slots, d.W - 1, d.C_ch), dt),
        _need(rec_pool, "rec_pool", (n_slots, d.H_v, d.d_v, d.d_k), torch.float32),
    ]
    if y is None:
        y = torch.empty((T_total, d.H_v, d.d_v), dtype=_dt(d.out_dtype), device=x.device)
    py = _need(y, "y", (T_total, d.H_v, d.d_v), _dt(d.out_dtype))
    need = L.gdn_prefill_varlen_workspace_bytes(ctypes.byref(d.c()), pcu, chunk)
    if need == 0:
        raise GdnError(-1, "gdn_prefill_varlen", "invalid sequence table or chunk")
    ws = _workspace(need, x, ws)
    rc = L.gdn_prefill_varlen(ctypes.byref(d.c()), pcu, chunk, *args, n_slots,
                              sl.ctypes.data_as(ctypes.c_void_p), py,
                              ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(),
                              _stream())
    _lib.check(rc, "gdn_prefill_varlen")
    return y


def attn_workspace_bytes(a: AttnDims, T: int, pos0: int = 0) -> int:
    return _lib.load().gdn_attn_workspace_bytes(ctypes.byref(a.c()), T, pos0)


def attn_prefill(a: AttnDims, q, k, v, k_cache, v_cache, pos0: int = 0, o=None, ws=None):
    """Attention over T new tokens at positions pos0..pos0+T-1: q [B,T,H_q,d_h],
    k/v [B,T,H_kv,d_h] bf16; k_cache/v_cache [B,T_max,H_kv,d_h] bf16 (updated);
    returns o [B,T,H_q,d_h] in a.out_dtype."""
    torch = _torch()
    L = _lib.load()
    T = q.shape[1]
    T_max = k_cache.shape[1]
    args = [_need(q, "q", (a.B, T, a.H_q, a.d_h), torch.bfloat16),
            _need(k, "k", (a.B, T, a.H_kv, a.d_h), torch.bfloat16),
            _need(v, "v", (a.B, T, a.H_kv, a.d_h), torch.bfloat16),
            _need(k_cache, "k_cache", (a.B, T_max, a.H_kv, a.d_h), torch.bfloat16),
            _need(v_cache, "v_cache", (a.B, T_max, a.H_kv, a.d_h), torch.bfloat16)]
    if o is None:
        o = torch.empty((a.B, T, a.H_q, a.d_h), dtype=_dt(a.out_dtype), device=q.device)
    po = _need(o, "o", (a.B, T, a.H_q, a.d_h), _dt(a.out_dtype))
    need = L.gdn_attn_workspace_bytes(ctypes.byref(a.c()), T, pos0)
    if need == 0:
        raise GdnError(-1, "gdn_attn_prefill", "invalid geometry or positions")
    ws = _workspace(need, q, ws)
    rc = L.gdn_attn_prefill(ctypes.byref(a.c()), T, pos0, *args, T_max, po,
                            ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(),
                            _stream())
    _lib.check(rc, "gdn_attn_prefill")
    return o


def in_proj(d: Dims, h, w_in, A_log, dt_bias, x=None, z=None, g=None, beta=None):
    """Input projections: h [B,T,hidden] bf16, w_in [C_ch + H_v*d_v + 2*H_v,
    hidden] bf16, A_log/dt_bias fp32 [H_v].  Returns (x [B,T,C_ch] bf16,
    z [B,T,H_v,d_v] bf16, g [B,T,H_v] fp32, beta [B,T,H_v] fp32)."""
    torch = _torch()
    L = _lib.load()
    B, T, hidden = h.shape
    N = d.C_ch + d.H_v * d.d_v + 2 * d.H_v
    dev = h.device
    x = torch.empty((d.B, T, d.C_ch), dtype=torch.bfloat16, device=dev) if x is None else x
    z = torch.empty((d.B, T, d.H_v, d.d_v), dtype=torch.bfloat16, device=dev) if z is None else z
    g = torch.empty((d.B, T, d.H_v), dtype=torch.float32, device=dev) if g is None else g
    beta = torch.empty((d.B, T, d.H_v), dtype=torch.float32, device=dev) if beta is None else beta
    args = [_need(h, "h", (d.B, T, hidden), torch.bfloat16),
            _need(w_in, "w_in", (N, hidden), torch.bfloat16),
            _need(A_log, "A_log", (d.H_v,), torch.float32),
            _need(dt_bias, "dt_bias", (d.H_v,), torch.float32),
            _need(x, "x", (d.B, T, d.C_ch), torch.bfloat16),
            _need(z, "z", (d.B, T, d.H_v, d.d_v), torch.bfloat16),
            _need(g, "g", (d.B, T, d.H_v), torch.float32),
            _need(beta, "beta", (d.B, T, d.H_v), torch.float32)]
    _lib.check(L.gdn_in_proj(ctypes.byref(d.c()), T, hidden, *args, _stream()), "gdn_in_proj")
    return x, z, g, beta


def gated_rmsnorm(d: Dims, o, z, norm_w=None, norm_eps: float = 1e-6, y=None):
    """Zero-centred grouped RMS norm + sigmoid gate over the ungated readout
    o (fp32, [..., H_v, d_v], from a layer call with z=None); z like o in the
    input dtype, or None (no gate); norm_w fp32 [d_v] or None.  Returns y in
    d.out_dtype, shaped like o."""
    torch = _torch()
    L = _lib.load()
    if tuple(o.shape[-2:]) != (d.H_v, d.d_v):
        raise ValueError(f"o: trailing shape {tuple(o.shape[-2:])} != {(d.H_v, d.d_v)}")
    rows = o.numel() // (d.H_v * d.d_v)
    shape = tuple(o.shape)
    po = _need(o, "o", shape, torch.float32)
    pz = _need_opt(z, "z", shape, _dt(d.in_dtype))
    pw = _need_opt(norm_w, "norm_w", (d.d_v,), torch.float32)
    if y is None:
        y = torch.empty(shape, dtype=_dt(d.out_dtype), device=o.device)
    py = _need(y, "y", shape, _dt(d.out_dtype))
    _lib.check(L.gdn_gated_rmsnorm(ctypes.byref(d.c()), rows, po, pz, pw, norm_eps, py, _stream()),
               "gdn_gated_rmsnorm")
    return y


def decode_step_noalloc(d: Dims, x, z, g, beta, conv_w, conv_state, rec_state, y):
    """decode_step through the entry point that allocates nothing: the caller
    passes every buffer including y (shaped like z), and the library uses its
    fixed per-GPU scratch as the workspace."""
    torch = _torch()
    L = _lib.load()
    dt = _dt(d.in_dtype)
    args = [
        _need(x.reshape(d.B, d.C_ch), "x", (d.B, d.C_ch), dt),
        _need(z.reshape(d.B, d.H_v, d.d_v), "z", (d.B, d.H_v, d.d_v), dt),
        _need(g.reshape(d.B, d.H_v), "g", (d.B, d.H_v), torch.float32),
        _need(beta.reshape(d.B, d.H_v), "beta", (d.B, d.H_v), torch.float32),
        _need(conv_w, "conv_w", (d.C_ch, d.W), dt),
        _need(conv_state, "conv_state", (d.B, d.W - 1, d.C_ch), dt),
        _need(rec_state, "rec_state", (d.B, d.H_v, d.d_v, d.d_k), torch.float32),
        _need(y.reshape(d.B, d.H_v, d.d_v), "y", (d.B, d.H_v, d.d_v), _dt(d.out_dtype)),
    ]
    _lib.check(L.gdn_decode_step_noalloc(ctypes.byref(d.c()), *args, _stream()),
               "gdn_decode_step_noalloc")
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
