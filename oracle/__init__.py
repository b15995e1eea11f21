"""fp64 CPU oracle for the Gated DeltaNet layer (ctypes wrapper over liboracle.so).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does.  It
shares no code with the HIP implementation.

The arithmetic lives in ``gdn_oracle.c`` (plain C, double precision, one token
at a time); this module only marshals numpy arrays.  Array conventions:

* ``x``  [B, T, C_ch] with C_ch = 2*H_k*d_k + H_v*d_v, channels ordered
  [q | k | v], head-major;  ``z`` [B, T, H_v, d_v];  ``w`` [C_ch, W];
  ``hist`` (conv history) [B, W-1, C_ch], oldest row first.  These are either
  float32 arrays or bf16 bit patterns held in uint16 arrays.
* ``g`` (log decay, a = exp(g)) and ``beta`` are float32 [B, T, H_v].
* ``S`` (recurrent state) is [B, H_v, d_v, d_k]; the oracle works on a float64
  copy and returns float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")
_LIB = None

F32, BF16 = 0, 1


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (IEEE double, no contraction)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
            "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lpthread", "-lm",
        ])
        os.replace(tmp, _SO)
    return _SO


def _lib():
    global _LIB
    if _LIB is None:
        build()
        L = ctypes.CDLL(_SO)
        i64, i32, vp, dp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_double
        L.oracle_conv_silu.argtypes = [i32, i64, i32, i32, i32, vp, vp, vp, vp]
        L.oracle_conv_history_next.argtypes = [i32, i64, i32, i32, i32, vp, vp, vp]
        L.oracle_l2norm.argtypes = [i64, i32, vp, dp, dp, vp]
        L.oracle_recurrence.argtypes = [i32, i64, i32, i32, i32, i32] + [vp] * 9
        L.oracle_layer.argtypes = ([i32, i64, i32, i32, i32, i32, i32, i32, dp, dp]
                                   + [vp] * 8 + [vp, i32, i32])
        for f in (L.oracle_conv_silu, L.oracle_conv_history_next, L.oracle_l2norm,
                  L.oracle_recurrence, L.oracle_layer):
            f.restype = i32
        _LIB = L
    return _LIB


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _dtype_code(a) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle inputs must be float32 or bf16 bits (uint16), got {a.dtype}")


def _c(a, dt=None):
    a = np.asarray(a) if dt is None else np.asarray(a, dtype=dt)
    return np.ascontiguousarray(a)


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def conv_silu(x, w, hist):
    """Stage a1: causal width-W conv + SiLU of every channel -> float64 [B,T,C_ch]."""
    x, w, hist = _c(x), _c(w), _c(hist)
    dt = _dtype_code(x)
    assert _dtype_code(w) == dt and _dtype_code(hist) == dt
    B, T, C = x.shape
    W = w.shape[1]
    assert w.shape == (C, W) and hist.shape == (B, W - 1, C)
    out = np.empty((B, T, C), np.float64)
    rc = _lib().oracle_conv_silu(B, T, C, W, dt, _ptr(x), _ptr(w), _ptr(hist), _ptr(out))
    assert rc == 0, rc
    return out


def conv_history_next(x, hist):
    """Conv history after the call: last W-1 rows of concat(hist, x), bit for bit."""
    x, hist = _c(x), _c(hist)
    dt = _dtype_code(x)
    B, T, C = x.shape
    W = hist.shape[1] + 1
    out = np.empty_like(hist)
    rc = _lib().oracle_conv_history_next(B, T, C, W, dt, _ptr(x), _ptr(hist), _ptr(out))
    assert rc == 0, rc
    return out


def l2norm(a, eps: float, scale: float = 1.0):
    """Stage a2 over the last axis: a / sqrt(sum a^2 + eps) * scale (float64)."""
    a = _c(a, np.float64)
    d = a.shape[-1]
    out = np.empty_like(a)
    rc = _lib().oracle_l2norm(a.size // d, d, _ptr(a), eps, scale, _ptr(out))
    assert rc == 0, rc
    return out


def recurrence(q, k, v, g, beta, z, S0):
    """Sequential gated delta rule on convolved inputs (all float64).

    q, k [B,T,H_k,d_k]; v, z [B,T,H_v,d_v]; g, beta [B,T,H_v]; S0 [B,H_v,d_v,d_k].
    Returns (y, S_final, o) with o the ungated readout.
    """
    q, k, v, g, beta, z = (_c(a, np.float64) for a in (q, k, v, g, beta, z))
    S = _c(S0, np.float64).copy()
    B, T, H_k, d_k = q.shape
    H_v, d_v = v.shape[2], v.shape[3]
    y = np.empty((B, T, H_v, d_v), np.float64)
    o = np.empty_like(y)
    rc = _lib().oracle_recurrence(B, T, H_k, H_v, d_k, d_v, _ptr(q), _ptr(k), _ptr(v),
                                  _ptr(g), _ptr(beta), _ptr(z), _ptr(S), _ptr(y), _ptr(o))
    assert rc == 0, rc
    return y, S, o


def layer(x, z, g, beta, w, hist, S0, *, H_k: int, H_v: int, d_k: int, d_v: int,
          eps: float, q_scale: float = 1.0, heads=None, nthreads: int | None = None):
    """Whole GDN layer from raw inputs.

    Returns (y float64 [B,T,H_v,d_v], S float64 [B,H_v,d_v,d_k], hist_next).
    ``heads``: optional iterable of (b, h) pairs; only those are computed (other
    entries of y are NaN and other state heads keep S0).
    """
    x, z, w, hist = _c(x), _c(z), _c(w), _c(hist)
    g, beta = _c(g, np.float32), _c(beta, np.float32)
    dt = _dtype_code(x)
    for a in (z, w, hist):
        assert _dtype_code(a) == dt
    B, T, C = x.shape
    W = w.shape[1]
    assert C == 2 * H_k * d_k + H_v * d_v, (C, H_k, d_k, H_v, d_v)
    assert z.shape == (B, T, H_v, d_v) and g.shape == (B, T, H_v) == beta.shape
    assert hist.shape == (B, W - 1, C)
    S = _c(S0, np.float64).copy()
    assert S.shape == (B, H_v, d_v, d_k)
    y = np.full((B, T, H_v, d_v), np.nan)
    tasks = None
    n = 0
    if heads is not None:
        tasks = np.ascontiguousarray(np.asarray(list(heads), np.int32).reshape(-1, 2))
        n = tasks.shape[0]
    nth = nthreads or default_threads()
    rc = _lib().oracle_layer(B, T, H_k, H_v, d_k, d_v, W, dt, eps, q_scale, _ptr(x), _ptr(z),
                             _ptr(g), _ptr(beta), _ptr(w), _ptr(hist), _ptr(S), _ptr(y),
                             _ptr(tasks), n, nth)
    assert rc == 0, rc
    return y, S, conv_history_next(x, hist)
