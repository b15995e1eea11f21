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
        L.oracle_gated_rmsnorm.argtypes = [i64, i32, vp, vp, vp, dp, vp]
        for f in (L.oracle_conv_silu, L.oracle_conv_history_next, L.oracle_l2norm,
                  L.oracle_recurrence, L.oracle_layer, L.oracle_gated_rmsnorm):
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
    ``z=None`` gives the ungated readout y = o = S_t q_t.
    ``heads``: optional iterable of (b, h) pairs; only those are computed (other
    entries of y are NaN and other state heads keep S0).
    """
    x, w, hist = _c(x), _c(w), _c(hist)
    z = None if z is None else _c(z)
    g, beta = _c(g, np.float32), _c(beta, np.float32)
    dt = _dtype_code(x)
    for a in (w, hist) if z is None else (z, w, hist):
        assert _dtype_code(a) == dt
    B, T, C = x.shape
    W = w.shape[1]
    assert C == 2 * H_k * d_k + H_v * d_v, (C, H_k, d_k, H_v, d_v)
    assert z is None or z.shape == (B, T, H_v, d_v)
    assert g.shape == (B, T, H_v) == beta.shape
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


def gated_rmsnorm(o, z, w, eps: float):
    """Zero-centred grouped RMS norm over the last axis, then the sigmoid gate:
    o / sqrt(mean(o^2) + eps) * (1 + w) * sigmoid(z) (float64).  z may be None
    (no gate), w may be None (all zero)."""
    o = _c(o, np.float64)
    d = o.shape[-1]
    zz = None if z is None else _c(z, np.float64)
    ww = None if w is None else _c(w, np.float64)
    assert zz is None or zz.shape == o.shape
    assert ww is None or ww.shape == (d,)
    y = np.empty_like(o)
    rc = _lib().oracle_gated_rmsnorm(o.size // d, d, _ptr(o), _ptr(zz), _ptr(ww), eps, _ptr(y))
    assert rc == 0, rc
    return y


# ---------------------------------------------------------------------------
# Serving-shaped calls, composed from `layer` (each sequence is one plain
# layer call on its own tokens and its own state; nothing else is computed).
# Sources: "Add Qwen3.8 MTP and multimodal inference on Metal without
# regressing text", section Correctness gates (MTP candidate generation,
# verification, cache updates, rollback); the model card "Qwen3.8-27B FP8 +
# native MTP + multimodal Core AI", section What is fused (a three-token
# target prefill); "Implement the Qwen3.8 Flash Next Rust and Metal text
# core", section Implementation (prefill/small-batch infrastructure) and its
# implementation comment (resident-state swaps).

def layer_varlen(x, z, g, beta, w, hist_pool, S_pool, cu_seqlens, slots, *, H_k: int, H_v: int,
                 d_k: int, d_v: int, eps: float, q_scale: float = 1.0, nthreads=None):
    """Packed variable-length prefill.

    x [T_total, C_ch], z [T_total, H_v, d_v], g/beta [T_total, H_v]: the
    sequences' tokens back to back; sequence n owns rows cu_seqlens[n] ..
    cu_seqlens[n+1]-1 and the states in slot slots[n] of hist_pool
    [n_slots, W-1, C_ch] and S_pool [n_slots, H_v, d_v, d_k].
    Returns (y float64 [T_total, H_v, d_v], S_pool float64, hist_pool): the
    slots of the sequences hold their states after their tokens, every other
    slot is returned unchanged (a sequence of length 0 leaves its slot as is).
    """
    cu = [int(c) for c in cu_seqlens]
    T_total = x.shape[0]
    assert cu[0] == 0 and cu[-1] == T_total and len(slots) == len(cu) - 1
    y = np.full((T_total, H_v, d_v), np.nan)
    S_out = np.array(S_pool, np.float64, copy=True)
    h_out = np.array(hist_pool, copy=True)
    for n, s in enumerate(slots):
        a, b = cu[n], cu[n + 1]
        if b == a:
            continue
        yn, Sn, hn = layer(x[None, a:b], z[None, a:b], g[None, a:b], beta[None, a:b], w,
                           hist_pool[None, s], S_pool[None, s], H_k=H_k, H_v=H_v, d_k=d_k,
                           d_v=d_v, eps=eps, q_scale=q_scale, nthreads=nthreads)
        y[a:b] = yn[0]
        S_out[s] = Sn[0]
        h_out[s] = hn[0]
    return y, S_out, h_out


def decode_multi(x, z, g, beta, w, hist_pool, S_pool, in_slots, out_slots, *, H_k: int,
                 H_v: int, d_k: int, d_v: int, eps: float, q_scale: float = 1.0):
    """T tokens per sequence from slot-indexed states, with the state after
    every token stored to a slot of its own (MTP verify and rollback keep
    the per-token states and pick one).

    x [B, T, C_ch], z [B, T, H_v, d_v], g/beta [B, T, H_v]; in_slots [B]:
    the slot each sequence starts from; out_slots [B, T]: the slot that
    receives the state after token t (or None: the in slot after the last
    token, nothing for earlier tokens).  A sequence whose in slot lies outside
    [0, n_slots) is a padding row (y zero, nothing stored); an out slot
    outside that range is not stored.  The state after token t is the plain
    layer over tokens 0..t from the in slot's state.
    Returns (y float64 [B, T, H_v, d_v], S_pool float64, hist_pool).
    """
    B, T = x.shape[0], x.shape[1]
    n_slots = S_pool.shape[0]
    y = np.zeros((B, T, H_v, d_v))
    S_out = np.array(S_pool, np.float64, copy=True)
    h_out = np.array(hist_pool, copy=True)
    for b in range(B):
        s = int(in_slots[b])
        if not 0 <= s < n_slots:
            continue
        for t in range(T):
            o = (s if t == T - 1 else -1) if out_slots is None else int(out_slots[b][t])
            yt, St, ht = layer(x[b:b + 1, :t + 1], z[b:b + 1, :t + 1], g[b:b + 1, :t + 1],
                               beta[b:b + 1, :t + 1], w, hist_pool[None, s], S_pool[None, s],
                               H_k=H_k, H_v=H_v, d_k=d_k, d_v=d_v, eps=eps, q_scale=q_scale)
            y[b, t] = yt[0, t]
            if 0 <= o < n_slots:
                S_out[o] = St[0]
                h_out[o] = ht[0]
    return y, S_out, h_out


# ---------------------------------------------------------------------------
# Input projections ("Implement the Qwen3.8 Flash Next Rust and Metal text
# core", section Verification: primitive vectors for the GDN projection).
# The pages give no formula; the reading: one fused weight whose rows are the
# C_ch conv inputs x, the H_v d_v gate inputs z, H_v rows b and H_v rows a;
# beta = sigmoid(b) and the log decay g = -exp(A_log) softplus(a + dt_bias)
# (Gated DeltaNet's Mamba2-style gate), per value head.

def _widen(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def decay_beta(a, b, A_log, dt_bias):
    """beta = sigmoid(b), g = -exp(A_log) * softplus(a + dt_bias), float64;
    a, b [..., H_v]; A_log, dt_bias [H_v]."""
    a, b = _widen(a), _widen(b)
    A_log, dt_bias = np.asarray(A_log, np.float64), np.asarray(dt_bias, np.float64)
    beta = 1.0 / (1.0 + np.exp(-b))
    g = -np.exp(A_log) * np.logaddexp(0.0, a + dt_bias)
    return g, beta


def in_proj(h, w_in, A_log, dt_bias, *, C_ch: int, Z: int, H_v: int):
    """h [..., hidden] (bf16 bits or float32), w_in [C_ch + Z + 2 H_v, hidden]:
    returns (x [..., C_ch], z [..., Z], g [..., H_v], beta [..., H_v]), all
    float64 (x and z unrounded)."""
    H = _widen(h)
    W = _widen(w_in)
    assert W.shape[0] == C_ch + Z + 2 * H_v and W.shape[1] == H.shape[-1]
    Y = H @ W.T  # library matmul as the product step
    x = Y[..., :C_ch]
    z = Y[..., C_ch:C_ch + Z]
    b = Y[..., C_ch + Z:C_ch + Z + H_v]
    a = Y[..., C_ch + Z + H_v:]
    g, beta = decay_beta(a, b, A_log, dt_bias)
    return x, z, g, beta


# ---------------------------------------------------------------------------
# Full attention of the hybrid schedule ("Add a performance-parity Qwen3.8-27B
# Q4 and Q8 text backend on Metal", section Model and reference contract:
# three Gated DeltaNet layers to one full-attention layer; section
# Measurements and gates: the hybrid block; "Implement the Qwen3.8 Flash Next
# Rust and Metal text core", section Implementation: Qwen RoPE and exact dense
# 24Q/2KV causal attention; its implementation comment: BF16 KV storage).
# Readings: RoPE rotates the pairs (i, i + r/2), i < r/2, of the first r
# dimensions of each head by pos * base^(-2i/r) (the rotate-half form); query
# head h reads key/value head h / (H_q / H_kv); o = softmax(scale q k^T over
# keys at positions <= the query's) v; the cache holds the rotated keys and
# the values in bf16.

def _to_bf16_bits(a):
    """float64 -> bf16 bits, round to nearest even (the cache's storage)."""
    a = np.ascontiguousarray(a, np.float64)
    bits = a.view(np.uint64)
    lsb = (bits >> np.uint64(45)) & np.uint64(1)
    r = ((bits + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)).view(np.float64)
    return (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def rope(u, pos, rot_dim: int, base: float):
    """Rotate the first rot_dim dimensions of u [..., T, H, d] (float64) at
    positions pos [T]."""
    u = np.array(u, np.float64, copy=True)
    half = rot_dim // 2
    if half == 0:
        return u
    inv = base ** (-2.0 * np.arange(half) / rot_dim)
    ang = np.asarray(pos, np.float64)[:, None] * inv[None, :]  # [T, half]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    a = u[..., :half].copy()
    b = u[..., half:rot_dim].copy()
    u[..., :half] = a * c - b * s
    u[..., half:rot_dim] = b * c + a * s
    return u


def attention(q, k, v, q_pos, k_pos, scale: float):
    """Causal GQA attention in float64: q [B, Tq, H_q, d] at positions q_pos
    [Tq], k, v [B, Tk, H_kv, d] at positions k_pos [Tk]; query t sees the keys
    with k_pos <= q_pos[t].  Returns o [B, Tq, H_q, d]."""
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    B, Tq, H_q, d = q.shape
    H_kv = k.shape[2]
    G = H_q // H_kv
    o = np.empty_like(q)
    mask = np.asarray(k_pos)[None, :] <= np.asarray(q_pos)[:, None]  # [Tq, Tk]
    for b in range(B):
        for h in range(H_q):
            kh = h // G
            s = scale * (q[b, :, h] @ k[b, :, kh].T)  # [Tq, Tk]
            s = np.where(mask, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            o[b, :, h] = p @ v[b, :, kh]
    return o


def attn_layer(q, k, v, k_cache, v_cache, pos0: int, *, rot_dim: int, base: float, scale: float):
    """One attention call over T new tokens at positions pos0 .. pos0+T-1 with
    the cache's first pos0 positions as earlier context.  q [B, T, H_q, d],
    k, v [B, T, H_kv, d] (bf16 bits or float32); k_cache, v_cache [B, T_max,
    H_kv, d] bf16 bits.  Returns (o float64, k_cache, v_cache updated: the
    rotated keys and the values of the new tokens, rounded to bf16)."""
    T = np.asarray(q).shape[1]
    pos = np.arange(pos0, pos0 + T)
    qr = rope(_widen(q), pos, rot_dim, base)
    kr = rope(_widen(k), pos, rot_dim, base)
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    kc[:, pos0:pos0 + T] = _to_bf16_bits(kr)
    vc[:, pos0:pos0 + T] = _to_bf16_bits(_widen(v))
    L = pos0 + T
    o = attention(qr, _widen(kc[:, :L]), _widen(vc[:, :L]), pos, np.arange(L), scale)
    return o, kc, vc
