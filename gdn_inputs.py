"""Seeded synthetic inputs for the GDN layer workloads.

This module only draws random numbers and casts them: it holds none of the
layer's arithmetic, and both the oracle checks and the GPU path take their
inputs from here.

Recipe (one numpy ``default_rng(seed)`` stream per workload, seed = workload
index unless given; draws are float64 in the order x, z, g_raw, beta_raw,
conv_w, conv_hist, S):

* x, z ~ N(0, 1); conv_w ~ N(0, 0.5) (0.5 is the standard deviation);
* g = -softplus(g_raw), so the decay a = exp(g) lies in (0, 1);
  beta = sigmoid(beta_raw); g_raw, beta_raw ~ N(0, 1); both cast to float32;
* conv history ~ N(0, 1) for the decode workloads, zero for prefill ones;
* recurrent state ~ N(0, 0.1) (std) as float32 for the decode workloads, zero
  for prefill ones;
* bf16 tensors are rounded to nearest-even straight from float64 and held as
  uint16 bit patterns; float32 tensors are rounded to nearest from float64.

Large tensors are drawn in row blocks from the same stream, which gives the
same values as one draw.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np


@dataclass(frozen=True)
class Geometry:
    B: int
    T: int
    H_k: int
    H_v: int
    d_k: int
    d_v: int
    W: int = 4
    dtype: str = "bf16"  # 'bf16' or 'f32' for x, z, conv_w, conv history
    zero_state: bool = True  # zero conv history and recurrent state
    g_scale: float = 1.0  # g = -g_scale * softplus(N(0,1)); < 1 gives weak decay

    @property
    def C_ch(self) -> int:
        return 2 * self.H_k * self.d_k + self.H_v * self.d_v


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    geom: Geometry
    chunks: tuple = field(default=())
    mode: str = "prefill"  # 'prefill' or 'decode'


WORKLOADS = {
    0: Workload(0, "tiny fp32 layer, B=1 T=64, 2/2 heads, d=16",
                Geometry(B=1, T=64, H_k=2, H_v=2, d_k=16, d_v=16, dtype="f32"),
                chunks=(16, 32, 64)),
    1: Workload(1, "decode step, B=1, 16/48 heads, d=128",
                Geometry(B=1, T=1, H_k=16, H_v=48, d_k=128, d_v=128, zero_state=False),
                mode="decode"),
    2: Workload(2, "prefill, B=1 T=4096, 16/48 heads, d=128, chunk 64",
                Geometry(B=1, T=4096, H_k=16, H_v=48, d_k=128, d_v=128), chunks=(64,)),
    3: Workload(3, "batched decode step, B=64, 16/48 heads, d=128",
                Geometry(B=64, T=1, H_k=16, H_v=48, d_k=128, d_v=128, zero_state=False),
                mode="decode"),
    4: Workload(4, "long prefill, B=1 T=65536, 16/48 heads, d=128, chunks 64/128",
                Geometry(B=1, T=65536, H_k=16, H_v=48, d_k=128, d_v=128), chunks=(64, 128)),
}

_ROUND_BITS = np.uint64(45)  # float64 keeps 52 mantissa bits, bf16 keeps 7


def f64_to_bf16_bits(a) -> np.ndarray:
    """Round float64 to bf16 (nearest, ties to even) -> uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float64)
    bits = a.view(np.uint64)
    lsb = (bits >> _ROUND_BITS) & np.uint64(1)
    half = np.uint64((1 << 44) - 1)
    mask = ~np.uint64((1 << 45) - 1)
    r = ((bits + half + lsb) & mask).view(np.float64).astype(np.float32)
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(a) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    return (np.asarray(a, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _cast(a64: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f64_to_bf16_bits(a64)
    if dtype == "f32":
        return a64.astype(np.float32)
    raise ValueError(dtype)


def _normal_cast(rng, shape, std, dtype, rows_per_block=2048):
    """Draw N(0, std^2) of ``shape`` row block by row block and cast."""
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, np.uint16 if dtype == "bf16" else np.float32)
    flat = out.reshape(-1, shape[-1]) if len(shape) > 1 else out.reshape(1, -1)
    n = flat.shape[0]
    for r0 in range(0, n, rows_per_block):
        r1 = min(n, r0 + rows_per_block)
        blk = rng.standard_normal((r1 - r0, flat.shape[1]))
        if std != 1.0:
            blk *= std
        flat[r0:r1] = _cast(blk, dtype)
    return out


def make_inputs(geom: Geometry, seed: int) -> dict:
    """All inputs of one layer call as numpy arrays (bf16 held as uint16)."""
    rng = np.random.default_rng(seed)
    g_ = geom
    x = _normal_cast(rng, (g_.B, g_.T, g_.C_ch), 1.0, g_.dtype)
    z = _normal_cast(rng, (g_.B, g_.T, g_.H_v, g_.d_v), 1.0, g_.dtype)
    g_raw = rng.standard_normal((g_.B, g_.T, g_.H_v))
    g = (-g_.g_scale * np.logaddexp(0.0, g_raw)).astype(np.float32)
    b_raw = rng.standard_normal((g_.B, g_.T, g_.H_v))
    beta = (1.0 / (1.0 + np.exp(-b_raw))).astype(np.float32)
    w = _cast(rng.standard_normal((g_.C_ch, g_.W)) * 0.5, g_.dtype)
    hist_shape = (g_.B, g_.W - 1, g_.C_ch)
    S_shape = (g_.B, g_.H_v, g_.d_v, g_.d_k)
    if g_.zero_state:
        hist = np.zeros(hist_shape, np.uint16 if g_.dtype == "bf16" else np.float32)
        S = np.zeros(S_shape, np.float32)
    else:
        hist = _normal_cast(rng, hist_shape, 1.0, g_.dtype)
        S = _normal_cast(rng, S_shape, 0.1, "f32")
    return dict(x=x, z=z, g=g, beta=beta, w=w, hist=hist, S=S)


def workload_inputs(index: int, **overrides) -> tuple[Workload, dict]:
    wl = WORKLOADS[index]
    geom = replace(wl.geom, **overrides) if overrides else wl.geom
    return replace(wl, geom=geom), make_inputs(geom, seed=index)


def make_proj_inputs(B: int, T: int, hidden: int, H_k: int, H_v: int, d: int, seed: int) -> dict:
    """Inputs of the input projections: hidden states h ~ N(0, 1) and the fused
    weight w_in ~ N(0, 1/hidden) (so the products are about N(0, 1)), both bf16;
    per value head A_log ~ U(0, 2.77) and dt_bias ~ U(-6.9, -2.25), fp32 (the
    usual initialisation ranges of this kind of gate: exp(A_log) in [1, 16],
    a decay step of 0.001 to 0.1 at zero input)."""
    rng = np.random.default_rng(seed)
    C_ch = 2 * H_k * d + H_v * d
    N = C_ch + H_v * d + 2 * H_v
    h = _normal_cast(rng, (B, T, hidden), 1.0, "bf16")
    w_in = _normal_cast(rng, (N, hidden), hidden ** -0.5, "bf16")
    A_log = rng.uniform(0.0, 2.77, H_v).astype(np.float32)
    dt_bias = rng.uniform(-6.9, -2.25, H_v).astype(np.float32)
    return dict(h=h, w_in=w_in, A_log=A_log, dt_bias=dt_bias)


def make_attn_inputs(B: int, T: int, pos0: int, T_max: int, H_q: int, H_kv: int, d: int, seed: int,
                     q_std: float = 1.0) -> dict:
    """Inputs of one full-attention call: q [B, T, H_q, d] ~ N(0, q_std^2),
    k, v [B, T, H_kv, d] ~ N(0, 1), all bf16; the KV cache [B, T_max, H_kv, d]
    holds N(0, 1) bf16 keys and values at positions 0 .. pos0 - 1 (the earlier
    context) and zeros after.  With the score scale 1/sqrt(d), q_std = 1 gives
    scores of about unit spread; a larger q_std gives sharper attention."""
    rng = np.random.default_rng(seed)
    q = _normal_cast(rng, (B, T, H_q, d), q_std, "bf16")
    k = _normal_cast(rng, (B, T, H_kv, d), 1.0, "bf16")
    v = _normal_cast(rng, (B, T, H_kv, d), 1.0, "bf16")
    kc = np.zeros((B, T_max, H_kv, d), np.uint16)
    vc = np.zeros_like(kc)
    if pos0:
        kc[:, :pos0] = _normal_cast(rng, (B, pos0, H_kv, d), 1.0, "bf16")
        vc[:, :pos0] = _normal_cast(rng, (B, pos0, H_kv, d), 1.0, "bf16")
    return dict(q=q, k=k, v=v, k_cache=kc, v_cache=vc)
