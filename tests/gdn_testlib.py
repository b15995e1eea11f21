"""Helpers shared by the GPU parity tests: moving the seeded inputs to the
device, running the library through its binding, and running the oracle on
the very same inputs."""
from __future__ import annotations

import numpy as np

from gdn_inputs import Geometry

EPS = 1e-6
TOL = 2e-3  # relative L2 bound on outputs and final state (fp32 state, bf16 inputs)
# Per-row bound: a row is one (sequence, token, value head) of y, or one
# (sequence, value head, state row) of S, and its error is measured against
# the larger of its own reference norm and the RMS row norm of its head.  The
# measured whole-tensor errors are about 1e-4 (4-5e-4 under weak decay), so
# 1e-2 leaves a margin of 20-100x for the tail of the row distribution, while
# a row that is wrong by a fraction f of a typical row (an indexing slip in one
# token or one head) shows f, and anything above 1e-2 fails.
ROW_TOL = 1e-2


def rel_l2(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    e, r = np.linalg.norm(got - ref), np.linalg.norm(ref)
    if r == 0:  # an all-zero reference needs an all-zero result
        return 0.0 if e == 0 else float("inf")
    return float(e / r)


def _sq_rows(a) -> np.ndarray:
    a = np.asarray(a)
    return np.einsum("...i,...i->...", a, a, dtype=np.float64)


def y_errors(y, yr, block=4096):
    """Per-head relative L2 [B, H_v] and per-row relative errors [B, T, H_v]
    of outputs shaped [B, T, H_v, d_v] (processed in token blocks, so the
    long-context case needs no second full-size difference array)."""
    B, T, H = yr.shape[:3]
    err2 = np.empty((B, T, H))
    ref2 = np.empty((B, T, H))
    for t0 in range(0, T, block):
        r = np.asarray(yr[:, t0:t0 + block], np.float64)
        g = np.asarray(y[:, t0:t0 + block], np.float64)
        err2[:, t0:t0 + block] = _sq_rows(g - r)
        ref2[:, t0:t0 + block] = _sq_rows(r)
    return _head_and_rows(err2, ref2, axis=1)


def s_errors(S, Sr):
    """Per-head relative L2 [B, H_v] and per-row relative errors [B, H_v, d_v]
    of states shaped [B, H_v, d_v, d_k]."""
    S = np.asarray(S, np.float64)
    Sr = np.asarray(Sr, np.float64)
    return _head_and_rows(_sq_rows(S - Sr), _sq_rows(Sr), axis=2)


def _head_and_rows(err2, ref2, axis):
    """err2, ref2: squared row norms of the error and the reference; `axis`
    runs over the rows of one head.  A head whose reference is exactly zero
    must have zero error."""
    e_head = np.sqrt(err2.sum(axis))
    r_head = np.sqrt(ref2.sum(axis))
    head = np.where(r_head > 0, e_head / np.where(r_head > 0, r_head, 1.0),
                    np.where(e_head > 0, np.inf, 0.0))
    rms = np.sqrt(ref2.mean(axis, keepdims=True))
    floor = np.maximum(np.sqrt(ref2), rms)
    rows = np.where(floor > 0, np.sqrt(err2) / np.where(floor > 0, floor, 1.0),
                    np.where(err2 > 0, np.inf, 0.0))
    return head, rows


def check_errors(name, y, yr, S, Sr, tol=TOL, row_tol=ROW_TOL):
    """The parity bar on outputs and final state: whole-tensor relative L2,
    every value head's relative L2 (both <= tol) and every row (<= row_tol).
    Prints the figures and returns them."""
    ey, eS = rel_l2(y, yr), rel_l2(S, Sr)
    hy, ry = y_errors(y, yr)
    hs, rs = s_errors(S, Sr)
    f = dict(y=ey, S=eS, y_head=float(hy.max()), S_head=float(hs.max()),
             y_row=float(ry.max()), S_row=float(rs.max()))
    worst = np.unravel_index(int(np.argmax(ry)), ry.shape)
    print(f"[parity] {name}: rel_l2 y={ey:.3e} S={eS:.3e}; worst head y={f['y_head']:.3e} "
          f"S={f['S_head']:.3e}; worst row y={f['y_row']:.3e} (b,t,h)={tuple(int(i) for i in worst)} "
          f"S={f['S_row']:.3e}", flush=True)
    assert ey <= tol and eS <= tol, f
    assert f["y_head"] <= tol and f["S_head"] <= tol, f
    assert f["y_row"] <= row_tol and f["S_row"] <= row_tol, f
    return f


def dims_of(geom: Geometry, out_dtype: int | None = None, eps: float = EPS, q_scale: float = 1.0):
    import gated_deltanet_layer_gdn_amd as gdn

    return gdn.Dims(B=geom.B, H_k=geom.H_k, H_v=geom.H_v, d_k=geom.d_k, d_v=geom.d_v, W=geom.W,
                    in_dtype=gdn.BF16 if geom.dtype == "bf16" else gdn.F32,
                    out_dtype=gdn.F32 if out_dtype is None else out_dtype, l2_eps=eps,
                    q_scale=q_scale)


def to_dev(a):
    import torch

    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def from_dev(t) -> np.ndarray:
    import torch

    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def dev_inputs(I: dict) -> dict:
    return {k: to_dev(v) for k, v in I.items()}


def to_f64(t) -> np.ndarray:
    import torch

    return t.to(torch.float64).cpu().numpy()


def oracle_run(geom: Geometry, I: dict, heads=None, eps=EPS, q_scale=1.0):
    import oracle

    return oracle.layer(I["x"], I["z"], I["g"], I["beta"], I["w"], I["hist"], I["S"],
                        H_k=geom.H_k, H_v=geom.H_v, d_k=geom.d_k, d_v=geom.d_v, eps=eps,
                        q_scale=q_scale, heads=heads)


def gpu_prefill(geom: Geometry, I: dict, chunk: int, dims=None):
    """Run gdn_prefill_chunked on fresh device copies; returns (y, S, hist) as numpy."""
    import gated_deltanet_layer_gdn_amd as gdn
    import torch

    d = dims or dims_of(geom)
    D = dev_inputs(I)
    y = gdn.prefill_chunked(d, D["x"], D["z"], D["g"], D["beta"], D["w"], D["hist"], D["S"],
                            chunk=chunk)
    torch.cuda.synchronize()
    return to_f64(y), D["S"].cpu().numpy(), from_dev(D["hist"])


def gpu_decode_seq(geom: Geometry, I: dict, dims=None):
    """Run T tokens one gdn_decode_step at a time; returns (y, S, hist)."""
    import gated_deltanet_layer_gdn_amd as gdn
    import torch

    d = dims or dims_of(geom)
    D = dev_inputs(I)
    ys = []
    for t in range(geom.T):
        ys.append(gdn.decode_step(d, D["x"][:, t].contiguous(), D["z"][:, t].contiguous(),
                                  D["g"][:, t].contiguous(), D["beta"][:, t].contiguous(),
                                  D["w"], D["hist"], D["S"]))
    torch.cuda.synchronize()
    y = torch.stack(ys, dim=1)
    return to_f64(y), D["S"].cpu().numpy(), from_dev(D["hist"])
