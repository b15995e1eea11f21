"""Helpers shared by the GPU parity tests: moving the seeded inputs to the
device, running the library through its binding, and running the oracle on
the very same inputs."""
from __future__ import annotations

import numpy as np

from gdn_inputs import Geometry

EPS = 1e-6
TOL = 2e-3  # relative L2 bound on outputs and final state (fp32 state, bf16 inputs)


def rel_l2(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


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
