"""GPU parity of the output epilogue variants against the oracle: the
ungated readout (z = NULL), fp16 y, and the zero-centred grouped RMS norm
before the sigmoid gate ("Implement the Qwen3.8 Flash Next Rust and Metal
text core", section Implementation: zero-centred norms; its implementation
comment: zero-centred grouped RMS and the sigmoid output gate).

fp16 y is held to the bar of the unrounded oracle: its rounding (unit
roundoff 2^-11) adds about 2.5e-4 relative L2 to the kernels' ~1.2e-4, well
inside 2e-3 (bf16 y, with 8 significant bits, is compared against the
oracle rounded to bf16 instead)."""
from __future__ import annotations

import numpy as np
import pytest

from gdn_inputs import Geometry, make_inputs
from gdn_testlib import (EPS, check_errors, dims_of, from_dev, gpu_decode_seq, gpu_prefill,
                         oracle_run, to_dev)

pytestmark = pytest.mark.gpu


def f16_round(a):
    return np.asarray(a, np.float64).astype(np.float16).astype(np.float64)


def bf16_round(a):
    from gdn_inputs import bf16_bits_to_f32, f64_to_bf16_bits

    return bf16_bits_to_f32(f64_to_bf16_bits(a)).astype(np.float64)


def ungated(I):
    J = dict(I)
    J["z"] = None
    return J


def oracle_ungated(geom, I):
    import oracle

    return oracle.layer(I["x"], None, I["g"], I["beta"], I["w"], I["hist"], I["S"], H_k=geom.H_k,
                        H_v=geom.H_v, d_k=geom.d_k, d_v=geom.d_v, eps=EPS)


def gpu_prefill_opt(geom, I, chunk, dims):
    """gpu_prefill with z possibly None."""
    import gated_deltanet_layer_gdn_amd as gdn
    import torch

    D = {k: (None if v is None else to_dev(v)) for k, v in I.items()}
    y = gdn.prefill_chunked(dims, D["x"], D["z"], D["g"], D["beta"], D["w"], D["hist"], D["S"],
                            chunk=chunk)
    torch.cuda.synchronize()
    return y.double().cpu().numpy(), D["S"].cpu().numpy(), from_dev(D["hist"])


@pytest.mark.parametrize("chunk", [64, 128])
def test_ungated_prefill_and_decode(chunk):
    geom = Geometry(B=2, T=333, H_k=4, H_v=12, d_k=128, d_v=128, zero_state=False)
    I = make_inputs(geom, seed=600 + chunk)
    yr, Sr, hr = oracle_ungated(geom, I)
    y, S, h = gpu_prefill_opt(geom, ungated(I), chunk, dims_of(geom))
    check_errors(f"ungated prefill C={chunk}", y, yr, S, Sr)
    np.testing.assert_array_equal(h, hr)
    if chunk == 64:
        import gated_deltanet_layer_gdn_amd as gdn
        import torch

        d = dims_of(geom)
        D = {k: to_dev(v) for k, v in I.items()}
        ys = [gdn.decode_step(d, D["x"][:, t].contiguous(), None, D["g"][:, t].contiguous(),
                              D["beta"][:, t].contiguous(), D["w"], D["hist"], D["S"])
              for t in range(geom.T)]
        torch.cuda.synchronize()
        yd = torch.stack(ys, 1).double().cpu().numpy()
        check_errors("ungated decode steps", yd, yr, D["S"].cpu().numpy(), Sr)


@pytest.mark.parametrize("chunk", [64, 128])
def test_fp16_output(chunk):
    import gated_deltanet_layer_gdn_amd as gdn

    geom = Geometry(B=1, T=400, H_k=16, H_v=48, d_k=128, d_v=128, zero_state=False)
    I = make_inputs(geom, seed=620 + chunk)
    yr, Sr, _ = oracle_run(geom, I)
    d = dims_of(geom, out_dtype=gdn.F16)
    y, S, _ = gpu_prefill(geom, I, chunk, dims=d)
    check_errors(f"fp16 y C={chunk} vs oracle", y, yr, S, Sr)
    check_errors(f"fp16 y C={chunk} vs fp16-rounded oracle", y, f16_round(yr), S, Sr)
    if chunk == 64:
        yd, Sd, _ = gpu_decode_seq(Geometry(B=1, T=40, H_k=16, H_v=48, d_k=128, d_v=128,
                                            zero_state=False),
                                   {k: (v[:, :40] if k in ("x", "z", "g", "beta") else v)
                                    for k, v in I.items()}, dims=d)
        yr40, Sr40, _ = oracle_run(Geometry(B=1, T=40, H_k=16, H_v=48, d_k=128, d_v=128,
                                            zero_state=False),
                                   {k: (np.ascontiguousarray(v[:, :40])
                                        if k in ("x", "z", "g", "beta") else v)
                                    for k, v in I.items()})
        check_errors("fp16 y, 40 decode steps", yd, yr40, Sd, Sr40)


@pytest.mark.parametrize("out", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("gate,weight", [(True, True), (False, True), (True, False)])
def test_gated_rmsnorm_kernel(out, gate, weight):
    import gated_deltanet_layer_gdn_amd as gdn
    import oracle
    import torch

    geom = Geometry(B=3, T=37, H_k=16, H_v=48, d_k=128, d_v=128, zero_state=False)
    code = {"f32": gdn.F32, "bf16": gdn.BF16, "f16": gdn.F16}[out]
    d = dims_of(geom, out_dtype=code)
    rng = np.random.default_rng(7)
    o = (rng.standard_normal((3, 37, 48, 128)) * rng.uniform(0.01, 5, (3, 37, 48, 1))).astype(np.float32)
    I = make_inputs(geom, seed=640)
    z = I["z"] if gate else None
    w = (0.2 * rng.standard_normal(128)).astype(np.float32) if weight else None
    eps = 1e-5
    z64 = None if z is None else (z.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = oracle.gated_rmsnorm(o, z64, w, eps)
    y = gdn.gated_rmsnorm(d, to_dev(o), None if z is None else to_dev(z),
                          None if w is None else to_dev(w), eps)
    torch.cuda.synchronize()
    got = y.double().cpu().numpy()
    if out == "bf16":
        ref = bf16_round(ref)
    elif out == "f16":
        ref = f16_round(ref)
    zero_S = np.ones((1, 1, 1, 1))
    check_errors(f"gated rmsnorm out={out} gate={gate} weight={weight}", got, ref, zero_S, zero_S)


def test_norm_variant_end_to_end():
    # The layer's ungated readout, then the zero-centred grouped RMS norm and
    # the gate, against the same two steps on the oracle.
    import gated_deltanet_layer_gdn_amd as gdn
    import oracle
    import torch

    geom = Geometry(B=1, T=500, H_k=16, H_v=48, d_k=128, d_v=128, zero_state=False)
    I = make_inputs(geom, seed=660)
    w = (0.1 * np.random.default_rng(3).standard_normal(128)).astype(np.float32)
    o_ref, S_ref, _ = oracle_ungated(geom, I)
    z64 = (I["z"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    y_ref = oracle.gated_rmsnorm(o_ref, z64, w, 1e-6)
    d = dims_of(geom)
    o, S, _ = gpu_prefill_opt(geom, ungated(I), 64, d)
    for out, code in (("bf16", gdn.BF16), ("f32", gdn.F32)):
        dn = dims_of(geom, out_dtype=code)
        y = gdn.gated_rmsnorm(dn, to_dev(o.astype(np.float32)), to_dev(I["z"]), to_dev(w), 1e-6)
        torch.cuda.synchronize()
        got = y.double().cpu().numpy()
        ref = bf16_round(y_ref) if out == "bf16" else y_ref
        check_errors(f"ungated prefill + rmsnorm + gate, y {out}", got, ref, S, S_ref)
