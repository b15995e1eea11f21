"""GPU parity of the input projections with the fused decay/beta
parametrisation (gdn_in_proj) against the oracle ("Implement the Qwen3.8
Flash Next Rust and Metal text core", section Verification: GDN projection).

x and z are bf16 products of an fp32-accumulated GEMM: they are compared with
the fp64 products rounded to bf16, every element within one bf16 step of it
(2^-7 of its magnitude, plus 1e-4 of the RMS for results near zero, where the
fp32 accumulation error decides the rounding); g and beta (fp32) to 1e-5
relative."""
from __future__ import annotations

import numpy as np
import pytest

from gdn_inputs import Geometry, bf16_bits_to_f32, f64_to_bf16_bits, make_inputs, make_proj_inputs
from gdn_testlib import check_errors, dims_of, gpu_prefill, oracle_run, rel_l2, to_dev

pytestmark = pytest.mark.gpu


def bf16_round(a):
    return bf16_bits_to_f32(f64_to_bf16_bits(a)).astype(np.float64)


def check_proj(name, got, ref, rows=None):
    x, z, g, beta = got
    xr, zr, gr, br = ref
    if rows is not None:
        x, z, g, beta = x[rows], z[rows], g[rows], beta[rows]
    for nm, a, r in (("x", x, xr), ("z", z, zr)):
        rr = bf16_round(r)
        step = np.abs(rr) * 2.0 ** -7 + 1e-4 * np.sqrt(np.mean(r ** 2))
        err = np.abs(a - rr)
        e = rel_l2(a, r)
        print(f"[parity] {name} {nm}: rel_l2 vs fp64 {e:.3e}, max |err|/step {np.max(err / step):.3f}, "
              f"elements off the rounded value {np.mean(err > 0):.2e}", flush=True)
        assert np.all(err <= step), nm
        assert e <= 3e-3
    for nm, a, r in (("g", g, gr), ("beta", beta, br)):
        e = np.max(np.abs(a - r) / np.maximum(np.abs(r), 1e-30))
        print(f"[parity] {name} {nm}: max rel err {e:.3e}", flush=True)
        assert e <= 1e-5, nm


def run_proj(d, P):
    import gated_deltanet_layer_gdn_amd as gdn
    import torch

    out = gdn.in_proj(d, to_dev(P["h"]), to_dev(P["w_in"]), to_dev(P["A_log"]), to_dev(P["dt_bias"]))
    torch.cuda.synchronize()
    return tuple(t.double().cpu().numpy() for t in out)


def oracle_proj(P, H_k, H_v, dd):
    import oracle

    return oracle.in_proj(P["h"], P["w_in"], P["A_log"], P["dt_bias"], C_ch=(2 * H_k + H_v) * dd,
                          Z=H_v * dd, H_v=H_v)


@pytest.mark.parametrize("B,T,hidden", [(2, 77, 256), (1, 129, 640), (3, 1, 64)])
def test_in_proj_small(B, T, hidden):
    geom = Geometry(B=B, T=T, H_k=16, H_v=48, d_k=128, d_v=128)
    P = make_proj_inputs(B, T, hidden, 16, 48, 128, seed=700 + T)
    got = run_proj(dims_of(geom), P)
    x, z, g, beta = oracle_proj(P, 16, 48, 128)
    ref = (x, z.reshape(B, T, 48, 128), g, beta)
    check_proj(f"in_proj B={B} T={T} hidden={hidden}", got, ref)


# Other head counts: C_ch = 640 (H_k=1, H_v=3) is not a multiple of 256, so
# the register-staged tiles cover x and z (one tile holds both); at H_k=2,
# H_v=4 (C_ch = 1024, H_v d_v = 512) the direct-to-LDS tiles do, with K = 192
# and 320 (six and ten K steps: the pipeline's peeled last steps).
@pytest.mark.parametrize("H_k,H_v,T,hidden", [(1, 3, 70, 192), (2, 4, 300, 320), (1, 3, 257, 64)])
def test_in_proj_other_head_counts(H_k, H_v, T, hidden):
    geom = Geometry(B=1, T=T, H_k=H_k, H_v=H_v, d_k=128, d_v=128)
    P = make_proj_inputs(1, T, hidden, H_k, H_v, 128, seed=730 + T)
    got = run_proj(dims_of(geom), P)
    x, z, g, beta = oracle_proj(P, H_k, H_v, 128)
    ref = (x, z.reshape(1, T, H_v, 128), g, beta)
    check_proj(f"in_proj H={H_k}/{H_v} T={T} hidden={hidden}", got, ref)


def test_in_proj_qwen_size_sampled_rows():
    # M = 4096 tokens, hidden 5120 (the pages' hidden size), all 16,480
    # output columns; the oracle computes 96 sampled token rows.
    B, T, hidden = 1, 4096, 5120
    geom = Geometry(B=B, T=T, H_k=16, H_v=48, d_k=128, d_v=128)
    P = make_proj_inputs(B, T, hidden, 16, 48, 128, seed=710)
    got = run_proj(dims_of(geom), P)
    rows = np.sort(np.random.default_rng(1).choice(T, 96, replace=False))
    Ps = dict(P, h=np.ascontiguousarray(P["h"][:, rows]))
    x, z, g, beta = oracle_proj(Ps, 16, 48, 128)
    got_s = tuple(a[:, rows] for a in got)
    check_proj("in_proj T=4096 hidden=5120 (96 rows)", got_s, (x, z.reshape(1, 96, 48, 128), g, beta))


def test_in_proj_feeds_the_layer():
    # Projections, then the chunked prefill, against the oracle's projections
    # (x and z rounded to bf16, as the layer takes them) and its layer.
    import gated_deltanet_layer_gdn_amd as gdn
    import torch

    B, T, hidden = 1, 300, 512
    geom = Geometry(B=B, T=T, H_k=16, H_v=48, d_k=128, d_v=128, zero_state=False)
    P = make_proj_inputs(B, T, hidden, 16, 48, 128, seed=720)
    base = make_inputs(geom, seed=721)
    d = dims_of(geom)
    x, z, g, beta = gdn.in_proj(d, to_dev(P["h"]), to_dev(P["w_in"]), to_dev(P["A_log"]),
                                to_dev(P["dt_bias"]))
    hist, S = to_dev(base["hist"]), to_dev(base["S"])
    y = gdn.prefill_chunked(d, x, z, g, beta, to_dev(base["w"]), hist, S, chunk=64)
    torch.cuda.synchronize()
    xo, zo, go, bo = oracle_proj(P, 16, 48, 128)
    I = dict(base, x=f64_to_bf16_bits(xo), z=f64_to_bf16_bits(zo.reshape(B, T, 48, 128)),
             g=go.astype(np.float32), beta=bo.astype(np.float32))
    yr, Sr, _ = oracle_run(geom, I)
    check_errors("in_proj + prefill vs oracle in_proj + layer", y.double().cpu().numpy(), yr,
                 S.cpu().numpy(), Sr)
