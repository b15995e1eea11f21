"""GPU invariants of the GDN layer, through the C ABI.

From the pages ("Implement the Qwen3.8 Flash Next Rust and Metal text core",
section Verification and the implementation comment): prefill and decode
agree across chunk sizes, checkpoint/resume reproduces the recurrent state and
the conv history byte for byte, and the state survives save/restore without
drift.  Plus: run-to-run determinism, the beta = 0 / a = 1 identity, bf16
output, replay of a captured decode graph, and the long-context workload.
"""
from __future__ import annotations

import numpy as np
import pytest

from gdn_inputs import Geometry, make_inputs, workload_inputs
from gdn_testlib import (TOL, check_errors, dev_inputs, dims_of, from_dev, gpu_decode_seq,
                         gpu_prefill, oracle_run, rel_l2)

pytestmark = pytest.mark.gpu


def qwen(T, B=1, seed=0, zero_state=True, **kw):
    geom = Geometry(B=B, T=T, H_k=16, H_v=48, d_k=128, d_v=128, zero_state=zero_state, **kw)
    return geom, make_inputs(geom, seed)


def run_split(geom, I, chunk, split):
    """Prefill [0, split) then [split, T) with the states carried on the device."""
    import gated_deltanet_layer_gdn_amd as gdn
    import torch

    d = dims_of(geom)
    D = dev_inputs(I)
    ys = []
    for a, b in ((0, split), (split, geom.T)):
        part = {k: D[k][:, a:b].contiguous() for k in ("x", "z", "g", "beta")}
        ys.append(gdn.prefill_chunked(d, part["x"], part["z"], part["g"], part["beta"], D["w"],
                                      D["hist"], D["S"], chunk=chunk))
    torch.cuda.synchronize()
    return torch.cat(ys, 1).cpu().numpy(), D["S"].cpu().numpy(), from_dev(D["hist"])


def test_prefill_equals_decode_steps_t4096():
    wl, I = workload_inputs(2)
    yp, Sp, hp = gpu_prefill(wl.geom, I, 64)
    yd, Sd, hd = gpu_decode_seq(wl.geom, I)
    check_errors("prefill vs 4096 decode steps", yp, yd, Sp, Sd)
    np.testing.assert_array_equal(hp, hd)


def test_chunk_sizes_agree():
    geom, I = qwen(T=600, seed=21, zero_state=False)
    ref = oracle_run(geom, I)
    outs = {C: gpu_prefill(geom, I, C) for C in (16, 32, 64, 128)}
    for C, (y, S, h) in outs.items():
        check_errors(f"chunk {C} vs oracle", y, ref[0], S, ref[1])
        np.testing.assert_array_equal(h, ref[2])
    for C in (16, 32, 128):
        assert rel_l2(outs[C][0], outs[64][0]) <= TOL


@pytest.mark.parametrize("chunk,split", [(64, 512), (128, 512), (16, 48), (64, 100)])
def test_split_resume(chunk, split):
    geom, I = qwen(T=1000, seed=5)
    y, S, h = gpu_prefill(geom, I, chunk)
    ys, Ss, hs = run_split(geom, I, chunk, split)
    np.testing.assert_array_equal(hs, h)
    if split % chunk == 0:  # chunk-aligned: the same chunk schedule, bit for bit
        np.testing.assert_array_equal(ys.view(np.uint32), y.astype(np.float32).view(np.uint32))
        np.testing.assert_array_equal(Ss.view(np.uint32), S.view(np.uint32))
    else:
        assert rel_l2(ys, y) <= TOL and rel_l2(Ss, S) <= TOL


def test_save_restore_resume_bitwise():
    import gated_deltanet_layer_gdn_amd as gdn
    import torch

    geom, I = qwen(T=512, seed=6)
    d = dims_of(geom)
    y_full, S_full, h_full = gpu_prefill(geom, I, 64)
    D = dev_inputs(I)
    a = {k: D[k][:, :256].contiguous() for k in ("x", "z", "g", "beta")}
    gdn.prefill_chunked(d, a["x"], a["z"], a["g"], a["beta"], D["w"], D["hist"], D["S"], chunk=64)
    torch.cuda.synchronize()
    blob = gdn.state_save(d, D["hist"], D["S"])
    assert blob.size == gdn.state_blob_bytes(d)
    assert gdn.state_check(d, blob) == 0
    # fresh buffers (garbage), restore, continue
    hist2 = torch.full_like(D["hist"], 3.0)
    S2 = torch.full_like(D["S"], -1.0)
    gdn.state_restore(d, blob, hist2, S2)
    np.testing.assert_array_equal(from_dev(hist2), from_dev(D["hist"]))
    np.testing.assert_array_equal(S2.cpu().numpy().view(np.uint32), D["S"].cpu().numpy().view(np.uint32))
    blob2 = gdn.state_save(d, hist2, S2)
    np.testing.assert_array_equal(blob2, blob)  # save -> restore -> save: identical bytes
    b = {k: D[k][:, 256:].contiguous() for k in ("x", "z", "g", "beta")}
    y2 = gdn.prefill_chunked(d, b["x"], b["z"], b["g"], b["beta"], D["w"], hist2, S2, chunk=64)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y2.cpu().numpy().view(np.uint32),
                                  y_full[:, 256:].astype(np.float32).view(np.uint32))
    np.testing.assert_array_equal(S2.cpu().numpy().view(np.uint32), S_full.view(np.uint32))
    # a corrupted blob is refused and the destination is not touched
    bad = blob.copy()
    bad[-3] ^= 0x10
    with pytest.raises(gdn.GdnError, match="CHECKSUM"):
        gdn.state_restore(d, bad, hist2, S2)
    np.testing.assert_array_equal(S2.cpu().numpy().view(np.uint32), S_full.view(np.uint32))


def test_run_twice_bitwise():
    geom, I = qwen(T=300, seed=8, zero_state=False)
    a = gpu_prefill(geom, I, 64)
    b = gpu_prefill(geom, I, 64)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(np.asarray(u).view(np.uint8), np.asarray(v).view(np.uint8))
    geom1, I1 = qwen(T=3, B=4, seed=9, zero_state=False)
    a = gpu_decode_seq(geom1, I1)
    b = gpu_decode_seq(geom1, I1)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(np.asarray(u).view(np.uint8), np.asarray(v).view(np.uint8))


def test_beta0_decay1_keeps_state_bitwise():
    geom, I = qwen(T=130, seed=10, zero_state=False)
    I["g"][:] = 0.0
    I["beta"][:] = 0.0
    _, S, _ = gpu_prefill(geom, I, 64)
    np.testing.assert_array_equal(S.view(np.uint32), I["S"].view(np.uint32))
    g1, I1 = qwen(T=2, seed=11, zero_state=False)
    I1["g"][:] = 0.0
    I1["beta"][:] = 0.0
    _, S1, _ = gpu_decode_seq(g1, I1)
    np.testing.assert_array_equal(S1.view(np.uint32), I1["S"].view(np.uint32))


def test_bf16_output():
    import gated_deltanet_layer_gdn_amd as gdn
    from gdn_inputs import bf16_bits_to_f32, f64_to_bf16_bits

    geom, I = qwen(T=200, seed=12, zero_state=False)
    y_ref, S_ref, _ = oracle_run(geom, I)
    d = dims_of(geom, out_dtype=gdn.BF16)
    y, S, _ = gpu_prefill(geom, I, 64, dims=d)
    y_ref_bf16 = bf16_bits_to_f32(f64_to_bf16_bits(y_ref)).astype(np.float64)
    check_errors("bf16 y vs bf16-rounded oracle", y, y_ref_bf16, S, S_ref)
    yd, Sd, _ = gpu_decode_seq(geom, I, dims=d)
    check_errors("bf16 y, decode steps, vs bf16-rounded oracle", yd, y_ref_bf16, Sd, S_ref)


def test_decode_graph_replay_matches_eager():
    import gated_deltanet_layer_gdn_amd as gdn
    import torch

    geom, I = qwen(T=1, B=8, seed=13, zero_state=False)
    d = dims_of(geom)
    D = dev_inputs(I)
    ws = torch.empty(gdn.decode_workspace_bytes(d), dtype=torch.uint8, device="cuda")
    S_g, h_g = D["S"].clone(), D["hist"].clone()
    S_e, h_e = D["S"].clone(), D["hist"].clone()
    y_g = torch.empty((geom.B, 1, geom.H_v, geom.d_v), device="cuda")
    args = (D["x"], D["z"], D["g"], D["beta"], D["w"])
    gdn.decode_step(d, *args, h_g, S_g, y=y_g, ws=ws)  # warm-up outside capture
    torch.cuda.synchronize()
    S_g.copy_(D["S"])
    h_g.copy_(D["hist"])
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gdn.decode_step(d, *args, h_g, S_g, y=y_g, ws=ws)
    # capture does not execute; replay three times with eager work in between
    for rep in range(3):
        graph.replay()
        torch.cuda.synchronize()
        y_e = gdn.decode_step(d, *args, h_e, S_e)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(S_g.cpu().numpy().view(np.uint32), S_e.cpu().numpy().view(np.uint32))
        np.testing.assert_array_equal(y_g.cpu().numpy().view(np.uint32), y_e.cpu().numpy().view(np.uint32))
        np.testing.assert_array_equal(from_dev(h_g), from_dev(h_e))


# ----------------------------------------------------------------- long context (T = 65536)

@pytest.fixture(scope="module")
def long_ctx():
    # Every value head of the long-context workload against one full oracle
    # run (the oracle has no chunk size, so one run serves both chunk sizes).
    wl, I = workload_inputs(4)
    print(f"[invariant] long-context inputs ready: {wl.name}", flush=True)
    ref = oracle_run(wl.geom, I)
    print("[invariant] long-context oracle done", flush=True)
    return wl.geom, I, ref


@pytest.mark.timeout(900)
@pytest.mark.parametrize("chunk", [64, 128])
def test_long_context_all_heads_and_resume(long_ctx, chunk):
    import torch

    geom, I, (yr, Sr, hr) = long_ctx
    y, S, h = gpu_prefill(geom, I, chunk)
    check_errors(f"T=65536 C={chunk}, all {geom.H_v} heads", y, yr, S, Sr)
    np.testing.assert_array_equal(h, hr)
    # checkpoint at token 32768 (through a saved blob), resume, compare bit for bit
    import gated_deltanet_layer_gdn_amd as gdn

    d = dims_of(geom)
    D = dev_inputs(I)
    half = geom.T // 2
    a = {k: D[k][:, :half].contiguous() for k in ("x", "z", "g", "beta")}
    ya = gdn.prefill_chunked(d, a["x"], a["z"], a["g"], a["beta"], D["w"], D["hist"], D["S"],
                             chunk=chunk)
    torch.cuda.synchronize()
    blob = gdn.state_save(d, D["hist"], D["S"])
    del a
    h2 = torch.zeros_like(D["hist"])
    S2 = torch.zeros_like(D["S"])
    gdn.state_restore(d, blob, h2, S2)
    b = {k: D[k][:, half:].contiguous() for k in ("x", "z", "g", "beta")}
    yb = gdn.prefill_chunked(d, b["x"], b["z"], b["g"], b["beta"], D["w"], h2, S2, chunk=chunk)
    torch.cuda.synchronize()
    y32 = y.astype(np.float32)
    np.testing.assert_array_equal(ya.cpu().numpy().view(np.uint32), y32[:, :half].view(np.uint32))
    np.testing.assert_array_equal(yb.cpu().numpy().view(np.uint32), y32[:, half:].view(np.uint32))
    np.testing.assert_array_equal(S2.cpu().numpy().view(np.uint32), S.view(np.uint32))
    np.testing.assert_array_equal(from_dev(h2), h)


def test_timed_variants_match_plain_calls():
    # The timed entry points (per-kernel durations from events at each
    # kernel's own start and end) leave every result bit-identical to the
    # plain calls; every kernel that ran reports a positive duration, and the
    # conv entry is 0 where prep computes the q/k conv (no conv launch).
    import gated_deltanet_layer_gdn_amd as gdn
    import torch

    geom = Geometry(B=1, T=300, H_k=4, H_v=12, d_k=128, d_v=128, zero_state=False)
    I = make_inputs(geom, 77)
    d = dims_of(geom)
    outs = []
    for timed in (False, True):
        D = dev_inputs(I)
        km = [] if timed else None
        y = gdn.prefill_chunked(d, D["x"], D["z"], D["g"], D["beta"], D["w"], D["hist"], D["S"],
                                chunk=64, kernel_ms=km)
        x1 = D["x"][:, :1].reshape(geom.B, -1).contiguous()
        z1 = D["z"][:, :1].reshape(geom.B, geom.H_v, geom.d_v).contiguous()
        g1 = D["g"][:, :1].reshape(geom.B, geom.H_v).contiguous()
        b1 = D["beta"][:, :1].reshape(geom.B, geom.H_v).contiguous()
        kd = [] if timed else None
        yd = gdn.decode_step(d, x1, z1, g1, b1, D["w"], D["hist"], D["S"], kernel_ms=kd)
        torch.cuda.synchronize()
        outs.append((y.cpu().numpy(), yd.cpu().numpy(), D["S"].cpu().numpy(), from_dev(D["hist"])))
        if timed:
            assert len(km) == 3 and all(v > 0 for v in km), km  # conv pass, prep, state pass
            assert len(kd) == 2 and all(v > 0 for v in kd), kd  # conv step, state stream
    for a, b in zip(*outs):
        np.testing.assert_array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))


@pytest.mark.timeout(900)
def test_largest_token_count_one_call_equals_split():
    # The largest T a call accepts (2^24 tokens), on one key head and one
    # value head of 128 (chunk 64: the passes whose q/k slices are addressed
    # with 32-bit offsets, which that limit keeps below 2^32): one call
    # against the same tokens in two chunk-aligned calls, bit for bit, and its
    # first 4096 outputs against the fp64 oracle.  Inputs are drawn on the
    # device in slices (same distributions as the seeded workloads).
    import gated_deltanet_layer_gdn_amd as gdn
    import oracle
    import torch

    T = 1 << 24
    geom = Geometry(B=1, T=T, H_k=1, H_v=1, d_k=128, d_v=128)
    d = dims_of(geom)
    C_ch = 3 * 128
    gen = torch.Generator(device="cuda").manual_seed(2024)
    x = torch.empty((1, T, C_ch), dtype=torch.bfloat16, device="cuda")
    z = torch.empty((1, T, 1, 128), dtype=torch.bfloat16, device="cuda")
    g = torch.empty((1, T, 1), dtype=torch.float32, device="cuda")
    beta = torch.empty((1, T, 1), dtype=torch.float32, device="cuda")
    step = 1 << 20
    for t0 in range(0, T, step):
        x[:, t0:t0 + step] = torch.randn((1, step, C_ch), device="cuda", generator=gen).to(torch.bfloat16)
        z[:, t0:t0 + step] = torch.randn((1, step, 1, 128), device="cuda", generator=gen).to(torch.bfloat16)
        g[:, t0:t0 + step] = -torch.nn.functional.softplus(torch.randn((1, step, 1), device="cuda", generator=gen))
        beta[:, t0:t0 + step] = torch.sigmoid(torch.randn((1, step, 1), device="cuda", generator=gen))
    w = (0.5 * torch.randn((C_ch, 4), device="cuda", generator=gen)).to(torch.bfloat16)
    print("[invariant] 2^24-token inputs drawn", flush=True)
    ws = torch.empty(gdn.prefill_workspace_bytes(d, T, 64), dtype=torch.uint8, device="cuda")

    def fresh():
        return (torch.zeros((1, 3, C_ch), dtype=torch.bfloat16, device="cuda"),
                torch.zeros((1, 1, 128, 128), dtype=torch.float32, device="cuda"))

    h1, S1 = fresh()
    y1 = gdn.prefill_chunked(d, x, z, g, beta, w, h1, S1, chunk=64, ws=ws)
    torch.cuda.synchronize()
    print("[invariant] one call done", flush=True)
    h2, S2 = fresh()
    half = T // 2
    ya = gdn.prefill_chunked(d, x[:, :half], z[:, :half], g[:, :half], beta[:, :half], w, h2, S2,
                             chunk=64, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(ya.view(torch.int32), y1[:, :half].view(torch.int32))
    del ya
    yb = gdn.prefill_chunked(d, x[:, half:], z[:, half:], g[:, half:], beta[:, half:], w, h2, S2,
                             chunk=64, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(yb.view(torch.int32), y1[:, half:].view(torch.int32))
    assert torch.equal(S2.view(torch.int32), S1.view(torch.int32))
    assert torch.equal(h2.view(torch.int16), h1.view(torch.int16))
    del yb
    assert bool(torch.isfinite(S1).all()) and bool(torch.isfinite(y1[:, -4096:]).all())
    # the first 4096 tokens against the oracle (they depend on nothing later)
    n = 4096
    I = {"x": from_dev(x[:, :n].contiguous()), "z": from_dev(z[:, :n].contiguous()),
         "g": g[:, :n].cpu().numpy(), "beta": beta[:, :n].cpu().numpy(), "w": from_dev(w),
         "hist": np.zeros((1, 3, C_ch), np.uint16), "S": np.zeros((1, 1, 128, 128), np.float32)}
    yr, _, _ = oracle.layer(I["x"], I["z"], I["g"], I["beta"], I["w"], I["hist"], I["S"],
                            H_k=1, H_v=1, d_k=128, d_v=128, eps=d.l2_eps)
    e = rel_l2(y1[:, :n].double().cpu().numpy(), yr)
    print(f"[invariant] T=2^24: first {n} outputs rel_l2 {e:.3e}", flush=True)
    assert e <= TOL
