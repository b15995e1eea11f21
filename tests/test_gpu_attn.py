"""GPU parity of the full-attention layer of the hybrid schedule (gdn_attn_prefill)
against the fp64 oracle ("Implement the Qwen3.8 Flash Next Rust and Metal text
core", section Implementation: Qwen RoPE, exact dense 24Q/2KV causal attention,
BF16 KV storage).

Error budget (fp32 output against the fp64 oracle).  The kernel rounds the
rotated queries and the softmax weights P to bf16 for the MFMA products and
accumulates in fp32; the keys and values are the cache's bf16 numbers on both
sides.  A weight rounded with relative error u (|u| <= 2^-9, RMS 2^-9/sqrt(3)
= 1.1e-3) moves o by about u times o's own size, whatever the attention's
spread, and the query rounding moves the scores by about 2^-9 / sqrt(3) of a
score's spread, a smaller effect on o.  The bound is rel L2 <= 3e-3 over the
tensor and per query head, and 1e-2 per row (one token of one head, against
the larger of its own norm and the head's RMS row norm), the rows' tail
holding a few times the RMS figure.  A bf16 output adds its own rounding
(2^-9 at most, RMS 1.1e-3) and is held to 4e-3.

The cache positions pos0 .. pos0+T-1 must hold the values bit for bit and the
rotated keys within half a bf16 step of the fp64 rotation (plus 2^-16 for keys
that cancel to near zero): the kernel rotates in fp32, so a key within fp32
error of a rounding boundary may round the other way than the oracle's (at
most 1e-3 of them may), and every other cache position must be unchanged."""
from __future__ import annotations

import numpy as np
import pytest

from gdn_inputs import bf16_bits_to_f32, make_attn_inputs
from gdn_testlib import from_dev, rel_l2, to_dev, y_errors

pytestmark = pytest.mark.gpu

QWEN = dict(H_q=24, H_kv=2, d=256, rot=64, base=1e7)  # the pages' attention shape
TOL_F32, TOL_BF16, ROW_TOL = 3e-3, 4e-3, 1e-2


def attn_dims(B, H_q, H_kv, d, rot, base, out_bf16=False):
    import gated_deltanet_layer_gdn_amd as gdn

    return gdn.AttnDims(B=B, H_q=H_q, H_kv=H_kv, d_h=d, rot_dim=rot, rope_base=base,
                        out_dtype=gdn.BF16 if out_bf16 else gdn.F32)


def run_gpu(a, I, pos0, kc=None, vc=None):
    """One call; returns (o float64, k_cache bits, v_cache bits) and the device caches."""
    import gated_deltanet_layer_gdn_amd as gdn
    import torch

    kc = to_dev(I["k_cache"]) if kc is None else kc
    vc = to_dev(I["v_cache"]) if vc is None else vc
    print(f"[attn] B={a.B} T={I['q'].shape[1]} pos0={pos0} T_max={kc.shape[1]} "
          f"H={a.H_q}/{a.H_kv} d={a.d_h} rot={a.rot_dim}", flush=True)
    o = gdn.attn_prefill(a, to_dev(I["q"]), to_dev(I["k"]), to_dev(I["v"]), kc, vc, pos0=pos0)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), kc, vc


def check_out(name, o, ref, tol):
    e = rel_l2(o, ref)
    head, rows = y_errors(o, ref)
    worst = np.unravel_index(int(np.argmax(rows)), rows.shape)
    print(f"[parity] {name}: rel_l2 {e:.3e}, worst head {head.max():.3e}, worst row {rows.max():.3e} "
          f"(b,t,h)={tuple(int(i) for i in worst)}", flush=True)
    assert e <= tol and head.max() <= tol and rows.max() <= ROW_TOL


def check_cache(name, kc, vc, kr, vr, pos0, T, k_new, a):
    """kc, vc: device caches; kr, vr: the oracle's caches (bf16 bits); k_new:
    the call's keys before rotation (bf16 bits)."""
    import oracle

    kg, vg = from_dev(kc), from_dev(vc)
    new = slice(pos0, pos0 + T)
    keep = np.ones(kg.shape[1], bool)
    keep[new] = False
    np.testing.assert_array_equal(vg, vr, err_msg=f"{name}: v cache")
    np.testing.assert_array_equal(kg[:, keep], kr[:, keep], err_msg=f"{name}: untouched k cache")
    got = bf16_bits_to_f32(kg[:, new]).astype(np.float64)
    exact = oracle.rope(oracle._widen(k_new), np.arange(pos0, pos0 + T), a.rot_dim, a.rope_base)
    off = got != bf16_bits_to_f32(kr[:, new])
    # rounding to bf16 (half a step, 2^-8 of the value at most) plus an
    # absolute 2^-16 for keys that cancel to near zero in the rotation
    bound = 2.0 ** -8 * np.abs(exact) + 2.0 ** -16
    print(f"[parity] {name}: rotated keys off the oracle's rounding {off.mean():.2e}, "
          f"max |err|/bound {np.max(np.abs(got - exact) / bound):.3f}", flush=True)
    assert np.all(np.abs(got - exact) <= bound) and off.mean() <= 1e-3


def oracle_call(I, pos0, a):
    import oracle

    return oracle.attn_layer(I["q"], I["k"], I["v"], I["k_cache"], I["v_cache"], pos0,
                             rot_dim=a.rot_dim, base=a.rope_base, scale=a.d_h ** -0.5)


# Calls with fewer than 64 blocks of 128 (token, head) rows split the KV range
# over several blocks and merge the partial results; the others run one pass.
@pytest.mark.parametrize("B,T,H_q,H_kv,d,rot,out_bf16", [
    (4, 300, 24, 2, 256, 64, False),   # one pass: 232 row blocks, the last one ragged
    (2, 700, 6, 2, 128, 32, True),     # one pass at d=128, bf16 output
    (2, 77, 6, 2, 128, 32, False),     # ragged: two query tiles, the second 13 rows
    (1, 200, 24, 2, 256, 64, False),   # the pages' heads and head size, four tiles
    (1, 200, 24, 2, 256, 64, True),    # bf16 output
    (3, 64, 8, 8, 128, 128, False),    # no grouping, full rotary width, one exact tile
    (1, 1, 24, 2, 256, 64, False),     # a single token
    (1, 130, 4, 1, 256, 0, False),     # no rotation, one KV head for all
])
def test_attn_prefill_small(B, T, H_q, H_kv, d, rot, out_bf16):
    a = attn_dims(B, H_q, H_kv, d, rot, 1e7 if d == 256 else 1e4, out_bf16)
    I = make_attn_inputs(B, T, 0, T + 5, H_q, H_kv, d, seed=900 + T + d)
    o, kc, vc = run_gpu(a, I, 0)
    ref, kr, vr = oracle_call(I, 0, a)
    check_out(f"attn B={B} T={T} H={H_q}/{H_kv} d={d} r={rot}", o, ref,
              TOL_BF16 if out_bf16 else TOL_F32)
    check_cache("cache", kc, vc, kr, vr, 0, T, I["k"], a)


def test_attn_sharp_scores():
    # q four times larger: scores of spread ~4, peaked weights, the running
    # maximum of the online softmax moves often across KV tiles.
    a = attn_dims(1, **QWEN)
    I = make_attn_inputs(1, 300, 0, 300, 24, 2, 256, seed=930, q_std=4.0)
    o, kc, vc = run_gpu(a, I, 0)
    ref, kr, vr = oracle_call(I, 0, a)
    check_out("attn sharp q_std=4 T=300", o, ref, TOL_F32)


def test_attn_continuation_through_the_cache():
    # 130 tokens, then 70 more at position 130, then a single token at 200:
    # against one oracle call over all 201 tokens.
    a = attn_dims(2, **QWEN)
    T_max = 256
    I = make_attn_inputs(2, 201, 0, T_max, 24, 2, 256, seed=940)
    ref, kr, vr = oracle_call(I, 0, a)
    kc, vc = to_dev(I["k_cache"]), to_dev(I["v_cache"])
    outs = []
    for s, e in ((0, 130), (130, 200), (200, 201)):
        part = {n: I[n][:, s:e] for n in ("q", "k", "v")}
        o, kc, vc = run_gpu(a, dict(part, k_cache=None), s, kc, vc)
        outs.append(o)
    check_out("attn 130 + 70 + 1 tokens", np.concatenate(outs, 1), ref, TOL_F32)
    check_cache("cache after three calls", kc, vc, kr, vr, 0, 201, I["k"], a)


def test_attn_long_position():
    # Eight new tokens after 100,000 cached ones: RoPE angles of 1e5 radians
    # on the fastest pair, attention over the whole context.
    a = attn_dims(1, **QWEN)
    pos0, T = 100_000, 8
    I = make_attn_inputs(1, T, pos0, pos0 + T, 24, 2, 256, seed=950)
    o, kc, vc = run_gpu(a, I, pos0)
    ref, kr, vr = oracle_call(I, pos0, a)
    check_out(f"attn pos0={pos0} T={T}", o, ref, TOL_F32)
    check_cache("cache", kc, vc, kr, vr, pos0, T, I["k"], a)


def test_attn_qwen_prefill_4096_sampled_rows():
    # The hybrid block's attention layer at 4096 tokens (the pages' shape);
    # the oracle computes 64 sampled query rows of every head over all keys.
    import oracle

    a = attn_dims(1, **QWEN)
    T = 4096
    I = make_attn_inputs(1, T, 0, T, 24, 2, 256, seed=960)
    o, kc, vc = run_gpu(a, I, 0)
    rows = np.sort(np.concatenate([[0, 63, 64, T - 1],
                                   np.random.default_rng(3).choice(np.arange(1, T - 1), 60, replace=False)]))
    rows = np.unique(rows)
    pos = np.arange(T)
    qr = oracle.rope(oracle._widen(I["q"][:, rows]), rows, a.rot_dim, a.rope_base)
    kr = oracle._to_bf16_bits(oracle.rope(oracle._widen(I["k"]), pos, a.rot_dim, a.rope_base))
    ref = oracle.attention(qr, oracle._widen(kr), oracle._widen(I["v"]), rows, pos, a.d_h ** -0.5)
    check_out(f"attn T={T} ({len(rows)} sampled rows)", o[:, rows], ref, TOL_F32)
    check_cache("cache", kc, vc, kr, I["v"], 0, T, I["k"], a)


@pytest.mark.parametrize("B,pos0,T", [(1, 4095, 1), (2, 1000, 40), (3, 2047, 2)])
def test_attn_split_kv_after_long_context(B, pos0, T):
    # Few query rows after a long cached context: the KV range is split over
    # several blocks and merged (decode steps, short chunks).
    a = attn_dims(B, **QWEN)
    I = make_attn_inputs(B, T, pos0, pos0 + T + 3, 24, 2, 256, seed=970 + T)
    o, kc, vc = run_gpu(a, I, pos0)
    ref, kr, vr = oracle_call(I, pos0, a)
    check_out(f"attn split B={B} pos0={pos0} T={T}", o, ref, TOL_F32)
    check_cache("cache", kc, vc, kr, vr, pos0, T, I["k"], a)


# Decode-shaped calls: a few query rows per KV head after a cached context
# (a decode token, a short MTP step), through the split KV pass and the
# combine, or one block when the context is short.
@pytest.mark.parametrize("B,pos0,T,H_q,H_kv,d,rot,out_bf16", [
    (1, 0, 1, 24, 2, 256, 64, False),       # the first token: one position
    (2, 15, 1, 24, 2, 256, 64, False),      # a context of 16 positions
    (3, 4113, 1, 24, 2, 256, 64, False),    # 65 KV tiles, a ragged last one
    (1, 100000, 1, 24, 2, 256, 64, False),  # 1,563 KV tiles over the largest split count
    (2, 37, 8, 8, 8, 128, 128, False),      # G = 1, 8 new tokens, rotation over the whole head
    (1, 60, 4, 4, 1, 256, 0, True),         # no rotation, no split: the smallest workspace
    (1, 62, 4, 4, 1, 256, 64, False),       # new tokens across a KV tile boundary
    (2, 300, 1, 12, 1, 128, 32, True),      # d = 128, one KV head
])
def test_attn_decode_path(B, pos0, T, H_q, H_kv, d, rot, out_bf16):
    a = attn_dims(B, H_q, H_kv, d, rot, 1e7 if d == 256 else 1e4, out_bf16)
    I = make_attn_inputs(B, T, pos0, pos0 + T + 2, H_q, H_kv, d, seed=990 + pos0 % 97 + T)
    o, kc, vc = run_gpu(a, I, pos0)
    ref, kr, vr = oracle_call(I, pos0, a)
    check_out(f"attn decode B={B} pos0={pos0} T={T} H={H_q}/{H_kv} d={d} r={rot}", o, ref,
              TOL_BF16 if out_bf16 else TOL_F32)
    check_cache("cache", kc, vc, kr, vr, pos0, T, I["k"], a)


@pytest.mark.parametrize("B,pos0,H_q,H_kv,d,rot", [
    (2, 4113, 24, 2, 256, 64),
    (1, 300, 12, 1, 128, 32),
    (1, 70, 4, 1, 256, 0),
])
def test_attn_single_token_cache_rows_match(B, pos0, H_q, H_kv, d, rot):
    # A one-token call writes its cache row inside the attention pass; a
    # two-token call writes its rows with the separate cache kernel.  Two
    # one-token calls at positions pos0 - 1 and pos0 must leave the cache
    # bit-identical to one two-token call over the same keys and values.
    import gated_deltanet_layer_gdn_amd as gdn
    import torch

    a = attn_dims(B, H_q, H_kv, d, rot, 1e7 if d == 256 else 1e4)
    I = make_attn_inputs(B, 2, pos0 - 1, pos0 + 3, H_q, H_kv, d, seed=1200 + pos0)
    q, k, v = to_dev(I["q"]), to_dev(I["k"]), to_dev(I["v"])
    kc2, vc2 = to_dev(I["k_cache"]), to_dev(I["v_cache"])
    gdn.attn_prefill(a, q, k, v, kc2, vc2, pos0=pos0 - 1)
    kc1, vc1 = to_dev(I["k_cache"]), to_dev(I["v_cache"])
    for t in range(2):
        gdn.attn_prefill(a, q[:, t:t + 1].contiguous(), k[:, t:t + 1].contiguous(),
                         v[:, t:t + 1].contiguous(), kc1, vc1, pos0=pos0 - 1 + t)
    torch.cuda.synchronize()
    print(f"[attn] single-token cache rows B={B} pos0={pos0} d={d} rot={rot}", flush=True)
    np.testing.assert_array_equal(from_dev(kc1), from_dev(kc2))
    np.testing.assert_array_equal(from_dev(vc1), from_dev(vc2))
