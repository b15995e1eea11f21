"""CPU pins of the oracle's RoPE and causal GQA attention ("Implement the
Qwen3.8 Flash Next Rust and Metal text core", section Implementation: Qwen
RoPE and exact dense 24Q/2KV causal attention)."""
from __future__ import annotations

import numpy as np

import oracle


def test_rope_closed_forms():
    rng = np.random.default_rng(0)
    u = rng.standard_normal((1, 7, 3, 16))
    # position 0 and a zero rotary width are the identity
    np.testing.assert_array_equal(oracle.rope(u[:, :1], [0], 16, 1e4), u[:, :1])
    np.testing.assert_array_equal(oracle.rope(u, np.arange(7), 0, 1e4), u)
    # the first pair turns by exactly pos radians (frequency base^0 = 1)
    e = np.zeros((1, 1, 1, 4))
    e[..., 0] = 1.0
    r = oracle.rope(e, [1], 4, 1e4)
    np.testing.assert_allclose(r[0, 0, 0], [np.cos(1.0), 0.0, np.sin(1.0), 0.0], atol=1e-16)
    # dimensions past the rotary width are untouched; pair norms are kept
    r = oracle.rope(u, np.arange(100, 107), 8, 1e4)
    np.testing.assert_array_equal(r[..., 8:], u[..., 8:])
    n0 = u[..., :4] ** 2 + u[..., 4:8] ** 2
    n1 = r[..., :4] ** 2 + r[..., 4:8] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-13)
    # relative positions: <R(p) q, R(p') k> depends only on p - p'
    q, k = u[:, :1, :1], u[:, 1:2, :1]
    d1 = np.sum(oracle.rope(q, [5], 16, 1e4) * oracle.rope(k, [2], 16, 1e4))
    d2 = np.sum(oracle.rope(q, [1005], 16, 1e4) * oracle.rope(k, [1002], 16, 1e4))
    np.testing.assert_allclose(d1, d2, rtol=1e-10)


def test_attention_special_cases():
    rng = np.random.default_rng(1)
    B, T, H_q, H_kv, d = 2, 9, 6, 2, 8
    q = rng.standard_normal((B, T, H_q, d))
    k = rng.standard_normal((B, T, H_kv, d))
    v = rng.standard_normal((B, T, H_kv, d))
    pos = np.arange(T)
    o = oracle.attention(q, k, v, pos, pos, 0.3)
    # the first token sees only itself: its output is its value
    np.testing.assert_allclose(o[:, 0, :3], np.repeat(v[:, 0, :1], 3, axis=1), rtol=1e-14)
    # equal keys: uniform weights, the running mean of the values
    ke = np.ones_like(k)
    oe = oracle.attention(q, ke, v, pos, pos, 0.3)
    mean = np.cumsum(v, axis=1) / np.arange(1, T + 1)[None, :, None, None]
    np.testing.assert_allclose(oe[:, :, 3:], np.repeat(mean[:, :, 1:], 3, axis=2), rtol=1e-13)
    # causal: a change at token 6 leaves tokens 0..5 unchanged
    k2 = k.copy()
    k2[:, 6] += 5
    o2 = oracle.attention(q, k2, v, pos, pos, 0.3)
    np.testing.assert_array_equal(o2[:, :6], o[:, :6])
    assert np.abs(o2[:, 6:] - o[:, 6:]).max() > 1e-3
    # query heads 0..2 read kv head 0, 3..5 kv head 1
    v3 = v.copy()
    v3[:, :, 1] += 1
    o3 = oracle.attention(q, k, v3, pos, pos, 0.3)
    np.testing.assert_array_equal(o3[:, :, :3], o[:, :, :3])
    np.testing.assert_allclose(o3[:, :, 3:], o[:, :, 3:] + 1, rtol=1e-13)


def test_attn_layer_chunked_equals_whole():
    # Prefill in two calls through the cache equals one call (fp64 apart from
    # the cache's bf16 rounding, which is the same either way).
    rng = np.random.default_rng(2)
    B, T, H_q, H_kv, d, Tm = 1, 12, 4, 2, 16, 16
    f = lambda *s: oracle._to_bf16_bits(rng.standard_normal(s))
    q, k, v = f(B, T, H_q, d), f(B, T, H_kv, d), f(B, T, H_kv, d)
    kc = np.zeros((B, Tm, H_kv, d), np.uint16)
    vc = np.zeros_like(kc)
    kw = dict(rot_dim=8, base=1e4, scale=0.25)
    o, kc1, vc1 = oracle.attn_layer(q, k, v, kc, vc, 0, **kw)
    oa, kc2, vc2 = oracle.attn_layer(q[:, :5], k[:, :5], v[:, :5], kc, vc, 0, **kw)
    ob, kc2, vc2 = oracle.attn_layer(q[:, 5:], k[:, 5:], v[:, 5:], kc2, vc2, 5, **kw)
    np.testing.assert_allclose(np.concatenate([oa, ob], 1), o, rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(kc2, kc1)
    np.testing.assert_array_equal(vc2, vc1)
