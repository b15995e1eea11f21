"""Pins of the fp64 oracle to facts it does not compute itself.

Each test holds the oracle against a library routine, a closed form, an
invariant of the gated delta rule, a brute-force dense product or the
independent chunked restatement in ``chunked_mirror``.  None of the pages
prints a worked example, so no expected value here comes from them.
"""
from __future__ import annotations

import numpy as np
import pytest
import scipy.special

from chunked_mirror import chunked_recurrence
from gdn_inputs import Geometry, bf16_bits_to_f32, f64_to_bf16_bits, make_inputs

RNG = np.random.default_rng(12345)


def unit_rows(a):
    return a / np.linalg.norm(a, axis=-1, keepdims=True)


def rand_problem(rng, B=1, T=12, H_k=1, H_v=1, d_k=6, d_v=5, unit=True, decay=1.0):
    q = rng.standard_normal((B, T, H_k, d_k))
    k = rng.standard_normal((B, T, H_k, d_k))
    if unit:
        q, k = unit_rows(q), unit_rows(k)
    v = rng.standard_normal((B, T, H_v, d_v))
    g = -decay * np.logaddexp(0, rng.standard_normal((B, T, H_v)))
    beta = scipy.special.expit(rng.standard_normal((B, T, H_v)))
    z = rng.standard_normal((B, T, H_v, d_v))
    S0 = 0.3 * rng.standard_normal((B, H_v, d_v, d_k))
    return q, k, v, g, beta, z, S0


# --------------------------------------------------------------------------- conv (a1)

def np_causal_conv(x, w, hist):
    """Causal depthwise conv via numpy.convolve on concat(history, x)."""
    B, T, C = x.shape
    W = w.shape[1]
    full = np.concatenate([hist, x], axis=1)
    out = np.empty((B, T, C))
    for b in range(B):
        for c in range(C):
            # convolve flips its kernel: reverse the taps so tap W-1 meets token t
            out[b, :, c] = np.convolve(full[b, :, c], w[c, ::-1], mode="valid")
    return out


@pytest.mark.parametrize("T", [1, 2, 3, 7, 33])
def test_conv_silu_matches_numpy_convolve(oracle_mod, T):
    rng = np.random.default_rng(T)
    B, C, W = 2, 5, 4
    x = rng.standard_normal((B, T, C)).astype(np.float32)
    w = rng.standard_normal((C, W)).astype(np.float32)
    hist = rng.standard_normal((B, W - 1, C)).astype(np.float32)
    got = oracle_mod.conv_silu(x, w, hist)
    xi = np_causal_conv(x.astype(np.float64), w.astype(np.float64), hist.astype(np.float64))
    np.testing.assert_allclose(got, xi * scipy.special.expit(xi), rtol=1e-13, atol=1e-14)


def test_conv_bf16_inputs_widen_exactly(oracle_mod):
    rng = np.random.default_rng(7)
    x64 = rng.standard_normal((1, 9, 4))
    w64 = rng.standard_normal((4, 4))
    h64 = rng.standard_normal((1, 3, 4))
    xb, wb, hb = (f64_to_bf16_bits(a) for a in (x64, w64, h64))
    got = oracle_mod.conv_silu(xb, wb, hb)
    xi = np_causal_conv(*(bf16_bits_to_f32(a).astype(np.float64) for a in (xb, wb, hb)))
    np.testing.assert_allclose(got, xi * scipy.special.expit(xi), rtol=1e-13, atol=1e-14)


def test_conv_identity_and_shift_taps(oracle_mod):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, 6, 3)).astype(np.float32)
    hist = rng.standard_normal((1, 3, 3)).astype(np.float32)
    w = np.zeros((3, 4), np.float32)
    w[:, 3] = 1.0  # current token only
    np.testing.assert_allclose(oracle_mod.conv_silu(x, w, hist),
                               scipy.special.expit(x.astype(np.float64)) * x, rtol=1e-15)
    w[:] = 0
    w[:, 0] = 1.0  # token t-3: history for t < 3
    got = oracle_mod.conv_silu(x, w, hist)
    src = np.concatenate([hist, x], axis=1)[:, :6].astype(np.float64)
    np.testing.assert_allclose(got, scipy.special.expit(src) * src, rtol=1e-15)
    # SiLU(0) = 0 exactly
    assert np.all(oracle_mod.conv_silu(np.zeros_like(x), w, np.zeros_like(hist)) == 0)


@pytest.mark.parametrize("T", [1, 2, 3, 4, 10])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_conv_history_next_is_last_rows(oracle_mod, T, dt):
    rng = np.random.default_rng(T)
    x64 = rng.standard_normal((2, T, 6))
    h64 = rng.standard_normal((2, 3, 6))
    cast = (lambda a: a.astype(np.float32)) if dt == "f32" else f64_to_bf16_bits
    x, hist = cast(x64), cast(h64)
    got = oracle_mod.conv_history_next(x, hist)
    want = np.concatenate([hist, x], axis=1)[:, -3:]
    assert got.dtype == x.dtype
    np.testing.assert_array_equal(got.view(np.uint8), np.ascontiguousarray(want).view(np.uint8))


# --------------------------------------------------------------------------- norm (a2)

def test_l2norm_matches_linalg_norm(oracle_mod):
    a = RNG.standard_normal((17, 128))
    got = oracle_mod.l2norm(a, eps=0.0)
    np.testing.assert_allclose(got, a / np.linalg.norm(a, axis=-1, keepdims=True), rtol=1e-14)
    np.testing.assert_allclose(np.linalg.norm(got, axis=-1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(oracle_mod.l2norm(a, eps=0.0, scale=0.25), 0.25 * got, rtol=1e-15)


def test_l2norm_epsilon_inside_root(oracle_mod):
    # For x = sqrt(eps) e_1 the epsilon-inside-the-root form gives exactly 1/sqrt(2);
    # eps added to the norm instead would give ~1, eps ignored would give 1.
    eps = 1e-6
    a = np.zeros((1, 8))
    a[0, 0] = np.sqrt(eps)
    np.testing.assert_allclose(oracle_mod.l2norm(a, eps=eps)[0, 0], 1 / np.sqrt(2), rtol=1e-14)
    # zero vector -> zero, no NaN
    assert np.all(oracle_mod.l2norm(np.zeros((2, 8)), eps=eps) == 0)


# --------------------------------------------------------------------------- recurrence (a3..a7)

def test_beta0_decay1_keeps_state_bitwise(oracle_mod):
    q, k, v, g, beta, z, S0 = rand_problem(np.random.default_rng(1))
    g[:] = 0.0
    beta[:] = 0.0
    y, S, o = oracle_mod.recurrence(q, k, v, g, beta, z, S0)
    np.testing.assert_array_equal(S, S0)
    np.testing.assert_allclose(o[0, :, 0], (S0[0, 0] @ q[0, :, 0].T).T, rtol=1e-13)


def test_gate_sigmoid_special_values(oracle_mod):
    q, k, v, g, beta, z, S0 = rand_problem(np.random.default_rng(2))
    z[:] = 0.0
    y, S, o = oracle_mod.recurrence(q, k, v, g, beta, z, S0)
    np.testing.assert_array_equal(y, o * 0.5)
    z[:] = 60.0
    y, _, o = oracle_mod.recurrence(q, k, v, g, beta, z, S0)
    np.testing.assert_allclose(y, o, rtol=1e-15)
    z2 = np.random.default_rng(5).standard_normal(z.shape)
    y, _, o = oracle_mod.recurrence(q, k, v, g, beta, z2, S0)
    np.testing.assert_allclose(y, o * scipy.special.expit(z2), rtol=1e-14)


def test_one_hot_keys_overwrite_exactly(oracle_mod):
    # beta = 1, a = 1, key e_j: column j of S becomes v exactly, other columns stay.
    d_k, d_v = 4, 3
    rng = np.random.default_rng(4)
    S0 = rng.standard_normal((1, 1, d_v, d_k))
    order = [2, 0, 3, 1]
    k = np.zeros((1, 4, 1, d_k))
    for t, j in enumerate(order):
        k[0, t, 0, j] = 1.0
    q = k.copy()
    v = rng.standard_normal((1, 4, 1, d_v))
    g = np.zeros((1, 4, 1))
    beta = np.ones((1, 4, 1))
    z = np.zeros((1, 4, 1, d_v))
    y, S, o = oracle_mod.recurrence(q, k, v, g, beta, z, S0)
    want = np.empty((d_v, d_k))
    for t, j in enumerate(order):
        want[:, j] = v[0, t, 0]
    np.testing.assert_array_equal(S[0, 0], want)
    # reading with the key just written returns its value
    np.testing.assert_array_equal(o[0, :, 0], v[0, :, 0])


def test_orthonormal_keys_overwrite(oracle_mod):
    d = 8
    rng = np.random.default_rng(6)
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    k = Qm.T.reshape(1, d, 1, d)  # d orthonormal keys
    v = rng.standard_normal((1, d, 1, 5))
    S0 = rng.standard_normal((1, 1, 5, d))
    y, S, o = oracle_mod.recurrence(k, k, v, np.zeros((1, d, 1)), np.ones((1, d, 1)),
                                    np.zeros((1, d, 1, 5)), S0)
    np.testing.assert_allclose(S[0, 0], v[0, :, 0].T @ k[0, :, 0], atol=1e-13)


def test_retrieval_identity_per_step(oracle_mod):
    # S_t k_t = a (1 - beta |k|^2) S_{t-1} k_t + beta |k|^2 v_t, for any k (not only unit)
    rng = np.random.default_rng(8)
    q, k, v, g, beta, z, S0 = rand_problem(rng, T=1, unit=False, d_k=7, d_v=4)
    _, S1, _ = oracle_mod.recurrence(q, k, v, g, beta, z, S0)
    kk = k[0, 0, 0]
    a, b = np.exp(g[0, 0, 0]), beta[0, 0, 0]
    n2 = kk @ kk
    want = a * (1 - b * n2) * (S0[0, 0] @ kk) + b * n2 * v[0, 0, 0]
    np.testing.assert_allclose(S1[0, 0] @ kk, want, rtol=1e-13, atol=1e-13)


def test_full_decay_forgets_state(oracle_mod):
    rng = np.random.default_rng(9)
    q, k, v, g, beta, z, S0 = rand_problem(rng, T=1)
    g[:] = -80.0  # a = exp(-80) ~ 1.8e-35
    _, S1, _ = oracle_mod.recurrence(q, k, v, g, beta, z, S0)
    want = beta[0, 0, 0] * np.outer(v[0, 0, 0], k[0, 0, 0])
    np.testing.assert_allclose(S1[0, 0], want, rtol=1e-12, atol=1e-30)


def test_frobenius_contraction_bound(oracle_mod):
    rng = np.random.default_rng(10)
    q, k, v, g, beta, z, S0 = rand_problem(rng, T=30)
    S = S0
    for t in range(30):
        sl = slice(t, t + 1)
        _, S_next, _ = oracle_mod.recurrence(q[:, sl], k[:, sl], v[:, sl], g[:, sl], beta[:, sl],
                                             z[:, sl], S)
        bound = (np.exp(g[0, t, 0]) * np.linalg.norm(S[0, 0])
                 + beta[0, t, 0] * np.linalg.norm(v[0, t, 0]) * np.linalg.norm(k[0, t, 0]))
        assert np.linalg.norm(S_next[0, 0]) <= bound * (1 + 1e-12)
        S = S_next


def brute_force_products(q, k, v, g, beta, S0):
    """S_t = S0 A_1...A_t + sum_s beta_s v_s k_s^T A_{s+1}...A_t with
    A_t = a_t (I - beta_t k_t k_t^T), as explicit dense matrix products."""
    T, d_k = k.shape
    A = [np.exp(g[t]) * (np.eye(d_k) - beta[t] * np.outer(k[t], k[t])) for t in range(T)]
    outs, states = [], []
    for t in range(T):
        P = np.eye(d_k)
        for r in range(t + 1):
            P = P @ A[r]
        St = S0 @ P
        for s in range(t + 1):
            Ps = np.eye(d_k)
            for r in range(s + 1, t + 1):
                Ps = Ps @ A[r]
            St = St + beta[s] * np.outer(v[s], k[s]) @ Ps
        states.append(St)
        outs.append(St @ q[t])
    return np.array(outs), states[-1]


def test_brute_force_dense_products(oracle_mod):
    rng = np.random.default_rng(11)
    T = 24
    q, k, v, g, beta, z, S0 = rand_problem(rng, T=T, d_k=16, d_v=16)
    y, S, o = oracle_mod.recurrence(q, k, v, g, beta, z, S0)
    o_bf, S_bf = brute_force_products(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0],
                                      beta[0, :, 0], S0[0, 0])
    np.testing.assert_allclose(o[0, :, 0], o_bf, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(S[0, 0], S_bf, rtol=1e-11, atol=1e-13)


def test_grouped_value_heads_read_their_key_head(oracle_mod):
    # value head h must read key head h // (H_v/H_k): perturbing key head 1 leaves
    # value heads 0..2 bit-identical and changes heads 3..5.
    rng = np.random.default_rng(12)
    q, k, v, g, beta, z, S0 = rand_problem(rng, T=5, H_k=2, H_v=6, d_k=4, d_v=3)
    y0, S0o, _ = oracle_mod.recurrence(q, k, v, g, beta, z, S0)
    k2, q2 = k.copy(), q.copy()
    k2[:, :, 1] = unit_rows(rng.standard_normal(k2[:, :, 1].shape))
    q2[:, :, 1] = unit_rows(rng.standard_normal(q2[:, :, 1].shape))
    y1, S1o, _ = oracle_mod.recurrence(q2, k2, v, g, beta, z, S0)
    np.testing.assert_array_equal(y0[:, :, :3], y1[:, :, :3])
    np.testing.assert_array_equal(S0o[:, :3], S1o[:, :3])
    assert np.all(np.abs(y0[:, :, 3:] - y1[:, :, 3:]).max(axis=(0, 1, 3)) > 0)


@pytest.mark.parametrize("C", [1, 4, 16, 64, 100])
@pytest.mark.parametrize("decay", [1.0, 0.01])
def test_chunked_form_equals_sequential(oracle_mod, C, decay):
    rng = np.random.default_rng(C)
    q, k, v, g, beta, z, S0 = rand_problem(rng, B=2, T=150, H_k=2, H_v=4, d_k=16, d_v=8,
                                           decay=decay)
    y, S, o = oracle_mod.recurrence(q, k, v, g, beta, z, S0)
    yc, Sc, oc = chunked_recurrence(q, k, v, g, beta, z, S0, C)
    scale = np.abs(o).max()
    np.testing.assert_allclose(oc, o, atol=1e-12 * scale, rtol=0)
    np.testing.assert_allclose(Sc, S, atol=1e-12 * np.abs(S).max(), rtol=0)


# --------------------------------------------------------------------------- whole layer

def _small_layer_inputs(dtype="f32", T=40, seed=0, zero_state=False):
    geom = Geometry(B=2, T=T, H_k=2, H_v=4, d_k=16, d_v=8, dtype=dtype, zero_state=zero_state)
    return geom, make_inputs(geom, seed)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_layer_equals_composed_stages(oracle_mod, dtype):
    geom, I = _small_layer_inputs(dtype)
    kw = dict(H_k=geom.H_k, H_v=geom.H_v, d_k=geom.d_k, d_v=geom.d_v)
    eps, qs = 1e-6, 0.7
    y, S, hist_next = oracle_mod.layer(I["x"], I["z"], I["g"], I["beta"], I["w"], I["hist"],
                                       I["S"], eps=eps, q_scale=qs, **kw)
    u = oracle_mod.conv_silu(I["x"], I["w"], I["hist"])
    B, T = geom.B, geom.T
    nq = geom.H_k * geom.d_k
    q = oracle_mod.l2norm(u[..., :nq].reshape(B, T, geom.H_k, geom.d_k), eps, qs)
    k = oracle_mod.l2norm(u[..., nq:2 * nq].reshape(B, T, geom.H_k, geom.d_k), eps)
    v = u[..., 2 * nq:].reshape(B, T, geom.H_v, geom.d_v)
    zz = I["z"].astype(np.float64) if dtype == "f32" else bf16_bits_to_f32(I["z"]).astype(np.float64)
    y2, S2, _ = oracle_mod.recurrence(q, k, v, I["g"].astype(np.float64),
                                      I["beta"].astype(np.float64), zz, I["S"])
    np.testing.assert_array_equal(y, y2)
    np.testing.assert_array_equal(S, S2)
    np.testing.assert_array_equal(hist_next, np.concatenate([I["hist"], I["x"]], axis=1)[:, -3:])


@pytest.mark.parametrize("split", [1, 3, 17, 39])
def test_layer_split_resume_bitwise(oracle_mod, split):
    geom, I = _small_layer_inputs("bf16", T=40, seed=1)
    kw = dict(H_k=geom.H_k, H_v=geom.H_v, d_k=geom.d_k, d_v=geom.d_v, eps=1e-6)
    y, S, h = oracle_mod.layer(I["x"], I["z"], I["g"], I["beta"], I["w"], I["hist"], I["S"], **kw)
    a = slice(0, split)
    b = slice(split, geom.T)
    ya, Sa, ha = oracle_mod.layer(I["x"][:, a], I["z"][:, a], I["g"][:, a], I["beta"][:, a],
                                  I["w"], I["hist"], I["S"], **kw)
    yb, Sb, hb = oracle_mod.layer(I["x"][:, b], I["z"][:, b], I["g"][:, b], I["beta"][:, b],
                                  I["w"], ha, Sa, **kw)
    np.testing.assert_array_equal(np.concatenate([ya, yb], axis=1), y)
    np.testing.assert_array_equal(Sb, S)
    np.testing.assert_array_equal(hb, h)


def test_layer_head_subset_matches_full(oracle_mod):
    geom, I = _small_layer_inputs("bf16", T=20, seed=2)
    kw = dict(H_k=geom.H_k, H_v=geom.H_v, d_k=geom.d_k, d_v=geom.d_v, eps=1e-6)
    y, S, _ = oracle_mod.layer(I["x"], I["z"], I["g"], I["beta"], I["w"], I["hist"], I["S"], **kw)
    heads = [(1, 3), (0, 1)]
    ys, Ss, _ = oracle_mod.layer(I["x"], I["z"], I["g"], I["beta"], I["w"], I["hist"], I["S"],
                                 heads=heads, nthreads=2, **kw)
    for b, h in heads:
        np.testing.assert_array_equal(ys[b, :, h], y[b, :, h])
        np.testing.assert_array_equal(Ss[b, h], S[b, h])
    np.testing.assert_array_equal(Ss[0, 0], I["S"][0, 0].astype(np.float64))
    assert np.isnan(ys[0, :, 0]).all()


def test_layer_padding_tokens_are_noops(oracle_mod):
    # Tokens with g = 0 and beta = 0 leave the recurrent state bit-identical.
    geom, I = _small_layer_inputs("f32", T=12, seed=3)
    kw = dict(H_k=geom.H_k, H_v=geom.H_v, d_k=geom.d_k, d_v=geom.d_v, eps=1e-6)
    _, S, _ = oracle_mod.layer(I["x"], I["z"], I["g"], I["beta"], I["w"], I["hist"], I["S"], **kw)
    I2 = {k_: np.concatenate([a, a[:, :5]], axis=1) if k_ in ("x", "z", "g", "beta") else a
          for k_, a in I.items()}
    I2["g"][:, 12:] = 0
    I2["beta"][:, 12:] = 0
    _, S2, _ = oracle_mod.layer(I2["x"], I2["z"], I2["g"], I2["beta"], I2["w"], I2["hist"],
                                I2["S"], **kw)
    np.testing.assert_array_equal(S2, S)


def test_golden_tiny_layer_fixture(oracle_mod):
    """The oracle still reproduces tests/golden/tiny_layer_oracle.txt (written by
    tests/golden/make_golden.py, which calls only the oracle)."""
    import importlib.util
    import os

    here = os.path.dirname(os.path.abspath(__file__))
    spec = importlib.util.spec_from_file_location("make_golden",
                                                  os.path.join(here, "golden", "make_golden.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    now = mod.compute()
    with open(os.path.join(here, "golden", "tiny_layer_oracle.txt")) as f:
        stored = {ln.split()[0]: np.array([float(a) for a in ln.split()[1:]])
                  for ln in f if not ln.startswith("#")}
    assert stored.keys() == now.keys()
    for k_, v_ in stored.items():
        np.testing.assert_allclose(now[k_], v_, rtol=1e-12, atol=1e-15, err_msg=k_)
