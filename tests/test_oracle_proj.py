"""CPU pins of the oracle's input projections and decay/beta
parametrisation ("Implement the Qwen3.8 Flash Next Rust and Metal text core",
section Verification: GDN projection)."""
from __future__ import annotations

import numpy as np

import oracle
from gdn_inputs import make_proj_inputs


def test_decay_beta_closed_forms():
    A_log = np.log(np.array([1.0, 4.0, 16.0]))
    dt = np.array([0.0, 0.5, -0.25])
    # a + dt_bias = 0: softplus(0) = ln 2, so g = -A ln 2; b = 0: beta = 1/2
    g, beta = oracle.decay_beta(-dt[None], np.zeros((1, 3)), A_log, dt)
    np.testing.assert_allclose(g[0], -np.array([1.0, 4.0, 16.0]) * np.log(2.0), rtol=1e-15)
    np.testing.assert_array_equal(beta, 0.5)
    # far positive: softplus(u) = u (to double precision); far negative: g -> 0-, decay -> 1
    g, _ = oracle.decay_beta(np.array([[80.0, -80.0, 40.0]]), np.zeros((1, 3)), A_log, dt)
    np.testing.assert_allclose(g[0, 0], -1.0 * 80.0, rtol=1e-14)
    assert -1e-30 < g[0, 1] < 0
    np.testing.assert_allclose(g[0, 2], -16.0 * 39.75, rtol=1e-14)
    # beta is the logistic function: beta(b) + beta(-b) = 1
    b = np.linspace(-7, 7, 29)[None]
    _, b1 = oracle.decay_beta(np.zeros_like(b), b, np.zeros(29), np.zeros(29))
    _, b2 = oracle.decay_beta(np.zeros_like(b), -b, np.zeros(29), np.zeros(29))
    np.testing.assert_allclose(b1 + b2, 1.0, rtol=1e-15)


def test_projection_against_brute_force_and_row_order():
    H_k, H_v, d, hidden = 1, 2, 16, 64
    I = make_proj_inputs(1, 5, hidden, H_k, H_v, d, seed=3)
    C_ch, Z = 2 * H_k * d + H_v * d, H_v * d
    x, z, g, beta = oracle.in_proj(I["h"], I["w_in"], I["A_log"], I["dt_bias"], C_ch=C_ch, Z=Z,
                                   H_v=H_v)
    # brute force: every output an explicit sum over the hidden dimension
    H = oracle._widen(I["h"])[0]
    W = oracle._widen(I["w_in"])
    Y = np.array([[sum(H[t, k] * W[n, k] for k in range(hidden)) for n in range(W.shape[0])]
                  for t in range(5)])
    np.testing.assert_allclose(x[0], Y[:, :C_ch], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(z[0], Y[:, C_ch:C_ch + Z], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(beta[0], 1 / (1 + np.exp(-Y[:, C_ch + Z:C_ch + Z + H_v])), rtol=1e-12)
    # one-hot weight rows route hidden unit k to exactly the output the row names
    w = np.zeros((C_ch + Z + 2 * H_v, hidden), np.float32)
    w[3, 7] = 1.0            # x channel 3 (a q channel)
    w[C_ch + 5, 9] = 1.0     # z channel 5
    w[C_ch + Z + 1, 11] = 1.0  # b of value head 1
    w[C_ch + Z + H_v + 0, 13] = 1.0  # a of value head 0
    hf = oracle._widen(I["h"]).astype(np.float32)
    x, z, g, beta = oracle.in_proj(hf, w, np.zeros(H_v, np.float32), np.zeros(H_v, np.float32),
                                   C_ch=C_ch, Z=Z, H_v=H_v)
    np.testing.assert_array_equal(x[..., 3], hf[..., 7])
    np.testing.assert_array_equal(z[..., 5], hf[..., 9])
    np.testing.assert_allclose(beta[..., 1], 1 / (1 + np.exp(-hf[..., 11].astype(np.float64))))
    np.testing.assert_allclose(g[..., 0], -np.logaddexp(0, hf[..., 13].astype(np.float64)))
    assert not np.any(x[..., :3]) and not np.any(x[..., 4:])
