"""CPU pins of the oracle's output epilogue pieces: the ungated readout
(layer with z=None) and the zero-centred grouped RMS norm before the sigmoid
gate ("Implement the Qwen3.8 Flash Next Rust and Metal text core", section
Implementation: zero-centred norms; its implementation comment: zero-centred
grouped RMS, sigmoid output gate)."""
from __future__ import annotations

import numpy as np

import oracle
from gdn_inputs import Geometry, make_inputs

KW = dict(H_k=2, H_v=4, d_k=16, d_v=16, eps=1e-6)


def test_ungated_layer_equals_recurrence_readout():
    # The layer's ungated readout against the other oracle path: conv + SiLU,
    # the L2 norm and the token recurrence run as separate stages (whose o is
    # the ungated readout), all in fp64.
    g = Geometry(B=2, T=33, H_k=2, H_v=4, d_k=16, d_v=16, dtype="f32", zero_state=False)
    I = make_inputs(g, 5)
    y, S, _ = oracle.layer(I["x"], None, I["g"], I["beta"], I["w"], I["hist"], I["S"], **KW)
    u = oracle.conv_silu(I["x"], I["w"], I["hist"])
    nq = g.H_k * g.d_k
    q = oracle.l2norm(u[..., :nq].reshape(2, 33, 2, 16), 1e-6)
    k = oracle.l2norm(u[..., nq:2 * nq].reshape(2, 33, 2, 16), 1e-6)
    v = u[..., 2 * nq:].reshape(2, 33, 4, 16)
    _, S2, o = oracle.recurrence(q, k, v, I["g"], I["beta"], np.zeros_like(v), I["S"])
    np.testing.assert_allclose(y, o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S, S2, rtol=1e-12, atol=1e-14)
    # and the gated layer is the ungated readout times sigmoid(z), element by element
    yg, _, _ = oracle.layer(I["x"], I["z"], I["g"], I["beta"], I["w"], I["hist"], I["S"], **KW)
    np.testing.assert_allclose(yg, y / (1 + np.exp(-I["z"].astype(np.float64))), rtol=1e-13)


def test_rmsnorm_worked_example():
    # o = (3, 4): mean square 12.5, so o / sqrt(12.5) = (0.8485..., 1.1313...);
    # sigmoid(0) = 1/2 halves it; w = (1, -1) doubles the first and zeroes the second.
    o = np.array([[3.0, 4.0]])
    r = 1 / np.sqrt(12.5)
    np.testing.assert_allclose(oracle.gated_rmsnorm(o, None, None, 0.0), [[3 * r, 4 * r]], rtol=1e-15)
    np.testing.assert_allclose(oracle.gated_rmsnorm(o, np.zeros_like(o), None, 0.0),
                               [[1.5 * r, 2 * r]], rtol=1e-15)
    np.testing.assert_allclose(oracle.gated_rmsnorm(o, None, np.array([1.0, -1.0]), 0.0),
                               [[6 * r, 0.0]], rtol=1e-15)


def test_rmsnorm_closed_forms():
    rng = np.random.default_rng(0)
    o = rng.standard_normal((50, 3, 32))
    eps = 1e-3
    y = oracle.gated_rmsnorm(o, None, None, eps)
    # unit weight, no gate: each group's mean square is ms / (ms + eps)
    ms = (o ** 2).mean(-1)
    np.testing.assert_allclose((y ** 2).mean(-1), ms / (ms + eps), rtol=1e-12)
    # a constant group c gives c / sqrt(c^2 + eps) everywhere
    c = np.full((1, 32), -0.25)
    np.testing.assert_allclose(oracle.gated_rmsnorm(c, None, None, eps), -0.25 / np.sqrt(0.0625 + eps),
                               rtol=1e-14)
    # without eps the result does not depend on the group's scale
    np.testing.assert_allclose(oracle.gated_rmsnorm(7.5 * o, None, None, 0.0),
                               oracle.gated_rmsnorm(o, None, None, 0.0), rtol=1e-13)
    # zero-centred weight: w = -1 silences a channel, w = c scales by 1 + c
    w = np.zeros(32)
    w[5] = -1.0
    w[6] = 0.5
    yw = oracle.gated_rmsnorm(o, None, w, eps)
    assert not np.any(yw[..., 5])
    np.testing.assert_allclose(yw[..., 6], 1.5 * y[..., 6], rtol=1e-14)
    # groups are independent: changing one group leaves every other one
    o2 = o.copy()
    o2[7, 1] *= -3
    y2 = oracle.gated_rmsnorm(o2, None, None, eps)
    mask = np.ones((50, 3), bool)
    mask[7, 1] = False
    np.testing.assert_array_equal(y2[mask], y[mask])
    # a very negative gate closes the output, a very positive one leaves it
    z = np.full_like(o, -800.0)
    assert not np.any(oracle.gated_rmsnorm(o, z, None, eps))
    np.testing.assert_allclose(oracle.gated_rmsnorm(o, -z, None, eps), y, rtol=1e-15)
