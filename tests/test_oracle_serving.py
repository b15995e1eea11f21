"""CPU pins of the oracle's serving-shaped compositions (packed varlen prefill
and slot-indexed multi-token decode): their bookkeeping checked against the
batched oracle path, which runs a separate code path inside the C oracle (one
task per (sequence, value head) over a [B, T] batch)."""
from __future__ import annotations

import numpy as np

import oracle
from gdn_inputs import Geometry, make_inputs

KW = dict(H_k=2, H_v=4, d_k=16, d_v=16, eps=1e-6)


def geom(B, T, seed):
    g = Geometry(B=B, T=T, H_k=2, H_v=4, d_k=16, d_v=16, dtype="f32", zero_state=False)
    return make_inputs(g, seed)


def test_varlen_of_equal_lengths_equals_batched_layer():
    I = geom(3, 20, 1)
    y_b, S_b, h_b = oracle.layer(I["x"], I["z"], I["g"], I["beta"], I["w"], I["hist"], I["S"], **KW)
    cu = np.array([0, 20, 40, 60])
    flat = {k: I[k].reshape((60,) + I[k].shape[2:]) for k in ("x", "z", "g", "beta")}
    # pool with the three states in reversed slots and one spare slot
    slots = [2, 1, 0]
    hp = np.zeros((4,) + I["hist"].shape[1:], I["hist"].dtype)
    Sp = np.full((4,) + I["S"].shape[1:], 7.0, np.float32)
    for n, s in enumerate(slots):
        hp[s], Sp[s] = I["hist"][n], I["S"][n]
    y, S, h = oracle.layer_varlen(flat["x"], flat["z"], flat["g"], flat["beta"], I["w"], hp, Sp,
                                  cu, slots, **KW)
    np.testing.assert_array_equal(y.reshape(y_b.shape), y_b)
    for n, s in enumerate(slots):
        np.testing.assert_array_equal(S[s], S_b[n])
        np.testing.assert_array_equal(h[s], h_b[n])
    np.testing.assert_array_equal(S[3], Sp[3])  # the spare slot is untouched


def test_varlen_empty_sequence_leaves_its_slot():
    I = geom(1, 9, 2)
    hp = np.stack([I["hist"][0], I["hist"][0] * 2])
    Sp = np.stack([I["S"][0], I["S"][0] * 3])
    y, S, h = oracle.layer_varlen(I["x"][0], I["z"][0], I["g"][0], I["beta"][0], I["w"], hp, Sp,
                                  [0, 0, 9], [1, 0], **KW)
    np.testing.assert_array_equal(S[1], Sp[1])
    np.testing.assert_array_equal(h[1], hp[1])
    y1, S1, _ = oracle.layer(I["x"], I["z"], I["g"], I["beta"], I["w"], I["hist"], I["S"], **KW)
    np.testing.assert_array_equal(y, y1[0])
    np.testing.assert_array_equal(S[0], S1[0])


def test_decode_multi_snapshots_are_prefix_states():
    T = 3
    I = geom(2, T, 3)
    hp = np.concatenate([I["hist"], np.zeros((4,) + I["hist"].shape[1:], np.float32)])
    Sp = np.concatenate([I["S"], np.zeros((4,) + I["S"].shape[1:], np.float32)])
    out = np.array([[2, 3, 0], [4, 5, 1]])
    y, S, h = oracle.decode_multi(I["x"], I["z"], I["g"], I["beta"], I["w"], hp, Sp, [0, 1],
                                  out, **KW)
    y_full, S_full, h_full = oracle.layer(I["x"], I["z"], I["g"], I["beta"], I["w"], I["hist"],
                                          I["S"], **KW)
    np.testing.assert_array_equal(y, y_full)  # the readout of token t does not see later tokens
    np.testing.assert_array_equal(S[[0, 1]], S_full)
    np.testing.assert_array_equal(h[[0, 1]], h_full)
    for t in range(T - 1):  # the snapshot after token t is the layer over tokens 0..t
        y_t, S_t, h_t = oracle.layer(I["x"][:, :t + 1], I["z"][:, :t + 1], I["g"][:, :t + 1],
                                     I["beta"][:, :t + 1], I["w"], I["hist"], I["S"], **KW)
        np.testing.assert_array_equal(S[out[:, t]], S_t)
        np.testing.assert_array_equal(h[out[:, t]], h_t)
        # and its conv history is the last three raw inputs up to token t
        cat = np.concatenate([I["hist"], I["x"][:, :t + 1]], axis=1)
        np.testing.assert_array_equal(h[out[:, t]], cat[:, -3:])


def test_decode_multi_padding_row_and_in_place():
    I = geom(2, 1, 4)
    y, S, h = oracle.decode_multi(I["x"], I["z"], I["g"], I["beta"], I["w"], I["hist"], I["S"],
                                  [1, -1], None, **KW)
    assert not np.any(y[1])
    np.testing.assert_array_equal(S[0], I["S"][0])  # slot 0 only belonged to the padding row
    y1, S1, h1 = oracle.layer(I["x"][:1], I["z"][:1], I["g"][:1], I["beta"][:1], I["w"],
                              I["hist"][1:], I["S"][1:], **KW)
    np.testing.assert_array_equal(y[0], y1[0])
    np.testing.assert_array_equal(S[1], S1[0])
    np.testing.assert_array_equal(h[1], h1[0])
