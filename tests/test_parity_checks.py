"""CPU checks of the parity bar itself (gdn_testlib.check_errors): a single
wrong row or head must fail it even when the whole-tensor figure passes.  The
mistakes are planted in oracle outputs on the CPU."""
from __future__ import annotations

import numpy as np
import pytest

from gdn_inputs import Geometry, make_inputs
from gdn_testlib import ROW_TOL, TOL, check_errors, oracle_run, rel_l2


@pytest.fixture(scope="module")
def ref():
    geom = Geometry(B=2, T=300, H_k=2, H_v=6, d_k=16, d_v=16, dtype="f32", zero_state=False)
    I = make_inputs(geom, seed=123)
    y, S, _ = oracle_run(geom, I)
    return y, S


def noisy(a, rel, seed):
    rng = np.random.default_rng(seed)
    return a + rel * np.abs(a).mean() * rng.standard_normal(a.shape)


def test_small_noise_passes(ref):
    y, S = ref
    f = check_errors("noise 1e-5", noisy(y, 1e-5, 1), y, noisy(S, 1e-5, 2), S)
    assert f["y_row"] < ROW_TOL and f["y_head"] < TOL


def test_one_wrong_row_fails_although_whole_tensor_passes(ref):
    y, S = ref
    bad = y.copy()
    bad[1, 123, 4] *= 1.08  # one (sequence, token, head) row off by 8% of its size
    assert rel_l2(bad, y) <= TOL  # the whole-tensor figure alone would pass
    with pytest.raises(AssertionError):
        check_errors("one bad row", bad, y, S, S)


def test_one_wrong_state_row_fails(ref):
    y, S = ref
    bad = S.copy()
    bad[0, 3, 7] = -bad[0, 3, 7]
    with pytest.raises(AssertionError):
        check_errors("one bad state row", y, y, bad, S)


def test_swapped_heads_fail(ref):
    y, S = ref
    bad = y.copy()
    bad[:, :, [2, 3]] = bad[:, :, [3, 2]]
    with pytest.raises(AssertionError):
        check_errors("two heads swapped", bad, y, S, S)


def test_zero_reference_needs_zero_error(ref):
    y, S = ref
    z = np.zeros_like(y)
    check_errors("all zero", z, z, S, S)
    off = z.copy()
    off[0, 0, 0, 0] = 1e-30
    with pytest.raises(AssertionError):
        check_errors("zero reference, nonzero output", off, z, S, S)
