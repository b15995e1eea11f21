"""gdn_decode_step_noalloc (the entry point that allocates nothing) against
gdn_decode_step, through the C ABI: bit-identical outputs, states and conv
histories on two calls in a row, the second with fewer sequences, each call
two decode steps long (so the second step reads what the first left in the
shared scratch)."""
from __future__ import annotations

import numpy as np
import pytest

from gdn_inputs import Geometry, make_inputs
from gdn_testlib import dev_inputs, dims_of, from_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B_first,B_second", [(8, 3)])
def test_decode_noalloc_matches_decode_step(B_first, B_second):
    import gated_deltanet_layer_gdn_amd as gdn
    import torch

    for call, B in enumerate((B_first, B_second)):
        geom = Geometry(B=B, T=2, H_k=16, H_v=48, d_k=128, d_v=128, zero_state=False)
        I = make_inputs(geom, seed=300 + call)
        d = dims_of(geom)
        ref = dev_inputs(I)
        got = dev_inputs(I)
        print(f"[no-alloc] call {call}: B={B}, {geom.T} steps", flush=True)
        for t in range(geom.T):
            args = lambda D: (D["x"][:, t].contiguous(), D["z"][:, t].contiguous(),
                              D["g"][:, t].contiguous(), D["beta"][:, t].contiguous(), D["w"],
                              D["hist"], D["S"])
            y_ref = gdn.decode_step(d, *args(ref))
            y_got = torch.full_like(y_ref, float("nan"))
            gdn.decode_step_noalloc(d, *args(got), y_got)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(y_got.cpu().numpy().view(np.uint32),
                                          y_ref.cpu().numpy().view(np.uint32))
        np.testing.assert_array_equal(got["S"].cpu().numpy().view(np.uint32),
                                      ref["S"].cpu().numpy().view(np.uint32))
        np.testing.assert_array_equal(from_dev(got["hist"]), from_dev(ref["hist"]))


def test_decode_noalloc_rejects_beyond_scratch():
    import ctypes

    from gated_deltanet_layer_gdn_amd import _lib

    L = _lib.load()
    d = _lib.GdnDims(_lib.ABI_VERSION, 500, 16, 48, 128, 128, 4, 1, 0, 1e-6, 1.0)
    assert L.gdn_decode_workspace_bytes(ctypes.byref(d)) > 16 << 20
    assert L.gdn_decode_step_noalloc(ctypes.byref(d), *[None] * 8, None) == -12
