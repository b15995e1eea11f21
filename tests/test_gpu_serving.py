"""GPU parity of the serving-shaped entry points against the oracle:
slot-indexed multi-token decode with per-token state snapshots (MTP verify
and rollback), and packed variable-length prefill into a slot pool.

Sources: "Add Qwen3.8 MTP and multimodal inference on Metal without
regressing text", section Correctness gates (candidate verification, cache
updates, rollback); the model card "Qwen3.8-27B FP8 + native MTP +
multimodal Core AI", section What is fused (three-token target prefill);
"Implement the Qwen3.8 Flash Next Rust and Metal text core", section
Implementation (prefill/small-batch infrastructure) and its implementation
comment (resident-state swaps)."""
from __future__ import annotations

import numpy as np
import pytest

from gdn_inputs import Geometry, make_inputs
from gdn_testlib import EPS, check_errors, dims_of, from_dev, to_dev

pytestmark = pytest.mark.gpu


def pools(geom, n_slots, seed):
    """A pool of n_slots random conv histories and recurrent states."""
    g = Geometry(B=n_slots, T=1, H_k=geom.H_k, H_v=geom.H_v, d_k=geom.d_k, d_v=geom.d_v,
                 dtype=geom.dtype, zero_state=False)
    I = make_inputs(g, seed)
    return I["hist"], I["S"]


def oracle_kw(geom):
    return dict(H_k=geom.H_k, H_v=geom.H_v, d_k=geom.d_k, d_v=geom.d_v, eps=EPS)


@pytest.mark.parametrize("T,d,dtype", [(1, 128, "bf16"), (2, 128, "bf16"), (3, 128, "bf16"),
                                       (4, 128, "bf16"), (3, 16, "f32")])
def test_decode_multi_snapshots(T, d, dtype):
    import gated_deltanet_layer_gdn_amd as gdn
    import oracle
    import torch

    geom = Geometry(B=5, T=T, H_k=4, H_v=12, d_k=d, d_v=d, dtype=dtype, zero_state=False)
    I = make_inputs(geom, seed=400 + T)
    n_slots = 32
    hp, Sp = pools(geom, n_slots, seed=450 + T)
    # rows 0..4 start from scattered slots; row 3 is a padding row; each real
    # row stores the state after every token to a distinct slot, the last
    # token's state back into its in slot (an update in place).
    in_slots = np.array([7, 0, 19, -1, 30], np.int32)
    out_slots = np.full((geom.B, T), -1, np.int32)
    free = iter(s for s in range(n_slots) if s not in in_slots)
    for b in range(geom.B):
        if in_slots[b] < 0:
            out_slots[b] = [next(free) for _ in range(T)]  # ignored for padding rows
            continue
        for t in range(T - 1):
            out_slots[b, t] = next(free)
        out_slots[b, T - 1] = in_slots[b]
    y_ref, S_ref, h_ref = oracle.decode_multi(I["x"], I["z"], I["g"], I["beta"], I["w"], hp, Sp,
                                              in_slots, out_slots, **oracle_kw(geom))
    dims = dims_of(geom)
    hp_d, Sp_d = to_dev(hp), to_dev(Sp)
    y = gdn.decode_multi(dims, to_dev(I["x"]), to_dev(I["z"]), to_dev(I["g"]), to_dev(I["beta"]),
                         to_dev(I["w"]), hp_d, Sp_d, to_dev(in_slots), to_dev(out_slots))
    torch.cuda.synchronize()
    y = y.double().cpu().numpy()
    S = Sp_d.cpu().numpy()
    h = from_dev(hp_d)
    real = in_slots >= 0
    check_errors(f"decode_multi T={T} d={d} (real rows)", y[real], y_ref[real], S, S_ref)
    assert not np.any(y[~real]), "padding rows must give zero y"
    np.testing.assert_array_equal(h, h_ref)
    touched = set(in_slots[real]) | set(out_slots[real].ravel())
    for s in range(n_slots):
        if s not in touched:  # untouched slots keep their bytes
            np.testing.assert_array_equal(S[s].view(np.uint32), Sp[s].view(np.uint32))
            np.testing.assert_array_equal(h[s], hp[s])


def test_decode_multi_equals_single_steps():
    # One three-token step against three single-token steps on the same
    # states: the per-token arithmetic is the same, so the results agree bit
    # for bit; the state after the first two tokens stays in their slots.
    import gated_deltanet_layer_gdn_amd as gdn
    import torch

    geom = Geometry(B=4, T=3, H_k=16, H_v=48, d_k=128, d_v=128, zero_state=False)
    I = make_inputs(geom, seed=470)
    d = dims_of(geom)
    D = {k: to_dev(v) for k, v in I.items()}
    S1, h1 = D["S"].clone(), D["hist"].clone()
    ys = []
    snaps = []
    for t in range(3):
        ys.append(gdn.decode_step(d, D["x"][:, t].contiguous(), D["z"][:, t].contiguous(),
                                  D["g"][:, t].contiguous(), D["beta"][:, t].contiguous(),
                                  D["w"], h1, S1))
        snaps.append((S1.clone(), h1.clone()))
    n_slots = 3 * geom.B
    Sp = torch.zeros((n_slots,) + tuple(D["S"].shape[1:]), device="cuda")
    hp = torch.zeros((n_slots,) + tuple(D["hist"].shape[1:]), dtype=D["hist"].dtype, device="cuda")
    Sp[:geom.B] = D["S"]
    hp[:geom.B] = D["hist"]
    in_slots = torch.arange(geom.B, dtype=torch.int32, device="cuda")
    out = np.stack([np.array([geom.B + b, 2 * geom.B + b, b]) for b in range(geom.B)]).astype(np.int32)
    y = gdn.decode_multi(d, D["x"], D["z"], D["g"], D["beta"], D["w"], hp, Sp, in_slots,
                         to_dev(out))
    torch.cuda.synchronize()
    y_single = torch.stack(ys, 1)
    np.testing.assert_array_equal(y.cpu().numpy().view(np.uint32),
                                  y_single.cpu().numpy().view(np.uint32))
    for t, slot0 in enumerate((geom.B, 2 * geom.B, 0)):
        S_t, h_t = snaps[t]
        np.testing.assert_array_equal(Sp[slot0:slot0 + geom.B].cpu().numpy().view(np.uint32),
                                      S_t.cpu().numpy().view(np.uint32))
        np.testing.assert_array_equal(from_dev(hp[slot0:slot0 + geom.B]), from_dev(h_t))


@pytest.mark.parametrize("chunk", [64, 128])
def test_prefill_varlen(chunk):
    import gated_deltanet_layer_gdn_amd as gdn
    import oracle
    import torch

    lens = [77, 0, 1, 200, 3, 64, 130]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T_total = int(cu[-1])
    geom = Geometry(B=1, T=T_total, H_k=4, H_v=12, d_k=128, d_v=128, zero_state=False)
    I = make_inputs(geom, seed=480 + chunk)
    n_slots = 10
    hp, Sp = pools(geom, n_slots, seed=490)
    slots = np.array([4, 9, 0, 7, 2, 5, 8], np.int32)
    x, z, g, beta = (I[k][0] for k in ("x", "z", "g", "beta"))
    y_ref, S_ref, h_ref = oracle.layer_varlen(x, z, g, beta, I["w"], hp, Sp, cu, slots,
                                              **oracle_kw(geom))
    d = dims_of(Geometry(B=len(lens), T=1, H_k=4, H_v=12, d_k=128, d_v=128))
    hp_d, Sp_d = to_dev(hp), to_dev(Sp)
    y = gdn.prefill_varlen(d, cu, to_dev(x), to_dev(z), to_dev(g), to_dev(beta), to_dev(I["w"]),
                           hp_d, Sp_d, slots, chunk=chunk)
    torch.cuda.synchronize()
    y = y.double().cpu().numpy()
    S = Sp_d.cpu().numpy()
    h = from_dev(hp_d)
    check_errors(f"prefill_varlen C={chunk} lens={lens}", y[None], y_ref[None], S, S_ref)
    np.testing.assert_array_equal(h, h_ref)
    for s in set(range(n_slots)) - set(int(v) for n, v in enumerate(slots) if lens[n] > 0):
        np.testing.assert_array_equal(S[s].view(np.uint32), Sp[s].view(np.uint32))
        np.testing.assert_array_equal(h[s], hp[s])
    # each sequence bit for bit as gdn_prefill_chunked alone gives it
    d1 = dims_of(Geometry(B=1, T=1, H_k=4, H_v=12, d_k=128, d_v=128))
    for n, L in enumerate(lens):
        if L == 0:
            continue
        a, b = int(cu[n]), int(cu[n + 1])
        h1, S1 = to_dev(hp[slots[n]][None].copy()), to_dev(Sp[slots[n]][None].copy())
        y1 = gdn.prefill_chunked(d1, to_dev(x[None, a:b].copy()), to_dev(z[None, a:b].copy()),
                                 to_dev(g[None, a:b].copy()), to_dev(beta[None, a:b].copy()),
                                 to_dev(I["w"]), h1, S1, chunk=chunk)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(y1.cpu().numpy()[0].view(np.uint32),
                                      y[a:b].astype(np.float32).view(np.uint32))
        np.testing.assert_array_equal(S1.cpu().numpy()[0].view(np.uint32),
                                      S[slots[n]].view(np.uint32))


def test_prefill_varlen_graph_replay():
    # The call forks its sequences onto up to three streams and joins them back
    # by events; captured into a graph and replayed three times (pools reset
    # in between, with eager work on the stream), every replay equals the
    # eager call bit for bit.
    import gated_deltanet_layer_gdn_amd as gdn
    import torch

    lens = [300, 5, 129, 64, 1, 250]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T_total = int(cu[-1])
    geom = Geometry(B=1, T=T_total, H_k=4, H_v=12, d_k=128, d_v=128, zero_state=False)
    I = make_inputs(geom, seed=510)
    n_slots = 8
    hp, Sp = pools(geom, n_slots, seed=511)
    slots = [3, 0, 6, 1, 7, 4]
    x, z, g, beta = (to_dev(I[k][0]) for k in ("x", "z", "g", "beta"))
    w = to_dev(I["w"])
    d = dims_of(Geometry(B=len(lens), T=1, H_k=4, H_v=12, d_k=128, d_v=128))
    hp0, Sp0 = to_dev(hp), to_dev(Sp)
    hp_d, Sp_d = hp0.clone(), Sp0.clone()
    y = torch.empty(T_total, 12, 128, device="cuda")
    ws = torch.empty(gdn.prefill_varlen_workspace_bytes(d, cu, 64), dtype=torch.uint8, device="cuda")
    gdn.prefill_varlen(d, cu, x, z, g, beta, w, hp_d, Sp_d, slots, chunk=64, y=y, ws=ws)
    torch.cuda.synchronize()
    y_ref, S_ref, h_ref = y.clone(), Sp_d.clone(), hp_d.clone()
    hp_d.copy_(hp0)
    Sp_d.copy_(Sp0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gdn.prefill_varlen(d, cu, x, z, g, beta, w, hp_d, Sp_d, slots, chunk=64, y=y, ws=ws)
    for rep in range(3):
        hp_d.copy_(hp0)
        Sp_d.copy_(Sp0)
        y.zero_()
        graph.replay()
        torch.cuda.synchronize()
        print(f"[parity] varlen graph replay {rep}", flush=True)
        assert torch.equal(y, y_ref) and torch.equal(Sp_d, S_ref) and torch.equal(hp_d, h_ref)
