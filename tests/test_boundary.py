"""Host-side tests of the C ABI (no GPU needed).

Every validation path of libgdn.so runs before any HIP call, so these tests
pass ordinary host buffers in place of device pointers: the library must
reject the call and leave every byte of them unchanged (fail before partial
execution).  The state-blob checks (header, dims, sizes, checksums) and the
injected launch failure run the same way.
"""
from __future__ import annotations

import ctypes
import os
import re
import struct

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

OK, INVALID, UNSUPPORTED, ALIGN, ALIAS, WORKSPACE = 0, -1, -2, -3, -4, -5
B_MAGIC, B_VERSION, B_SHAPE, B_SIZE, B_CHECKSUM, HIP, TOO_LARGE = -6, -7, -8, -9, -10, -11, -12


@pytest.fixture(scope="module")
def lib():
    from gated_deltanet_layer_gdn_amd import _lib

    if not os.path.exists(_lib.SO_PATH):
        from gated_deltanet_layer_gdn_amd import build

        build.build()
    return _lib.load()


@pytest.fixture
def dims():
    from gated_deltanet_layer_gdn_amd import _lib

    return _lib.GdnDims(_lib.ABI_VERSION, 2, 2, 6, 16, 16, 4, 1, 0, 1e-6, 1.0)


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"GDN_API\s+[\w\s\*]+?\b(gdn_\w+)\s*\(", text)


def test_exports_every_declared_symbol(lib):
    from gated_deltanet_layer_gdn_amd import _lib

    names = declared_functions()
    assert len(names) == len(set(names)) >= 14
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.EXPORTS)


def test_abi_version_and_status_strings(lib):
    assert lib.gdn_abi_version() == 1
    for code in range(-12, 1):
        s = lib.gdn_status_str(code).decode()
        assert s and s != "unknown status"
    assert lib.gdn_status_str(-99).decode() == "unknown status"
    assert lib.gdn_last_hip_error().decode() == ""


def C_ch(d):
    return 2 * d.H_k * d.d_k + d.H_v * d.d_v


def test_size_queries(lib, dims):
    d = dims
    b = ctypes.byref(d)
    assert lib.gdn_rec_state_bytes(b) == d.B * d.H_v * d.d_v * d.d_k * 4
    assert lib.gdn_conv_state_bytes(b) == d.B * (d.W - 1) * C_ch(d) * 2
    assert lib.gdn_state_blob_bytes(b) == 128 + lib.gdn_rec_state_bytes(b) + lib.gdn_conv_state_bytes(b)
    assert lib.gdn_decode_workspace_bytes(b) >= d.B * C_ch(d) * 4
    w = [lib.gdn_prefill_workspace_bytes(b, T, 64) for T in (1, 64, 65, 1000)]
    assert all(x > 0 for x in w) and w == sorted(w)
    assert lib.gdn_prefill_workspace_bytes(b, 0, 64) == 0
    assert lib.gdn_prefill_workspace_bytes(b, 1 << 24, 64) > 0  # the largest T accepted
    assert lib.gdn_prefill_workspace_bytes(b, (1 << 24) + 1, 64) == 0
    assert lib.gdn_prefill_workspace_bytes(b, 64, 48) == 0
    for C in (16, 32, 64, 128):
        assert lib.gdn_prefill_workspace_bytes(b, 100, C) > 0
    d.d_k = d.d_v = 64  # not a built geometry
    assert lib.gdn_rec_state_bytes(b) == 0


class Bufs:
    """Host stand-ins for every buffer of a prefill call, filled with canary
    bytes, 256-byte aligned inside one big array each."""

    def __init__(self, d, T, ws_bytes):
        es = 2 if d.in_dtype == 1 else 4
        eo = 2 if d.out_dtype == 1 else 4
        sizes = dict(x=d.B * T * C_ch(d) * es, z=d.B * T * d.H_v * d.d_v * es,
                     g=d.B * T * d.H_v * 4, beta=d.B * T * d.H_v * 4, w=C_ch(d) * d.W * es,
                     hist=d.B * (d.W - 1) * C_ch(d) * es, S=d.B * d.H_v * d.d_v * d.d_k * 4,
                     y=d.B * T * d.H_v * d.d_v * eo, ws=ws_bytes)
        rng = np.random.default_rng(0)
        self.arr = {}
        for k, n in sizes.items():
            raw = rng.integers(0, 256, n + 512, dtype=np.uint8)
            off = (-raw.ctypes.data) % 256
            self.arr[k] = (raw, off, n)
        self.snap = {k: v[0].copy() for k, v in self.arr.items()}

    def p(self, k, shift=0):
        raw, off, _ = self.arr[k]
        return ctypes.c_void_p(raw.ctypes.data + off + shift)

    def n(self, k):
        return self.arr[k][2]

    def unchanged(self):
        return all(np.array_equal(self.arr[k][0], self.snap[k]) for k in self.arr)


def prefill_call(lib, d, T, C, b, **over):
    args = dict(x=b.p("x"), z=b.p("z"), g=b.p("g"), beta=b.p("beta"), w=b.p("w"),
                hist=b.p("hist"), S=b.p("S"), y=b.p("y"), ws=b.p("ws"), ws_bytes=b.n("ws"))
    args.update(over)
    return lib.gdn_prefill_chunked(ctypes.byref(d), T, C, args["x"], args["z"], args["g"],
                                   args["beta"], args["w"], args["hist"], args["S"], args["y"],
                                   args["ws"], args["ws_bytes"], None)


def test_prefill_rejects_and_leaves_buffers_untouched(lib, dims):
    d, T, C = dims, 40, 16
    need = lib.gdn_prefill_workspace_bytes(ctypes.byref(d), T, C)
    b = Bufs(d, T, need)
    cases = [
        (dict(x=None), INVALID),
        (dict(S=None), INVALID),
        (dict(ws=None), INVALID),
        (dict(S=b.p("S", 4)), ALIGN),          # state must be 16-byte aligned
        (dict(ws=b.p("ws", 8)), ALIGN),
        (dict(x=b.p("x", 1)), ALIGN),          # bf16 input at an odd address
        (dict(x=b.p("x", 2)), ALIGN),          # prefill x must be 16-byte aligned
        (dict(hist=b.p("hist", 2)), ALIGN),    # and so must the conv history
        (dict(y=b.p("x")), ALIAS),             # output over an input
        (dict(ws=b.p("S")), ALIAS),            # workspace over the state
        (dict(hist=b.p("S")), ALIAS),          # conv state over the recurrent state
        (dict(ws_bytes=need - 1), WORKSPACE),
    ]
    for over, want in cases:
        assert prefill_call(lib, d, T, C, b, **over) == want, over
    assert prefill_call(lib, d, 0, C, b) == INVALID
    assert prefill_call(lib, d, (1 << 24) + 1, C, b) == INVALID  # past the largest T
    assert prefill_call(lib, d, T, 48, b) == UNSUPPORTED
    assert prefill_call(lib, d, T, 8, b) == UNSUPPORTED
    for field, val, want in [("abi", 2, UNSUPPORTED), ("d_k", 64, UNSUPPORTED),
                             ("W", 3, UNSUPPORTED), ("H_v", 5, UNSUPPORTED), ("B", 0, INVALID),
                             ("in_dtype", 7, UNSUPPORTED), ("l2_eps", -1.0, INVALID),
                             ("l2_eps", float("nan"), INVALID)]:
        old = getattr(d, field)
        setattr(d, field, val)
        assert prefill_call(lib, d, T, C, b) == want, field
        setattr(d, field, old)
    assert lib.gdn_prefill_chunked(None, T, C, *[None] * 9, 0, None) == INVALID
    assert b.unchanged()


def test_decode_and_conv_reject_and_leave_buffers_untouched(lib, dims):
    d = dims
    need = lib.gdn_decode_workspace_bytes(ctypes.byref(d))
    b = Bufs(d, 1, need)
    dec = lambda **o: lib.gdn_decode_step(
        ctypes.byref(d), o.get("x", b.p("x")), b.p("z"), b.p("g"), b.p("beta"), b.p("w"),
        o.get("hist", b.p("hist")), o.get("S", b.p("S")), o.get("y", b.p("y")),
        o.get("ws", b.p("ws")), o.get("ws_bytes", need), None)
    assert dec(x=None) == INVALID
    assert dec(S=b.p("S", 4)) == ALIGN
    assert dec(y=b.p("z")) == ALIAS
    assert dec(ws_bytes=need - 4) == WORKSPACE
    conv = lambda T, **o: lib.gdn_conv1d(ctypes.byref(d), T, o.get("x", b.p("x")), b.p("w"),
                                         o.get("hist", b.p("hist")), o.get("out", b.p("y")),
                                         None)
    assert conv(0) == INVALID
    assert conv(1, out=None) == INVALID
    assert conv(1, out=b.p("x")) == ALIAS
    assert conv(1, hist=b.p("w")) == ALIAS
    assert b.unchanged()


def test_decode_noalloc_validates_before_any_hip_call(lib, dims):
    # The entry point that allocates nothing: the same argument checks as
    # gdn_decode_step (there is no workspace argument), and sizes beyond its
    # fixed 16 MiB scratch are refused before anything else.
    d = dims
    b = Bufs(d, 1, 0)
    call = lambda **o: lib.gdn_decode_step_noalloc(
        ctypes.byref(d), o.get("x", b.p("x")), b.p("z"), b.p("g"), b.p("beta"), b.p("w"),
        o.get("hist", b.p("hist")), o.get("S", b.p("S")), o.get("y", b.p("y")), None)
    assert call(x=None) == INVALID
    assert call(S=b.p("S", 4)) == ALIGN
    assert call(y=b.p("z")) == ALIAS
    assert b.unchanged()
    from gated_deltanet_layer_gdn_amd import _lib

    big = _lib.GdnDims(_lib.ABI_VERSION, 500, 16, 48, 128, 128, 4, 1, 0, 1e-6, 1.0)
    assert lib.gdn_decode_workspace_bytes(ctypes.byref(big)) > 16 << 20
    assert lib.gdn_decode_step_noalloc(ctypes.byref(big), *[None] * 8, None) == TOO_LARGE
    assert "fixed scratch" in lib.gdn_status_str(TOO_LARGE).decode()


def test_decode_multi_rejects_and_leaves_buffers_untouched(lib, dims):
    # Slot-indexed multi-token decode: every argument check runs on the host
    # before any HIP call (the slot values themselves live on the device).
    d = dims
    d.d_k = d.d_v = 128
    T = 3
    need = T * lib.gdn_decode_workspace_bytes(ctypes.byref(d))
    b = Bufs(d, T, need)
    slots = np.zeros(d.B * T + 64, np.int32)
    sp = lambda off=0: ctypes.c_void_p(slots.ctypes.data + off)
    pool_S = b.p("S")  # B = 2 slots' worth; n_slots = 2 below unless changed

    def call(**o):
        return lib.gdn_decode_multi(
            ctypes.byref(d), o.get("T", T), b.p("x"), b.p("z"), b.p("g"), b.p("beta"), b.p("w"),
            o.get("hist", b.p("hist")), o.get("S", pool_S), o.get("n_slots", d.B),
            o.get("ins", sp()), o.get("outs", sp(64)), o.get("y", b.p("y")), b.p("ws"),
            o.get("ws_bytes", need), None)

    assert call(T=0) == INVALID
    assert call(T=5) == INVALID
    assert call(n_slots=0) == INVALID
    assert call(ins=None) == INVALID
    assert call(y=b.p("S")) == ALIAS
    assert call(S=b.p("S", 4)) == ALIGN
    assert call(ws_bytes=need - 1) == WORKSPACE
    assert b.unchanged()


def test_prefill_varlen_rejects_bad_tables_and_leaves_buffers_untouched(lib, dims):
    d = dims
    d.B = 3
    cu = np.array([0, 5, 5, 12], np.int64)
    pcu = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    need = lib.gdn_prefill_varlen_workspace_bytes(ctypes.byref(d), pcu(cu), 64)
    assert need > 0
    one = lib.gdn_prefill_workspace_bytes(ctypes.byref(d), 7, 64)  # B=3 here: an upper bound
    assert need <= one
    b = Bufs(d, 4, need)  # 3 * 4 = 12 token rows
    slots = np.array([2, 0, 1], np.int32)

    def call(cu_=cu, slots_=slots, n_slots=3, chunk=64, **o):
        return lib.gdn_prefill_varlen(
            ctypes.byref(d), pcu(cu_), chunk, b.p("x"), b.p("z"), b.p("g"), b.p("beta"),
            b.p("w"), b.p("hist"), b.p("S"), n_slots, slots_.ctypes.data_as(ctypes.c_void_p),
            o.get("y", b.p("y")), b.p("ws"), o.get("ws_bytes", need), None)

    assert call(cu_=np.array([1, 5, 5, 12], np.int64)) == INVALID   # does not start at 0
    assert call(cu_=np.array([0, 5, 4, 12], np.int64)) == INVALID   # decreasing
    assert call(slots_=np.array([2, 0, 3], np.int32)) == INVALID    # slot out of range
    assert call(slots_=np.array([2, 0, 2], np.int32)) == INVALID    # two sequences, one slot
    assert call(chunk=48) == UNSUPPORTED
    assert call(y=b.p("x")) == ALIAS
    assert call(ws_bytes=need - 1) == WORKSPACE
    assert lib.gdn_prefill_varlen_workspace_bytes(ctypes.byref(d), None, 64) == 0
    assert b.unchanged()


def test_attn_rejects_and_leaves_buffers_untouched(lib):
    from gated_deltanet_layer_gdn_amd import _lib

    B, T, T_max, H_q, H_kv, d = 2, 40, 64, 6, 2, 128
    a = _lib.GdnAttnDims(_lib.ABI_VERSION, B, H_q, H_kv, d, 32, 1, 0, 1e4, d ** -0.5)
    need = lib.gdn_attn_workspace_bytes(ctypes.byref(a), T, 0)
    assert need >= T * 16 * 8  # RoPE cos/sin table (+ split partials)
    assert lib.gdn_attn_workspace_bytes(ctypes.byref(a), 0, 0) == 0
    assert lib.gdn_attn_workspace_bytes(ctypes.byref(a), 1 << 22, 0) == 0  # launch size limit
    # no rotation and no KV split (one block of rows): still a non-zero size,
    # since zero means invalid arguments
    a0 = _lib.GdnAttnDims(_lib.ABI_VERSION, 1, 4, 1, 256, 0, 1, 1, 1e7, 256 ** -0.5)
    assert lib.gdn_attn_workspace_bytes(ctypes.byref(a0), 4, 60) > 0
    rng = np.random.default_rng(0)
    mk = lambda n: rng.integers(0, 255, n, dtype=np.uint8)
    bufs = dict(q=mk(B * T * H_q * d * 2 + 64), k=mk(B * T * H_kv * d * 2 + 64),
                v=mk(B * T * H_kv * d * 2 + 64), kc=mk(B * T_max * H_kv * d * 2 + 64),
                vc=mk(B * T_max * H_kv * d * 2 + 64), o=mk(B * T * H_q * d * 4 + 64),
                ws=mk(need + 64))
    copies = {n: v.copy() for n, v in bufs.items()}
    p = lambda n, off=0: ctypes.c_void_p(bufs[n].ctypes.data + (-bufs[n].ctypes.data % 16) + off)

    def call(dims_=a, T_=T, pos0=0, T_max_=T_max, ws_bytes=need, **o):
        return lib.gdn_attn_prefill(ctypes.byref(dims_), T_, pos0, o.get("q", p("q")), p("k"), p("v"),
                                    o.get("kc", p("kc")), p("vc"), T_max_, o.get("o", p("o")),
                                    p("ws"), ws_bytes, None)

    def variant(**f):
        b = _lib.GdnAttnDims.from_buffer_copy(a)
        for k_, v_ in f.items():
            setattr(b, k_, v_)
        return b

    assert call(T_=0) == INVALID
    assert call(pos0=T_max - T + 1) == INVALID                  # past the cache
    assert call(T_max_=T - 1) == INVALID
    assert call(dims_=variant(H_q=5)) == UNSUPPORTED            # not a multiple of H_kv
    assert call(dims_=variant(d_h=64)) == UNSUPPORTED
    assert call(dims_=variant(rot_dim=33)) == INVALID
    assert call(dims_=variant(rot_dim=24)) == INVALID             # not a multiple of 16
    assert call(dims_=variant(rot_dim=130)) == INVALID
    assert call(dims_=variant(in_dtype=0)) == UNSUPPORTED
    assert call(dims_=variant(out_dtype=2)) == UNSUPPORTED
    assert call(dims_=variant(rope_base=1.0)) == INVALID
    assert call(dims_=variant(abi=7)) == UNSUPPORTED
    assert call(q=None) == INVALID
    assert call(q=p("q", 2)) == ALIGN
    assert call(o=p("kc")) == ALIAS
    assert call(kc=p("vc")) == ALIAS
    assert call(ws_bytes=need - 1) == WORKSPACE
    for n in bufs:
        np.testing.assert_array_equal(bufs[n], copies[n], err_msg=n)


def test_injected_launch_failure_leaves_buffers_untouched(lib, dims, monkeypatch):
    d, T, C = dims, 20, 32
    need = lib.gdn_prefill_workspace_bytes(ctypes.byref(d), T, C)
    b = Bufs(d, T, need)
    monkeypatch.setenv("GDN_TEST_FAIL_LAUNCH", "1")
    assert prefill_call(lib, d, T, C, b) == HIP
    assert "injected" in lib.gdn_last_hip_error().decode()
    assert b.unchanged()


# ----------------------------------------------------------------- state blob

def fnv1a64(data: bytes) -> int:
    h = 0xCBF29CE484222325
    for c in data:
        h ^= c
        h = (h * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h


def make_blob(d, conv: bytes, rec: bytes, version=1, magic=b"GDNSTATE"):
    head = magic + struct.pack("<II6iiiQQ", version, 128, d.B, d.H_k, d.H_v, d.d_k, d.d_v, d.W,
                               d.in_dtype, 0, len(conv), len(rec))
    head += struct.pack("<Q", fnv1a64(conv + rec))
    head += struct.pack("<Q", fnv1a64(head))
    head += bytes(128 - len(head))
    return np.frombuffer(head + conv + rec, np.uint8).copy()


def check(lib, d, blob):
    return lib.gdn_state_check(ctypes.byref(d), blob.ctypes.data_as(ctypes.c_void_p), blob.size)


def test_state_blob_validation(lib, dims):
    d = dims
    cb = lib.gdn_conv_state_bytes(ctypes.byref(d))
    rb = lib.gdn_rec_state_bytes(ctypes.byref(d))
    rng = np.random.default_rng(1)
    conv = rng.integers(0, 256, cb, dtype=np.uint8).tobytes()
    rec = rng.integers(0, 256, rb, dtype=np.uint8).tobytes()
    good = make_blob(d, conv, rec)
    assert good.size == lib.gdn_state_blob_bytes(ctypes.byref(d))
    assert check(lib, d, good) == OK
    assert check(lib, d, make_blob(d, conv, rec, magic=b"GDNSTATX")) == B_MAGIC
    assert check(lib, d, make_blob(d, conv, rec, version=2)) == B_VERSION
    bad = good.copy()
    bad[20] ^= 1  # header byte changed without fixing its checksum
    assert check(lib, d, bad) == B_CHECKSUM
    bad = good.copy()
    bad[128 + cb + 5] ^= 0x40  # one payload bit
    assert check(lib, d, bad) == B_CHECKSUM
    assert check(lib, d, good[:-1]) == B_SIZE
    assert check(lib, d, good[:64]) == B_SIZE
    other = type(d).from_buffer_copy(d)
    other.H_v = 4  # blob written for different dims
    assert check(lib, other, good) == B_SHAPE
    # restore validates first: a corrupt blob leaves the (host stand-in) state alone
    canary_c = np.full(cb + 64, 7, np.uint8)
    canary_r = np.full(rb + 64, 9, np.uint8)
    pc = ctypes.c_void_p(canary_c.ctypes.data + ((-canary_c.ctypes.data) % 16))
    pr = ctypes.c_void_p(canary_r.ctypes.data + ((-canary_r.ctypes.data) % 16))
    bad = good.copy()
    bad[-1] ^= 1
    rc = lib.gdn_state_restore(ctypes.byref(d), bad.ctypes.data_as(ctypes.c_void_p), bad.size,
                               pc, pr, None)
    assert rc == B_CHECKSUM
    assert np.all(canary_c == 7) and np.all(canary_r == 9)


def test_binding_has_no_fallback(monkeypatch):
    """The Python binding fails loudly when libgdn.so is missing."""
    from gated_deltanet_layer_gdn_amd import _lib

    monkeypatch.setattr(_lib, "_LIB", None)
    monkeypatch.setattr(_lib, "SO_PATH", "/nonexistent/libgdn.so")
    with pytest.raises(RuntimeError, match="missing"):
        _lib.load()
