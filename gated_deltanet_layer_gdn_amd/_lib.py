"""ctypes declarations for libgdn.so (the C ABI in include/gdn.h).

The library must have been built (``python -m gated_deltanet_layer_gdn_amd.build``
or ``__graft_entry__.build()``); loading fails loudly otherwise.  There is no
fallback implementation of any step.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
SO_PATH = os.path.join(HERE, "libgdn.so")

GDN_OK = 0
STATUS = {
    0: "GDN_OK", -1: "GDN_ERR_INVALID_ARG", -2: "GDN_ERR_UNSUPPORTED", -3: "GDN_ERR_ALIGNMENT",
    -4: "GDN_ERR_ALIAS", -5: "GDN_ERR_WORKSPACE", -6: "GDN_ERR_BLOB_MAGIC",
    -7: "GDN_ERR_BLOB_VERSION", -8: "GDN_ERR_BLOB_SHAPE", -9: "GDN_ERR_BLOB_SIZE",
    -10: "GDN_ERR_BLOB_CHECKSUM", -11: "GDN_ERR_HIP", -12: "GDN_ERR_TOO_LARGE",
}
F32, BF16, F16 = 0, 1, 2
ABI_VERSION = 1

EXPORTS = (
    "gdn_abi_version", "gdn_status_str", "gdn_last_hip_error", "gdn_rec_state_bytes",
    "gdn_conv_state_bytes", "gdn_state_blob_bytes", "gdn_prefill_workspace_bytes",
    "gdn_decode_workspace_bytes", "gdn_conv1d", "gdn_prefill_chunked", "gdn_decode_step",
    "gdn_state_save", "gdn_state_restore", "gdn_state_check", "gdn_prefill_chunked_timed",
    "gdn_decode_step_timed", "gdn_decode_step_noalloc", "gdn_decode_multi",
    "gdn_prefill_varlen", "gdn_prefill_varlen_workspace_bytes", "gdn_gated_rmsnorm",
    "gdn_in_proj", "gdn_attn_workspace_bytes", "gdn_attn_prefill",
)


class GdnDims(ctypes.Structure):
    _fields_ = [
        ("abi", ctypes.c_int32), ("B", ctypes.c_int32), ("H_k", ctypes.c_int32),
        ("H_v", ctypes.c_int32), ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
        ("W", ctypes.c_int32), ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("l2_eps", ctypes.c_float), ("q_scale", ctypes.c_float),
    ]


class GdnAttnDims(ctypes.Structure):
    _fields_ = [
        ("abi", ctypes.c_int32), ("B", ctypes.c_int32), ("H_q", ctypes.c_int32),
        ("H_kv", ctypes.c_int32), ("d_h", ctypes.c_int32), ("rot_dim", ctypes.c_int32),
        ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("rope_base", ctypes.c_float), ("scale", ctypes.c_float),
    ]


class GdnError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        name = STATUS.get(status, str(status))
        super().__init__(f"{where}: {name}" + (f" ({detail})" if detail else ""))


_LIB = None


def load():
    """Load libgdn.so once and declare its signatures."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(SO_PATH):
        raise RuntimeError(
            f"{SO_PATH} is missing: build it with `python -m gated_deltanet_layer_gdn_amd.build`")
    L = ctypes.CDLL(SO_PATH)
    vp, sz, i32, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
    dp = ctypes.POINTER(GdnDims)
    L.gdn_abi_version.restype = ctypes.c_int
    L.gdn_abi_version.argtypes = []
    L.gdn_status_str.restype = ctypes.c_char_p
    L.gdn_status_str.argtypes = [ctypes.c_int]
    L.gdn_last_hip_error.restype = ctypes.c_char_p
    L.gdn_last_hip_error.argtypes = []
    for f in ("gdn_rec_state_bytes", "gdn_conv_state_bytes", "gdn_state_blob_bytes",
              "gdn_decode_workspace_bytes"):
        getattr(L, f).restype = sz
        getattr(L, f).argtypes = [dp]
    L.gdn_prefill_workspace_bytes.restype = sz
    L.gdn_prefill_workspace_bytes.argtypes = [dp, i64, i32]
    L.gdn_conv1d.restype = ctypes.c_int
    L.gdn_conv1d.argtypes = [dp, i64, vp, vp, vp, vp, vp]
    L.gdn_prefill_chunked.restype = ctypes.c_int
    L.gdn_prefill_chunked.argtypes = [dp, i64, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.gdn_decode_step.restype = ctypes.c_int
    L.gdn_decode_step.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.gdn_prefill_chunked_timed.restype = ctypes.c_int
    L.gdn_prefill_chunked_timed.argtypes = L.gdn_prefill_chunked.argtypes + [vp]
    L.gdn_decode_step_timed.restype = ctypes.c_int
    L.gdn_decode_step_timed.argtypes = L.gdn_decode_step.argtypes + [vp]
    L.gdn_decode_multi.restype = ctypes.c_int
    L.gdn_decode_multi.argtypes = [dp, i32, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, sz, vp]
    L.gdn_prefill_varlen_workspace_bytes.restype = sz
    L.gdn_prefill_varlen_workspace_bytes.argtypes = [dp, vp, i32]
    L.gdn_prefill_varlen.restype = ctypes.c_int
    L.gdn_prefill_varlen.argtypes = [dp, vp, i32, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, sz,
                                     vp]
    ap = ctypes.POINTER(GdnAttnDims)
    L.gdn_attn_workspace_bytes.restype = sz
    L.gdn_attn_workspace_bytes.argtypes = [ap, i64, i64]
    L.gdn_attn_prefill.restype = ctypes.c_int
    L.gdn_attn_prefill.argtypes = [ap, i64, i64, vp, vp, vp, vp, vp, i64, vp, vp, sz, vp]
    L.gdn_in_proj.restype = ctypes.c_int
    L.gdn_in_proj.argtypes = [dp, i64, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.gdn_gated_rmsnorm.restype = ctypes.c_int
    L.gdn_gated_rmsnorm.argtypes = [dp, i64, vp, vp, vp, ctypes.c_float, vp, vp]
    L.gdn_decode_step_noalloc.restype = ctypes.c_int
    L.gdn_decode_step_noalloc.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.gdn_state_save.restype = ctypes.c_int
    L.gdn_state_save.argtypes = [dp, vp, vp, vp, sz, vp]
    L.gdn_state_restore.restype = ctypes.c_int
    L.gdn_state_restore.argtypes = [dp, vp, sz, vp, vp, vp]
    L.gdn_state_check.restype = ctypes.c_int
    L.gdn_state_check.argtypes = [dp, vp, sz]
    if L.gdn_abi_version() != ABI_VERSION:
        raise RuntimeError("libgdn.so ABI version mismatch")
    _LIB = L
    return L


def check(status: int, where: str) -> None:
    if status != GDN_OK:
        detail = ""
        if status == -11:
            detail = load().gdn_last_hip_error().decode()
        raise GdnError(status, where, detail)
