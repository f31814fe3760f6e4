"""ctypes view of the C ABI declared in include/moe.h.

Loading fails loudly if the built library is missing: there is no fallback
implementation of any step in Python.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "lib", "libqmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARGUMENT = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE_TOO_SMALL = 3
MOE_ERR_HIP = 4

MOE_Q4_SYM = 0
MOE_Q4_ASYM = 1

MOE_W_ROWS = 0
MOE_W_TILED = 1

MOE_WS_LAYER = 0
MOE_WS_ROUTE = 1
MOE_WS_PERMUTE = 2
MOE_WS_EXPERT_FFN = 3
MOE_WS_LAYER_I8 = 4
MOE_WS_EXPERT_FFN_I8 = 5

MOE_STATIC_WS_BYTES = 128 << 20   # the static workspace of moe_layer_forward_static

# Every symbol include/moe.h declares.
EXPORTED = [
    "moe_abi_version",
    "moe_last_error",
    "moe_workspace_size",
    "moe_route",
    "moe_permute",
    "moe_expert_ffn",
    "moe_combine",
    "moe_layer_forward",
    "moe_layer_forward_static",
    "moe_quantize_rows_i8",
    "moe_expert_ffn_i8",
    "moe_layer_forward_i8",
    "moe_expert_ffn_mixed",
    "moe_layer_forward_mixed",
    "moe_stream_stage_bytes",
    "moe_layer_forward_streamed",
    "moe_pack_w4",
    "moe_pack_tier",
    "moe_rmsnorm",
    "moe_profile_enable",
    "moe_profile_reset",
    "moe_profile_read",
]


class MoeShape(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int64),
        ("num_experts", ctypes.c_int64),
        ("top_k", ctypes.c_int64),
        ("inter", ctypes.c_int64),
        ("group_size", ctypes.c_int64),
        ("quant", ctypes.c_int32),
        ("w_layout", ctypes.c_int32),
        ("shared_inter", ctypes.c_int64),
    ]


class MoeExperts(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "w13", "w13_scale", "w13_min", "w2", "w2_scale", "w2_min",
        "s13", "s13_scale", "s13_min", "s2", "s2_scale", "s2_min")]


class MoeTier(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("w13", ctypes.c_void_p), ("w13_scale", ctypes.c_void_p),
                ("w2", ctypes.c_void_p), ("w2_scale", ctypes.c_void_p)]


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"status {status}: {msg}")
        self.status = status


_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m quantized_moe_prefill_amd.build` "
            "(or __graft_entry__.build()); there is no non-HIP implementation")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    i64 = ctypes.c_int64
    i32 = ctypes.c_int32
    st = ctypes.c_int
    sp = ctypes.POINTER(MoeShape)
    ep = ctypes.POINTER(MoeExperts)
    L.moe_abi_version.restype = ctypes.c_int
    L.moe_abi_version.argtypes = []
    L.moe_last_error.restype = ctypes.c_char_p
    L.moe_last_error.argtypes = []
    L.moe_workspace_size.restype = st
    L.moe_workspace_size.argtypes = [sp, i64, i32, ctypes.POINTER(ctypes.c_size_t)]
    L.moe_route.restype = st
    L.moe_route.argtypes = [sp, i64, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    L.moe_permute.restype = st
    L.moe_permute.argtypes = [sp, i64, P, P, P, P, P, P, ctypes.c_size_t, P]
    L.moe_expert_ffn.restype = st
    L.moe_expert_ffn.argtypes = [sp, i64, P, ep, P, P, P, P, P, P, ctypes.c_size_t, P]
    L.moe_combine.restype = st
    L.moe_combine.argtypes = [sp, i64, P, P, P, P, P, P, P, P]
    L.moe_layer_forward.restype = st
    L.moe_layer_forward.argtypes = [sp, i64, P, P, P, P, ep, P, P, P, ctypes.c_size_t, P]
    L.moe_layer_forward_static.restype = st
    L.moe_layer_forward_static.argtypes = [sp, i64, P, P, P, P, ep, P, P, P]
    L.moe_quantize_rows_i8.restype = st
    L.moe_quantize_rows_i8.argtypes = [i64, i64, P, P, P, P]
    L.moe_expert_ffn_i8.restype = st
    L.moe_expert_ffn_i8.argtypes = [sp, i64, P, ep, P, P, P, P, P, P, ctypes.c_size_t, P]
    L.moe_layer_forward_i8.restype = st
    L.moe_layer_forward_i8.argtypes = [sp, i64, P, P, P, ep, P, P, P, ctypes.c_size_t, P]
    tp = ctypes.POINTER(MoeTier)
    L.moe_expert_ffn_mixed.restype = st
    L.moe_expert_ffn_mixed.argtypes = [sp, i64, P, tp, i32, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    L.moe_layer_forward_mixed.restype = st
    L.moe_layer_forward_mixed.argtypes = [sp, i64, P, P, P, tp, i32, P, P, P, P, P,
                                          ctypes.c_size_t, P]
    L.moe_stream_stage_bytes.restype = st
    L.moe_stream_stage_bytes.argtypes = [sp, i32, ctypes.POINTER(ctypes.c_size_t)]
    L.moe_layer_forward_streamed.restype = st
    L.moe_layer_forward_streamed.argtypes = [sp, i64, P, P, P, ep, i32, ep, P, P, ctypes.c_size_t,
                                             P, P, P, ctypes.c_size_t, P, P]
    L.moe_pack_w4.restype = st
    L.moe_pack_w4.argtypes = [P, P, i64, i64, P]
    L.moe_pack_tier.restype = st
    L.moe_pack_tier.argtypes = [P, P, i64, i64, i32, i32, P]
    L.moe_rmsnorm.restype = st
    L.moe_rmsnorm.argtypes = [i64, i64, P, P, ctypes.c_float, P, P]
    L.moe_profile_enable.restype = st
    L.moe_profile_enable.argtypes = [i32]
    L.moe_profile_reset.restype = st
    L.moe_profile_reset.argtypes = []
    L.moe_profile_read.restype = st
    L.moe_profile_read.argtypes = [ctypes.c_char_p, ctypes.POINTER(i64),
                                   ctypes.POINTER(ctypes.c_double)]
    _lib = L
    return L


def check(status: int):
    if status != MOE_OK:
        msg = lib().moe_last_error().decode(errors="replace")
        raise MoeError(status, msg)
