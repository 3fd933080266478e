"""ctypes loader for libmoe_routing.so: argument and return types of every
entry point declared in include/moe_routing.h.  No compute happens here."""
from __future__ import annotations

import ctypes
import os
import re

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libmoe_routing.so")
HEADER = os.path.join(os.path.dirname(PKG_DIR), "include", "moe_routing.h")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_HIP, MOE_ERR_WORKSPACE, MOE_ERR_SCRATCH_LIMIT = range(6)
MOE_F32, MOE_BF16, MOE_MXFP4, MOE_BF16_TILED = range(4)
MOE_MXFP4_MMA_BF16, MOE_MXFP4_MMA_F8F6F4 = 0, 1

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t
_int = ctypes.c_int

SIGNATURES = {
    "moe_topk_softmax": (_int, [_p, _int, _i64, _i32, _i32, _i32, _p, _p, _p, _p]),
    "moe_topk_sigmoid": (_int, [_p, _int, _i64, _i32, _i32, _i32, _p, _p, _p, _p]),
    "moe_route_compact": (_int, [_p, _i64, _i32, _p, _i32, _i32, _p, _p, _p, _p, _p, _sz, _p]),
    "moe_route_compact_workspace_bytes": (_sz, [_i64, _i32, _i32]),
    "moe_topk_compact": (_int, [_p, _int, _i64, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _i32, _p, _p, _p, _p, _p,
                                _sz, _p]),
    "moe_route_align": (_int, [_p, _i64, _i32, _p, _i32, _i32, _i32, _p, _p, _p, _p, _p, _sz, _p]),
    "moe_route_align_workspace_bytes": (_sz, [_i64, _i32, _i32]),
    "moe_grouped_ffn": (_int, [_p, _int, _i64, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _int, _p, _p, _p, _p, _int,
                               _p, _sz, _p]),
    "moe_grouped_ffn_workspace_bytes": (_sz, [_i64, _i32, _i32, _i32, _i32, _int]),
    "moe_grouped_ffn_noalloc": (_int, [_p, _int, _i64, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _int, _p, _p, _p, _p,
                                       _int, _p]),
    "moe_grouped_ffn_control": (_int, [_p, _int, _i64, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _int, _p, _p, _p, _p,
                                       _int, _p, _sz, _p]),
    "moe_grouped_ffn_control_workspace_bytes": (_sz, [_i64, _i32, _i32, _i32, _i32, _int]),
    "moe_combine": (_int, [_p, _int, _p, _p, _i64, _i32, _i32, _p, _int, _p]),
    "moe_pack_ffn_weights": (_int, [_p, _p, _i32, _i32, _i32, _p, _p, _p]),
    "moe_fused_experts": (_int, [_p, _int, _i64, _i32, _i32, _i32, _p, _p, _p, _i32, _i32, _p, _p, _p, _p, _int,
                                 _p, _p, _p, _p, _p, _int, _p, _sz, _p]),
    "moe_fused_experts_workspace_bytes": (_sz, [_i64, _i32, _i32, _i32, _i32, _int]),
    "moe_probe_read": (_int, [_p, _sz, _p, _sz, _p]),
    "moe_probe_copy": (_int, [_p, _p, _sz, _p]),
    "moe_probe_mfma": (_int, [_i64, _i32, _p, _p]),
    "moe_probe_mfma_clock": (_int, [_i64, _i32, _i32, _p, _p, _p]),
    "moe_probe_gate_loads": (_int, [_p, _i64, _i32, _i32, _p, _p, _p, _p]),
    "moe_set_mxfp4_mma": (_int, [_int]),
    "moe_get_mxfp4_mma": (_int, []),
    "moe_status_string": (ctypes.c_char_p, [_int]),
    "moe_last_hip_error": (_int, []),
    "moe_version": (ctypes.c_char_p, []),
}

_lib = None


def header_symbols(path: str = HEADER):
    """Function names declared in the public header."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def load():
    """Load the in-tree library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -m mixture_experts_routing_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().moe_status_string(code).decode()
