"""ctypes loader for libw4a16_moe.so (the gfx950 HIP library).

There is no fallback: if the library is missing this raises, and every layer
computation happens in the library's HIP kernels.
"""
from __future__ import annotations

import ctypes
import os

# W4A16_MOE_LIB may point at another build of the same library (A/B timing)
LIB_PATH = os.environ.get("W4A16_MOE_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                            "libw4a16_moe.so")

_lib = None

# name -> (restype, argtypes); mirrors include/w4a16_moe.h
P = ctypes.c_void_p
I32 = ctypes.c_int32
SZ = ctypes.c_size_t
SIGNATURES = {
    "w4a16_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "w4a16_packed_bytes": (ctypes.c_int, [P, ctypes.POINTER(SZ), ctypes.POINTER(SZ)]),
    "w4a16_repack": (ctypes.c_int, [P, P, P, P, P, P, P, P]),
    "moe_align_capacity": (SZ, [I32, I32, I32, I32]),
    "moe_align_workspace_bytes": (SZ, [I32, I32, I32, I32]),
    "w4a16_choose_block_m": (I32, [I32, I32, I32, I32]),
    "moe_align": (ctypes.c_int, [P, I32, I32, I32, I32, P, I32, P, P, P, P, SZ, P]),
    "moe_align_filtered": (ctypes.c_int, [P, I32, I32, I32, I32, I32, I32, P, I32, P, P, P, P, SZ, P]),
    "moe_align_split": (ctypes.c_int, [P, I32, I32, I32, I32, I32, I32, P, P, I32, I32, P, P, P, P, SZ, P]),
    "w4a16_moe_routed_workspace_bytes": (SZ, [P, I32, I32, I32]),
    "w4a16_moe_routed_split": (I32, [P, I32, I32, I32]),
    "w4a16_moe_routed_forward": (ctypes.c_int, [P, P, I32, I32, I32, P, P, P, P, P, P, SZ, P]),
    "w4a16_moe_routed_forward_noalloc": (ctypes.c_int, [P, P, I32, I32, I32, P, P, P, P, P, P]),
    "moe_route_align": (ctypes.c_int, [P, P, I32, I32, I32, I32, I32, P, P, P, I32, P, P, P, P, SZ, P]),
    "w4a16_moe_contiguous_workspace_bytes": (SZ, [P, I32]),
    "w4a16_moe_contiguous_forward": (ctypes.c_int, [P, P, I32, P, P, P, P, P, SZ, P]),
    "w4a16_moe_masked_block_m": (I32, [I32, I32]),
    "w4a16_moe_masked_workspace_bytes": (SZ, [P, I32, I32]),
    "w4a16_moe_masked_forward": (ctypes.c_int, [P, P, I32, P, I32, P, P, P, P, SZ, P]),
    "w4a16_moe_workspace_bytes": (SZ, [P, I32, I32, I32]),
    "w4a16_moe_stage_workspace_bytes": (SZ, [P, I32, I32, I32]),
    "w4a16_moe_forward": (ctypes.c_int, [P, P, I32, I32, P, P, P, I32, P, P, I32, P, P, P, P, SZ, P]),
    "w4a16_moe_prepare_x": (ctypes.c_int, [P, P, I32, I32, P, I32, P, SZ, P]),
    "w4a16_moe_gate_up": (ctypes.c_int, [P, P, I32, I32, P, I32, P, P, I32, P, P, P, SZ, P]),
    "w4a16_moe_prepare_h": (ctypes.c_int, [P, I32, I32, P, P, I32, P, I32, P, SZ, P]),
    "w4a16_moe_down": (ctypes.c_int, [P, I32, I32, P, P, I32, P, P, I32, P, P, P, SZ, P]),
    "w4a16_moe_combine": (ctypes.c_int, [P, I32, I32, P, P, P, P, P]),
}


def load():
    """Load the library (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m w4a16_grouped_gemm_amd.build` "
                "(the W4A16 MoE layer has no CPU or fallback path)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class Shape(ctypes.Structure):
    """w4a16_moe_shape."""
    _fields_ = [("num_experts", I32), ("hidden", I32), ("intermediate", I32), ("group_size", I32)]
