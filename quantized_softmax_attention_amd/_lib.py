"""ctypes view of libkia.so: the structs and signatures of include/kia.h.

Loading fails loudly when the library has not been built; there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkia.so")


class KiaParams(ctypes.Structure):
    _fields_ = [("n_intervals", c_int32), ("tau", c_float), ("calibration", c_int32),
                ("reconstruction", c_int32), ("surrogate", c_int32), ("grad_rule", c_int32)]


class KiaStatsLayout(ctypes.Structure):
    _fields_ = [("total_bytes", c_size_t), ("scores", c_size_t), ("row_m", c_size_t),
                ("row_n", c_size_t), ("row_a", c_size_t), ("row_b", c_size_t),
                ("row_w", c_size_t), ("row_wl", c_size_t), ("o_lerp", c_size_t),
                ("tiles_per_head", c_int64)]


class KiaWorkspaceLayout(ctypes.Structure):
    _fields_ = [("total_bytes", c_size_t), ("probs", c_size_t), ("dscores", c_size_t),
                ("row_cm", c_size_t), ("row_cn", c_size_t), ("prefix_k", c_size_t), ("chunk_k", c_size_t)]


class KiaExt(ctypes.Structure):
    _fields_ = [("events", POINTER(c_void_p)), ("n_events", c_int32), ("idx_dump", c_void_p)]


P = POINTER(KiaParams)
_SHAPE = [c_int, c_int, c_int, c_int]

# name -> (restype, argtypes); every function include/kia.h declares
SIGNATURES = {
    "kia_stats_bytes": (c_size_t, [P] + _SHAPE),
    "kia_workspace_bytes": (c_size_t, [P] + _SHAPE),
    "kia_stats_layout_query": (c_int, [P] + _SHAPE + [POINTER(KiaStatsLayout)]),
    "kia_workspace_layout_query": (c_int, [P] + _SHAPE + [POINTER(KiaWorkspaceLayout)]),
    "kia_forward": (c_int, [P] + _SHAPE + [c_void_p] * 5 + [c_size_t, c_void_p]),
    "kia_backward": (c_int, [P] + _SHAPE + [c_void_p] * 6 + [c_size_t] + [c_void_p] * 4
                     + [c_size_t, c_void_p]),
    "kia_forward_ext": (c_int, [P] + _SHAPE + [c_void_p] * 5 + [c_size_t, c_void_p, POINTER(KiaExt)]),
    "kia_backward_ext": (c_int, [P] + _SHAPE + [c_void_p] * 6 + [c_size_t] + [c_void_p] * 4
                         + [c_size_t, c_void_p, POINTER(KiaExt)]),
    "kia_backward_noalloc": (c_int, [P] + _SHAPE + [c_void_p] * 6 + [c_size_t] + [c_void_p] * 4),
    "kia_geometry_bytes": (c_size_t, [c_int, c_int, c_int]),
    "kia_geometry": (c_int, [P] + _SHAPE + [c_void_p] * 3 + [c_size_t, c_void_p, c_size_t, c_void_p]),
    "kia_tiles_to_dense": (c_int, [c_int, c_int, c_int, c_void_p, c_int, c_void_p, c_void_p]),
    "kia_status_str": (c_char_p, [c_int]),
    "kia_abi_version": (c_int32, []),
}

_lib = None


def load():
    """Load libkia.so (once) and attach the signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"libkia.so is not built ({LIB_PATH}); build it with "
            "`python -m quantized_softmax_attention_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
