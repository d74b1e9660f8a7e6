"""ctypes binding of libtmoe.so (the C ABI in include/tmoe.h). Argument marshalling only.

There is no fallback: if the HIP library is not built this module raises on import, so nothing
can silently run another implementation."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtmoe.so")

TMOE_OK = 0
STATUS_NAMES = {0: "TMOE_OK", 1: "TMOE_ERR_INVALID_ARG", 2: "TMOE_ERR_UNSUPPORTED", 3: "TMOE_ERR_SCRATCH",
                4: "TMOE_ERR_CAPACITY", 5: "TMOE_ERR_ALIGNMENT", 6: "TMOE_ERR_HIP",
                7: "TMOE_ERR_STATIC_SCRATCH"}
STATIC_SCRATCH_BYTES = 32 << 20
ROT_HADAMARD, ROT_IDENTITY = 0, 1
FC2_DETERMINISTIC, FC2_ATOMIC = 0, 1
IDS_I32, IDS_I64 = 0, 1

# every symbol declared in include/tmoe.h
EXPORTS = ["tmoe_plan", "tmoe_plan_destroy", "tmoe_plan_get_info", "tmoe_plan_expert_offset",
           "tmoe_build_route_map", "tmoe_forward_w4a16", "tmoe_forward_w4a8", "tmoe_forward_w4a16_static",
           "tmoe_forward_stages",
           "tmoe_status_str",
           "tmoe_debug_decode", "tmoe_debug_mxfp8", "tmoe_debug_rotate", "tmoe_debug_get_views",
           "tmoe_linear_plan", "tmoe_linear_plan_destroy", "tmoe_linear_w4a16"]


class Config(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("max_tokens", ctypes.c_int32),
                ("expert_bits", ctypes.POINTER(ctypes.c_uint8)), ("rotation", ctypes.c_int32),
                ("ids_dtype", ctypes.c_int32), ("block_m", ctypes.c_int32),
                ("smallm_max_tokens", ctypes.c_int32), ("fc2_reduce", ctypes.c_int32)]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("payload", "scale1", "scale2", "su1", "sv1", "su2", "sv2")]


class RouteMap(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("counts", "offsets", "sorted_routes", "route_slot",
                                               "tile_expert", "tile_row0", "tile_rows", "num_tiles",
                                               "status")] + \
               [("max_tiles", ctypes.c_int32), ("block_m", ctypes.c_int32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("scratch_bytes", ctypes.c_size_t), ("payload_words", ctypes.c_size_t),
                ("block_m", ctypes.c_int32), ("max_tiles", ctypes.c_int32)]


class DebugViews(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("a1", "a1_scale", "z", "b", "b_scale", "v", "splits")] + \
               [("a1_pitch", ctypes.c_int32), ("b_pitch", ctypes.c_int32), ("arm_status", ctypes.c_void_p),
                ("half_planes", ctypes.c_void_p)]


class LinearConfig(ctypes.Structure):
    _fields_ = [("in_features", ctypes.c_int32), ("out_features", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("max_tokens", ctypes.c_int32), ("rotation", ctypes.c_int32)]


class LinearWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("payload", "scale", "su", "sv")]


class TmoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}")
        self.status = status


def _load():
    # torch ships its own HIP runtime library. Loading it first makes libtmoe.so bind to that same
    # runtime (same soname), so device pointers and streams from torch are valid for our launches;
    # loading libtmoe.so first would pull in a second runtime from the system ROCm.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.tmoe_plan.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(P), ctypes.POINTER(SZ), ctypes.POINTER(SZ)]
    lib.tmoe_plan_destroy.argtypes = [P]
    lib.tmoe_plan_get_info.argtypes = [P, ctypes.POINTER(PlanInfo)]
    lib.tmoe_plan_expert_offset.argtypes = [P, I32, ctypes.POINTER(SZ)]
    lib.tmoe_build_route_map.argtypes = [P, P, I32, P, SZ, ctypes.POINTER(RouteMap), P]
    fwd = [P, P, P, P, I32, ctypes.POINTER(Weights), P, P, SZ, P]
    lib.tmoe_forward_w4a16.argtypes = fwd
    lib.tmoe_forward_w4a8.argtypes = fwd
    lib.tmoe_forward_w4a16_static.argtypes = [P, P, P, P, I32, ctypes.POINTER(Weights), P, P]
    lib.tmoe_forward_stages.argtypes = [P, I32, I32, I32, P, P, P, I32, ctypes.POINTER(Weights), P, P, SZ, P]
    lib.tmoe_status_str.argtypes = [I32]
    lib.tmoe_status_str.restype = ctypes.c_char_p
    lib.tmoe_debug_decode.argtypes = [P, ctypes.POINTER(Weights), I32, I32, I32, P, P]
    lib.tmoe_debug_mxfp8.argtypes = [P, I64, I32, P, P, P]
    lib.tmoe_debug_rotate.argtypes = [P, I64, I32, P]
    lib.tmoe_debug_get_views.argtypes = [P, I32, I32, P, SZ, ctypes.POINTER(DebugViews)]
    lib.tmoe_linear_plan.argtypes = [ctypes.POINTER(LinearConfig), ctypes.POINTER(P), ctypes.POINTER(SZ),
                                     ctypes.POINTER(SZ)]
    lib.tmoe_linear_plan_destroy.argtypes = [P]
    lib.tmoe_linear_w4a16.argtypes = [P, P, I32, ctypes.POINTER(LinearWeights), P, P, SZ, P]
    for name in EXPORTS:
        if name != "tmoe_status_str":
            getattr(lib, name).restype = I32
    return lib


lib = _load()


def check(status: int, where: str) -> None:
    if status != TMOE_OK:
        raise TmoeError(status, where)
