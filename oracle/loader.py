"""Build and load the oracle shared library (plain g++, no HIP)."""
from __future__ import annotations

import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "tmoe_oracle.cpp")
LIB = os.path.join(HERE, "libtmoe_oracle.so")

_lib = None


def build(verbose: bool = False) -> str:
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
           "-ffp-contract=off", "-o", LIB + ".tmp", SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def _sig(lib):
    c = ctypes
    P = c.c_void_p
    lib.orc_codebook_fp16.argtypes = [c.c_uint16]
    lib.orc_codebook_fp16.restype = c.c_uint16
    lib.orc_half_to_double.argtypes = [c.c_uint16]
    lib.orc_half_to_double.restype = c.c_double
    lib.orc_double_to_half.argtypes = [c.c_double]
    lib.orc_double_to_half.restype = c.c_uint16
    lib.orc_double_to_e4m3.argtypes = [c.c_double]
    lib.orc_double_to_e4m3.restype = c.c_uint8
    lib.orc_e4m3_to_double.argtypes = [c.c_uint8]
    lib.orc_e4m3_to_double.restype = c.c_double
    lib.orc_mx_exponent.argtypes = [c.c_float]
    lib.orc_mx_exponent.restype = c.c_int
    lib.orc_hardware_threads.argtypes = []
    lib.orc_hardware_threads.restype = c.c_int
    lib.orc_decode_tile_bitwise.argtypes = [P, c.c_int, P]
    lib.orc_decode_tile_bitwise.restype = None
    lib.orc_decode_tile_shiftreg.argtypes = [P, c.c_int, P]
    lib.orc_decode_tile_shiftreg.restype = None
    lib.orc_decode_matrix.argtypes = [P, c.c_int, c.c_int, c.c_int, P]
    lib.orc_decode_matrix.restype = None
    lib.orc_hadamard_explicit.argtypes = [c.c_int, P]
    lib.orc_hadamard_explicit.restype = c.c_int
    lib.orc_rotate_rows.argtypes = [P, c.c_int64, c.c_int, c.c_int]
    lib.orc_rotate_rows.restype = c.c_int
    lib.orc_route_map.argtypes = [P, c.c_int64, c.c_int, c.c_int] + [P] * 9
    lib.orc_route_map.restype = c.c_int
    lib.orc_mxfp8_quantize.argtypes = [P, c.c_int64, c.c_int, P, P]
    lib.orc_mxfp8_quantize.restype = c.c_int
    lib.orc_forward.argtypes = [c.c_int] * 5 + [P] * 11 + [c.c_int, c.c_int, c.c_int, P]
    lib.orc_forward.restype = c.c_int
    lib.orc_route_trace.argtypes = ([c.c_int] * 5 + [P] * 10 + [c.c_int] * 4 + [P] * 6)
    lib.orc_route_trace.restype = c.c_int
    lib.orc_linear.argtypes = [c.c_int] * 4 + [P] * 5 + [c.c_int, P]
    lib.orc_linear.restype = c.c_int
    return lib


def load(rebuild_if_missing: bool = True):
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB) or (rebuild_if_missing and os.path.getmtime(LIB) < os.path.getmtime(SRC)):
        build()
    _lib = _sig(ctypes.CDLL(LIB))
    return _lib
