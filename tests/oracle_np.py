"""numpy-facing wrappers around the float64 oracle library (test infrastructure)."""
from __future__ import annotations

import ctypes

import numpy as np

import oracle


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def lib():
    return oracle.load()


def codebook(state: int) -> int:
    return int(lib().orc_codebook_fp16(state))


def half_to_double(h: int) -> float:
    return float(lib().orc_half_to_double(h))


def decode_tile(words: np.ndarray, bits: int, method: str = "shiftreg") -> np.ndarray:
    w = np.ascontiguousarray(words, dtype=np.uint16)
    assert w.size == 16 * bits
    out = np.zeros(256, np.uint16)
    fn = lib().orc_decode_tile_shiftreg if method == "shiftreg" else lib().orc_decode_tile_bitwise
    fn(_p(w), bits, _p(out))
    return out


def decode_matrix(words: np.ndarray, bits: int, K: int, N: int) -> np.ndarray:
    """fp16 codebook values (uint16 bit patterns) of a K x N trellis matrix, row-major."""
    w = np.ascontiguousarray(words, dtype=np.uint16)
    out = np.zeros((K, N), np.uint16)
    lib().orc_decode_matrix(_p(w), bits, K, N, _p(out))
    return out


def expert_codes(inp, e: int):
    """(C1 [H, 2I], C2 [I, H]) fp16 bit patterns of expert e."""
    H, I = inp.hidden, inp.inter
    off = inp.payload_offsets()
    b = int(inp.bits[e])
    base = inp.payload[off[e]:off[e + 1]]
    n1 = H * 2 * I * b // 16
    return decode_matrix(base[:n1], b, H, 2 * I), decode_matrix(base[n1:], b, I, H)


def hadamard_explicit(n: int) -> np.ndarray:
    out = np.zeros((n, n), np.float64)
    rc = lib().orc_hadamard_explicit(n, _p(out))
    assert rc == 0
    return out


def rotate_rows(v: np.ndarray, identity: bool = False) -> np.ndarray:
    a = np.ascontiguousarray(v, dtype=np.float64).copy()
    rows = a.size // a.shape[-1]
    rc = lib().orc_rotate_rows(_p(a), rows, a.shape[-1], int(identity))
    assert rc == 0
    return a


def route_map(ids: np.ndarray, E: int, block_m: int):
    ids64 = np.ascontiguousarray(ids, dtype=np.int64).reshape(-1)
    R = ids64.size
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    sorted_routes = np.full(max(R, 1), -7, np.int32)
    route_slot = np.full(max(R, 1), -7, np.int32)
    max_tiles = R // block_m + E + 1
    tile_expert = np.full(max_tiles, -7, np.int32)
    tile_row0 = np.full(max_tiles, -7, np.int32)
    tile_rows = np.full(max_tiles, -7, np.int32)
    num_tiles = np.zeros(1, np.int32)
    invalid = np.zeros(1, np.int32)
    rc = lib().orc_route_map(_p(ids64), R, E, block_m, _p(counts), _p(offsets), _p(sorted_routes),
                             _p(route_slot), _p(tile_expert), _p(tile_row0), _p(tile_rows),
                             _p(num_tiles), _p(invalid))
    assert rc == 0
    valid = int(offsets[-1])
    nt = int(num_tiles[0])
    return dict(counts=counts, offsets=offsets, sorted_routes=sorted_routes[:valid],
                route_slot=route_slot[:R], tile_expert=tile_expert[:nt], tile_row0=tile_row0[:nt],
                tile_rows=tile_rows[:nt], num_tiles=nt, invalid=int(invalid[0]))


def mxfp8_quantize(x: np.ndarray):
    a = np.ascontiguousarray(x, dtype=np.float64)
    rows, cols = a.shape
    q = np.zeros((rows, cols), np.uint8)
    e = np.zeros((rows, cols // 32), np.uint8)
    rc = lib().orc_mxfp8_quantize(_p(a), rows, cols, _p(q), _p(e))
    assert rc == 0
    return q, e


def _layer_args(inp):
    arrs = [np.ascontiguousarray(inp.bits, np.uint8), np.ascontiguousarray(inp.payload, np.uint16)]
    for name in ("scale1", "scale2", "su1", "sv1", "su2", "sv2"):
        arrs.append(np.ascontiguousarray(getattr(inp, name)).view(np.uint16))
    arrs.append(np.ascontiguousarray(inp.x_bf16, np.uint16))
    arrs.append(np.ascontiguousarray(inp.ids, np.int64))
    return arrs


def forward(inp, mode: str = "w4a16", identity: bool = False, nthreads: int = 0) -> np.ndarray:
    arrs = _layer_args(inp)
    w = np.ascontiguousarray(inp.weights, np.float32)
    y = np.zeros((inp.tokens, inp.hidden), np.float64)
    rc = lib().orc_forward(inp.tokens, inp.hidden, inp.inter, inp.experts, inp.top_k,
                           *[_p(a) for a in arrs], _p(w), 1 if mode == "w4a8" else 0,
                           int(identity), nthreads, _p(y))
    assert rc == 0, rc
    return y


def route_trace(inp, t: int, j: int, mode: str = "w4a16", identity: bool = False) -> dict:
    arrs = _layer_args(inp)
    H, I = inp.hidden, inp.inter
    out = dict(a=np.zeros(H), z=np.zeros(2 * I), h=np.zeros(I), b=np.zeros(I), v=np.zeros(H),
               o=np.zeros(H))
    rc = lib().orc_route_trace(inp.tokens, H, I, inp.experts, inp.top_k, *[_p(a) for a in arrs],
                               1 if mode == "w4a8" else 0, int(identity), t, j,
                               *[_p(out[k]) for k in ("a", "z", "h", "b", "v", "o")])
    assert rc == 0, rc
    return out


def linear(inp, identity: bool = False) -> np.ndarray:
    """The oracle's dense trellis linear (reading R8): y = sv * R_N(scale * (C^T R_K(su * x)))."""
    y = np.zeros((inp.tokens, inp.out_features), np.float64)
    arrs = [np.ascontiguousarray(inp.payload, np.uint16), np.ascontiguousarray(inp.scale).view(np.uint16),
            np.ascontiguousarray(inp.su).view(np.uint16), np.ascontiguousarray(inp.sv).view(np.uint16),
            np.ascontiguousarray(inp.x_bf16, np.uint16)]
    rc = lib().orc_linear(inp.tokens, inp.in_features, inp.out_features, inp.bits, *[_p(a) for a in arrs],
                          int(identity), _p(y))
    assert rc == 0, rc
    return y
