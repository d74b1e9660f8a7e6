"""Seeded synthetic inputs for the trellis-quantized routed MoE layer.

This module only draws random inputs. It holds none of the layer's arithmetic
(no decode, no rotation, no GEMM), so both the HIP path and the float64 CPU
reference can be fed from it without sharing any of the method.

Geometries follow the workloads described on the pages:
  * "serve canonical Fruit QSRT atoms" (b12x PR #129, Summary): H=1024, I=512;
  * "integrate EXL3 Trellis into the fused W4A16 API" (sparkinfer PR #90):
    trellis3_t256 tiles of 256 weights stored as 16*bits 16-bit words;
  * "TrellisMX (procedural NPK) ... P8 runtime" (flashinfer PR #69, commit
    list): the synthetic H2560/I320/top-k10 rank geometry.

Draw order (fixed, so a seed names one input set):
  expert bits -> payload words -> scale1, scale2 -> su1, sv1, su2, sv2 -> x
  -> ids -> routing logits -> weights = fp32(softmax(logits)).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

# name -> (H, I, E, top_k, token counts, bit choices, routing, x_sigma, outliers, path)
GEOMETRIES = {
    "tiny":    dict(hidden=256,  inter=128, experts=8,   top_k=2,  tokens=(4,),
                    bits=(4,), routing="uniform", x_sigma=1.0, outliers=False, path="w4a16"),
    "decode":  dict(hidden=1024, inter=512, experts=96,  top_k=8,  tokens=(1, 4, 16),
                    bits=(4,), routing="uniform", x_sigma=1.0, outliers=False, path="w4a16"),
    "prefill": dict(hidden=1024, inter=512, experts=96,  top_k=8,  tokens=(2048,),
                    bits=(4,), routing="zipf", x_sigma=1.0, outliers=False, path="w4a16"),
    "wide":    dict(hidden=2560, inter=320, experts=128, top_k=10, tokens=(16, 512),
                    bits=(2, 3, 4), routing="uniform", x_sigma=1.0, outliers=False, path="w4a16"),
    "w4a8":    dict(hidden=1024, inter=512, experts=256, top_k=8,  tokens=(1, 8, 32, 64),
                    bits=(4,), routing="uniform", x_sigma=float(np.sqrt(2.0)), outliers=True,
                    path="w4a8"),
}
GEOMETRY_INDEX = {"tiny": 0, "decode": 1, "prefill": 2, "wide": 3, "w4a8": 4}
ZIPF_S = 1.1
OUTLIER_P = 0.01
OUTLIER_GAIN = 20.0


def payload_words_per_expert(hidden: int, inter: int, bits: int) -> int:
    """16-bit words of one expert: FC1 (H x 2I) then FC2 (I x H), 16*bits words per 16x16 tile."""
    tiles = (hidden // 16) * (2 * inter // 16) + (inter // 16) * (hidden // 16)
    return tiles * 16 * bits


def payload_offsets(hidden: int, inter: int, bits) -> np.ndarray:
    """Word offset of each expert's region; experts are concatenated in index order."""
    sizes = [payload_words_per_expert(hidden, inter, int(b)) for b in bits]
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)


def bf16_bits_from_f32(v: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16, returned as uint16 bit patterns (finite inputs)."""
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class LayerInputs:
    """One seeded input set. All arrays are host numpy arrays in the layout the C ABI expects."""
    name: str
    seed: int
    hidden: int
    inter: int
    experts: int
    top_k: int
    tokens: int
    bits: np.ndarray          # uint8 [E]
    payload: np.ndarray       # uint16 [total words]
    scale1: np.ndarray        # float16 [E, 2I]
    scale2: np.ndarray        # float16 [E, H]
    su1: np.ndarray           # float16 [E, H]
    sv1: np.ndarray           # float16 [E, 2I]
    su2: np.ndarray           # float16 [E, I]
    sv2: np.ndarray           # float16 [E, H]
    x_bf16: np.ndarray        # uint16 [T, H] bf16 bit patterns
    ids: np.ndarray           # int64 [T, k]
    weights: np.ndarray       # float32 [T, k]

    @property
    def routes(self) -> int:
        return self.tokens * self.top_k

    def payload_offsets(self) -> np.ndarray:
        return payload_offsets(self.hidden, self.inter, self.bits)

    def x_f32(self) -> np.ndarray:
        return bf16_bits_to_f32(self.x_bf16)


def _distinct_uniform_ids(rng: np.random.Generator, tokens: int, experts: int, k: int) -> np.ndarray:
    keys = rng.random((tokens, experts))
    return np.argsort(keys, axis=1, kind="stable")[:, :k].astype(np.int64)


def _zipf_ids(rng: np.random.Generator, tokens: int, experts: int, k: int, s: float) -> np.ndarray:
    """k distinct experts per token, weighted sampling without replacement (Gumbel top-k).

    Popularity p(rank) ~ rank^-s, ranks assigned to experts by a seeded permutation."""
    perm = rng.permutation(experts)
    p_rank = np.arange(1, experts + 1, dtype=np.float64) ** (-s)
    p = np.empty(experts)
    p[perm] = p_rank / p_rank.sum()
    g = rng.gumbel(size=(tokens, experts))
    keys = np.log(p)[None, :] + g
    return np.argsort(-keys, axis=1, kind="stable")[:, :k].astype(np.int64)


def make_inputs(name: str, tokens: Optional[int] = None, seed: Optional[int] = None,
                identity_signs: bool = False, bits_override: Optional[int] = None,
                hidden: Optional[int] = None, inter: Optional[int] = None,
                experts: Optional[int] = None, top_k: Optional[int] = None,
                bits_choices: Optional[tuple] = None) -> LayerInputs:
    """Draw one input set for geometry `name` (see GEOMETRIES).

    seed defaults to 1000*geometry_index + tokens. identity_signs sets every sign vector to +1
    (used with the identity-rotation test mode). Shape overrides make small variants of a
    geometry for edge-case tests; bits_override (one width) or bits_choices (widths drawn per
    expert) replace the geometry's widths. The draw order is unchanged."""
    g = GEOMETRIES[name]
    H = int(hidden or g["hidden"])
    I = int(inter or g["inter"])
    E = int(experts or g["experts"])
    k = int(top_k or g["top_k"])
    T = int(tokens if tokens is not None else g["tokens"][0])
    if seed is None:
        seed = 1000 * GEOMETRY_INDEX[name] + T
    rng = np.random.Generator(np.random.PCG64(seed))

    choices = g["bits"] if bits_override is None else (bits_override,)
    if bits_choices is not None:
        choices = tuple(bits_choices)
    if len(choices) > 1:
        bits = rng.choice(np.asarray(choices, dtype=np.uint8), size=E)
    else:
        bits = np.full(E, choices[0], dtype=np.uint8)
    offs = payload_offsets(H, I, bits)
    payload = rng.integers(0, 1 << 16, size=int(offs[-1]), dtype=np.uint16)

    scale1 = (rng.uniform(0.5, 1.5, size=(E, 2 * I)) / 16.0).astype(np.float16)
    scale2 = (rng.uniform(0.5, 1.5, size=(E, H)) / 16.0).astype(np.float16)

    def signs(shape):
        s = np.where(rng.random(shape) < 0.5, -1.0, 1.0).astype(np.float16)
        return np.ones(shape, np.float16) if identity_signs else s

    su1 = signs((E, H))
    sv1 = signs((E, 2 * I))
    su2 = signs((E, I))
    sv2 = signs((E, H))

    xv = rng.standard_normal((T, H)) * g["x_sigma"]
    if g["outliers"]:
        mask = rng.random((T, H)) < OUTLIER_P
        xv = np.where(mask, xv * OUTLIER_GAIN, xv)
    x_bf16 = bf16_bits_from_f32(xv.astype(np.float32))

    if g["routing"] == "zipf":
        ids = _zipf_ids(rng, T, E, k, ZIPF_S)
    else:
        ids = _distinct_uniform_ids(rng, T, E, k)
    logits = rng.standard_normal((T, k))
    ex = np.exp(logits - logits.max(axis=1, keepdims=True))
    weights = (ex / ex.sum(axis=1, keepdims=True)).astype(np.float32)

    return LayerInputs(name=name, seed=int(seed), hidden=H, inter=I, experts=E, top_k=k,
                       tokens=T, bits=bits, payload=payload, scale1=scale1, scale2=scale2,
                       su1=su1, sv1=sv1, su2=su2, sv2=sv2, x_bf16=x_bf16, ids=ids,
                       weights=weights)


def all_cases():
    """(name, T) for every workload in the five geometries."""
    out = []
    for name, g in GEOMETRIES.items():
        for t in g["tokens"]:
            out.append((name, t))
    return out


# Dense trellis linear (one matrix, no routing): the decode geometry's FC1 shape as a single
# matrix (E = 1, k = 1), the wide geometry's hidden size as the non-power-of-two case, and the
# largest supported square matrix (8 MB of 4-bit payload) for measurement.
LINEAR_GEOMETRIES = {
    "linear":      dict(in_features=1024, out_features=1024, bits=4, tokens=(1, 16, 2048)),
    "linear_wide": dict(in_features=2560, out_features=320, bits=3, tokens=(16,)),
    "linear_4k":   dict(in_features=4096, out_features=4096, bits=4, tokens=(16, 2048)),
}


@dataclasses.dataclass
class LinearInputs:
    name: str
    seed: int
    in_features: int          # K
    out_features: int         # N
    tokens: int
    bits: int
    payload: np.ndarray       # uint16 [K/16 * N/16 * 16 * bits]
    scale: np.ndarray         # float16 [N]
    su: np.ndarray            # float16 [K], +-1
    sv: np.ndarray            # float16 [N], +-1
    x_bf16: np.ndarray        # uint16 [T, K]


def make_linear_inputs(name: str = "linear", tokens: Optional[int] = None, seed: Optional[int] = None,
                       in_features: Optional[int] = None, out_features: Optional[int] = None,
                       bits: Optional[int] = None, identity_signs: bool = False) -> LinearInputs:
    """Draw one dense-linear input set. Draw order: payload words -> scale -> su, sv -> x.
    seed defaults to 7000 + tokens."""
    g = LINEAR_GEOMETRIES[name]
    K = int(in_features or g["in_features"])
    N = int(out_features or g["out_features"])
    B = int(bits or g["bits"])
    T = int(tokens if tokens is not None else g["tokens"][0])
    if seed is None:
        seed = 7000 + T
    rng = np.random.Generator(np.random.PCG64(seed))
    payload = rng.integers(0, 1 << 16, size=(K // 16) * (N // 16) * 16 * B, dtype=np.uint16)
    scale = (rng.uniform(0.5, 1.5, size=N) / 16.0).astype(np.float16)

    def signs(n):
        s = np.where(rng.random(n) < 0.5, -1.0, 1.0).astype(np.float16)
        return np.ones(n, np.float16) if identity_signs else s

    su = signs(K)
    sv = signs(N)
    x_bf16 = bf16_bits_from_f32(rng.standard_normal((T, K)).astype(np.float32))
    return LinearInputs(name=name, seed=int(seed), in_features=K, out_features=N, tokens=T, bits=B,
                        payload=payload, scale=scale, su=su, sv=sv, x_bf16=x_bf16)
