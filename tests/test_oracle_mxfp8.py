"""Pins of the oracle's MXFP8 quantizer and E4M3 rounding.

UE8M0 rule: 'TrellisMX (procedural NPK) ... P8 runtime' (flashinfer PR #69), Precision notes;
K/32 scale plane: same page, description of _activation_scale_cols_pad."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle_np as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold():
    with open(os.path.join(GOLD, "mxfp8.json")) as f:
        return json.load(f)


def test_exponent_hand_worked():
    for c in _gold()["exponent"]:
        a = c["amax"]
        if a == "nextafter(448, inf)":
            a = float(np.nextafter(np.float32(448.0), np.float32(np.inf)))
        assert O.lib().orc_mx_exponent(float(a)) == c["e"], c


def test_e4m3_hand_worked():
    for c in _gold()["e4m3"]:
        b = int(O.lib().orc_double_to_e4m3(c["v"]))
        if "byte" in c:
            assert b == int(c["byte"], 16), c
        assert O.lib().orc_e4m3_to_double(b) == c["value"], c


def test_e4m3_vs_torch_float8():
    """E4M3 round-to-nearest-even agrees with torch.float8_e4m3fn (a library routine) for values
    up to the 448 saturation point, including ties and subnormals."""
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(20000) * 30, rng.standard_normal(5000) * 0.01,
                        np.arange(-448, 449, 0.5), np.ldexp(np.arange(0, 64), -12),
                        -np.ldexp(np.arange(0, 64), -12)]).astype(np.float32)
    v = v[np.abs(v) <= 448]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([O.lib().orc_double_to_e4m3(float(x)) for x in v], np.uint8)
    # torch keeps -0 for negative values that round to zero; so does the oracle
    assert np.array_equal(got, ref)


def test_e4m3_decode_all_bytes_vs_torch():
    allb = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(allb).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([O.lib().orc_e4m3_to_double(int(b)) for b in allb])
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok]) and np.all(np.isnan(got[~ok]))


def test_quantizer_block_properties():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((64, 256)) * np.exp(rng.standard_normal((64, 1)) * 3)).astype(np.float32)
    x[3, :32] = 0.0
    q, e = O.mxfp8_quantize(x.astype(np.float64))
    deq = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    scale = np.ldexp(1.0, e.astype(np.int64) - 127)
    deq = deq * np.repeat(scale, 32, axis=1)
    blocks = np.abs(x.astype(np.float64)).reshape(64, 8, 32).max(axis=2)
    for r in range(64):
        for b in range(8):
            amax = blocks[r, b]
            ex = int(e[r, b]) - 127
            if amax == 0:
                assert ex == -127
                continue
            # 2^e is the smallest power of two with amax / 2^e <= 448 (up to the fp32 quotient)
            assert amax / 2.0 ** ex <= 448 * (1 + 2 ** -23)
            assert amax / 2.0 ** (ex - 1) > 448 * (1 - 2 ** -23)
    # relative error of each element is at most half an E4M3 step (2^-4) of its block scale
    err = np.abs(deq - x)
    bound = np.repeat(np.ldexp(1.0, e.astype(np.int64) - 127), 32, axis=1) * 2.0 ** 5  # coarse
    assert np.all(err <= bound)
    assert np.all(q[3, :32] == 0) and e[3, 0] == 0


def test_quantizer_lossless_on_representable_input():
    """Values that are E4M3 codes times a power of two with block max 448*2^s come back exactly."""
    rng = np.random.default_rng(9)
    codes = rng.integers(0, 0x7F, size=(4, 64)).astype(np.uint8)
    codes[:, 0] = 0x7E                                   # 448 in every block
    codes[:, 32] = 0x7E
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy() * 2.0 ** -5
    q, e = O.mxfp8_quantize(vals)
    assert np.array_equal(q, codes)
    assert np.all(e == 127 - 5)
