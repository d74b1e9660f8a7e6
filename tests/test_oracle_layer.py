"""Pins of the oracle's layer: dense reconstruction, identity reduction, closed forms.

Steps and order: 'serve canonical Fruit QSRT atoms' (b12x PR #129), Hot path (input rotation,
route-major FC1, route-major FC2 with exact top-k weighting); 'integrate EXL3 Trellis into the
fused W4A16 API' (sparkinfer PR #90), review of kernel.py (activation epilogue
H128 -> svh -> silu -> suh_down -> H128)."""
import dataclasses

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle_np as O
from trellis_quantized_moe_tmoe_amd.workloads import bf16_bits_from_f32, make_inputs


def _R(n, identity=False):
    if identity:
        return np.eye(n)
    if n & (n - 1) == 0:
        sizes = [n]
    else:
        sizes = [128] * (n // 128) + ([n % 128] if n % 128 else [])
    return scipy.linalg.block_diag(*[scipy.linalg.hadamard(b) / np.sqrt(b) for b in sizes])


def _f16(a):
    return np.asarray(a, np.float16).astype(np.float64)


def _e4m3_round(v):
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()


def _mx_qdq(v):
    q, e = O.mxfp8_quantize(v[None, :])
    deq = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy()[0]
    return deq * np.repeat(np.ldexp(1.0, e[0].astype(np.int64) - 127), 32)


def dense_layer(inp, identity=False, w4a8=False):
    """Brute-force layer from explicit matrices: W1eff = [S(sv1g) R_I; S(sv1u) R_I] S(c1) C1^T R_H S(su1),
    W2eff = S(sv2) R_H S(c2) C2^T R_I S(su2). Uses scipy's Hadamard matrices and numpy matmuls;
    from the oracle only its (separately pinned) tile decoder and MX quantizer."""
    H, I, k = inp.hidden, inp.inter, inp.top_k
    RH, RI = _R(H, identity), _R(I, identity)
    x = inp.x_f32().astype(np.float64)
    y = np.zeros((inp.tokens, H))
    for t in range(inp.tokens):
        for j in range(k):
            e = int(inp.ids[t, j])
            c1b, c2b = O.expert_codes(inp, e)
            C1 = c1b.view(np.float16).astype(np.float64)
            C2 = c2b.view(np.float16).astype(np.float64)
            if w4a8:
                C1, C2 = _e4m3_round(C1), _e4m3_round(C2)
            S = np.diag
            if not w4a8:
                Wg = S(_f16(inp.sv1[e, :I])) @ RI @ S(_f16(inp.scale1[e, :I])) @ C1[:, :I].T @ RH @ S(_f16(inp.su1[e]))
                Wu = S(_f16(inp.sv1[e, I:])) @ RI @ S(_f16(inp.scale1[e, I:])) @ C1[:, I:].T @ RH @ S(_f16(inp.su1[e]))
                W2 = S(_f16(inp.sv2[e])) @ RH @ S(_f16(inp.scale2[e])) @ C2.T @ RI @ S(_f16(inp.su2[e]))
                g, u = Wg @ x[t], Wu @ x[t]
                h = g / (1 + np.exp(-g)) * u
                o = W2 @ h
            else:
                a = _mx_qdq(RH @ (_f16(inp.su1[e]) * x[t]))
                z = _f16(inp.scale1[e]) * (C1.T @ a)
                g = _f16(inp.sv1[e, :I]) * (RI @ z[:I])
                u = _f16(inp.sv1[e, I:]) * (RI @ z[I:])
                h = g / (1 + np.exp(-g)) * u
                b = _mx_qdq(RI @ (_f16(inp.su2[e]) * h))
                v = _f16(inp.scale2[e]) * (C2.T @ b)
                o = _f16(inp.sv2[e]) * (RH @ v)
            y[t] += float(inp.weights[t, j]) * o
    return y


def _rel(a, b):
    return np.max(np.abs(a - b)) / np.max(np.abs(b))


CASES = [dict(name="tiny"), dict(name="wide", tokens=3, hidden=320, inter=160, experts=4, top_k=2),
         dict(name="decode", tokens=2, hidden=128, inter=64, experts=5, top_k=3)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c["name"])
def test_dense_reconstruction_w4a16(case):
    inp = make_inputs(**case)
    assert _rel(O.forward(inp), dense_layer(inp)) < 1e-12


@pytest.mark.parametrize("case", CASES[:2], ids=lambda c: c["name"])
def test_dense_reconstruction_w4a8(case):
    inp = make_inputs(**case)
    assert _rel(O.forward(inp, mode="w4a8"), dense_layer(inp, w4a8=True)) < 1e-9


def test_identity_reduces_to_plain_dense_moe():
    inp = make_inputs("tiny", identity_signs=True)
    H, I = inp.hidden, inp.inter
    x = inp.x_f32().astype(np.float64)
    y = np.zeros((inp.tokens, H))
    for t in range(inp.tokens):
        for j in range(inp.top_k):
            e = int(inp.ids[t, j])
            c1b, c2b = O.expert_codes(inp, e)
            W1 = c1b.view(np.float16).astype(np.float64) * _f16(inp.scale1[e])[None, :]
            W2 = c2b.view(np.float16).astype(np.float64) * _f16(inp.scale2[e])[None, :]
            g, u = W1[:, :I].T @ x[t], W1[:, I:].T @ x[t]
            y[t] += float(inp.weights[t, j]) * (W2.T @ (g / (1 + np.exp(-g)) * u))
    assert _rel(O.forward(inp, identity=True), y) < 1e-12


def test_zero_input_gives_exact_zero():
    inp = make_inputs("tiny")
    inp = dataclasses.replace(inp, x_bf16=np.zeros_like(inp.x_bf16))
    assert np.array_equal(O.forward(inp), np.zeros((inp.tokens, inp.hidden)))


def test_linear_in_weights_and_batch_independent():
    inp = make_inputs("tiny")
    y = O.forward(inp)
    y2 = O.forward(dataclasses.replace(inp, weights=(inp.weights * 2).astype(np.float32)))
    assert np.array_equal(y2, 2 * y)
    sub = dataclasses.replace(inp, tokens=2, x_bf16=inp.x_bf16[[1, 3]], ids=inp.ids[[1, 3]],
                              weights=inp.weights[[1, 3]])
    assert np.array_equal(O.forward(sub), y[[1, 3]])


def test_identical_experts_make_output_independent_of_ids():
    inp = make_inputs("tiny")
    off = inp.payload_offsets()
    one = inp.payload[off[0]:off[1]]
    same = dict(payload=np.tile(one, inp.experts))
    for nm in ("scale1", "scale2", "su1", "sv1", "su2", "sv2"):
        a = getattr(inp, nm)
        same[nm] = np.repeat(a[:1], inp.experts, axis=0)
    a = dataclasses.replace(inp, **same)
    b = dataclasses.replace(a, ids=np.roll(a.ids, 1, axis=0)[:, ::-1].copy())
    ya, yb = O.forward(a), O.forward(b)
    tr = [O.route_trace(a, t, 0)["o"] for t in range(a.tokens)]
    wsum = a.weights.astype(np.float64).sum(axis=1)
    assert np.allclose(ya, yb, rtol=1e-12, atol=1e-12)
    assert np.allclose(ya, np.array(tr) * wsum[:, None], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "wide", "w4a8"])
def test_generated_topk_weights_sum_to_one(name):
    inp = make_inputs(name, tokens=64, hidden=64, inter=32)
    assert np.all(np.abs(inp.weights.astype(np.float64).sum(axis=1) - 1.0) <= 1e-6)
    assert all(len(set(r)) == inp.top_k for r in inp.ids.tolist())


def test_route_trace_matches_forward():
    inp = make_inputs("tiny")
    y = O.forward(inp)
    rec = np.zeros_like(y)
    for t in range(inp.tokens):
        for j in range(inp.top_k):
            rec[t] += float(inp.weights[t, j]) * O.route_trace(inp, t, j)["o"]
    assert np.allclose(rec, y, rtol=1e-13, atol=1e-13)


def test_bf16_generator_rounding():
    v = np.array([1.0, 1.00390625, 1.005859375, -3.14159265], np.float32)
    b = bf16_bits_from_f32(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, ref)
