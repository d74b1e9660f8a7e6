"""GPU parity of the dense trellis linear (tmoe_linear_w4a16) against the float64 oracle (reading R8:
y = sv * R_N(scale * (C^T R_K(su * x))); "integrate EXL3 Trellis into the fused W4A16 API",
sparkinfer PR #90, names the dense trellis GEMM and trellis_linear beside the fused MoE).

Tolerance: the only rounding beyond fp32 accumulation is the fp16 operand a = fp16(R_K(su * x))
(relative 2^-11 per element); it moves each output by about 2^-11 of its rms over K random terms,
so max |y - y_ref| / max |y_ref| stays well inside 3e-3 (the layer's stated bound is 1e-2)."""
import numpy as np
import pytest
import torch

import oracle_np as O
from gpu_cases import rel_err, say
from trellis_quantized_moe_tmoe_amd.workloads import make_linear_inputs

pytestmark = pytest.mark.gpu
TOL_LINEAR = 3e-3


class LinearCase:
    def __init__(self, name, T, max_tokens=None, rotation="hadamard", identity_signs=False, **over):
        from trellis_quantized_moe_tmoe_amd import layer as L
        self.inp = make_linear_inputs(name, tokens=T, identity_signs=identity_signs, **over)
        i = self.inp
        self.label = f"{name} T={T} K={i.in_features} N={i.out_features} bits={i.bits} seed={i.seed} rot={rotation}"
        say(f"[case] linear {self.label}")
        self.plan = L.LinearPlan.for_inputs(i, max_tokens=max_tokens, rotation=rotation)
        self.w = L.LinearWeightsDev.from_inputs(i)
        self.x = torch.from_numpy(i.x_bf16.view(np.int16).copy()).cuda()
        self.scratch = self.plan.alloc_scratch()
        self.rotation = rotation

    def run(self, y=None):
        y = self.plan.forward(self.x, self.w, self.scratch, y=y)
        torch.cuda.synchronize()
        return y

    def oracle(self):
        return O.linear(self.inp, identity=self.rotation == "identity")


@pytest.mark.parametrize("name,T,over", [
    ("linear", 1, {}),                                             # one 16-row tile, 8 K splits
    ("linear", 16, {}),
    ("linear", 37, dict(in_features=256, out_features=192)),       # 32/64-row tiles, ragged, 128+64 output
    ("linear", 300, {}),                                           # 128-row workgroup tiles, ragged tail
    ("linear", 2048, {}),                                          # full size of the prefill-like case
    ("linear", 16, dict(bits=2)),
    ("linear", 16, dict(bits=3)),
    ("linear", 16, dict(bits=5)),                                  # two half windows per 8-element group
    ("linear", 300, dict(bits=6, in_features=512, out_features=256)),  # 64-row tiles at widths 5-6
    ("linear", 16, dict(in_features=2048, out_features=4096)),     # rows of 2048 and 4096 values: both
    ("linear", 5, dict(in_features=4096, out_features=1024, bits=3)),  # rotations split over a workgroup
    ("linear_wide", 16, {}),                                       # 2560 x 320, 3-bit, both rotations blocked
    ("linear_wide", 2100, dict(in_features=320, out_features=2560)),   # many tokens: per-route rotation,
                                                                   # per-block combine wavefronts
])
def test_linear_matches_oracle(name, T, over):
    c = LinearCase(name, T, **over)
    err = rel_err(c.run().cpu().numpy(), c.oracle())
    say(f"[result] {c.label} rel err {err:.3e}")
    assert err <= TOL_LINEAR


def test_linear_identity_mode_and_capacity_above_T():
    c = LinearCase("linear", 24, max_tokens=512, rotation="identity", identity_signs=True,
                   in_features=128, out_features=256)
    assert rel_err(c.run().cpu().numpy(), c.oracle()) <= TOL_LINEAR


def test_linear_identity_mode_long_rows():
    c = LinearCase("linear", 9, rotation="identity", identity_signs=True, in_features=4096, out_features=2048)
    assert rel_err(c.run().cpu().numpy(), c.oracle()) <= TOL_LINEAR


def test_linear_deterministic_and_poison_independent():
    c = LinearCase("linear", 40, in_features=512, out_features=384)
    y0 = c.run().clone()
    c.scratch.fill_(0xFF)
    y1 = c.run(y=torch.full_like(y0, float("nan")))
    assert torch.equal(y0, y1)


def test_linear_zero_tokens_leaves_y():
    c = LinearCase("linear", 4, in_features=128, out_features=128)
    x0 = c.x[:0]
    y = torch.full((4, 128), 7.0, device="cuda")
    c.plan.forward(x0, c.w, c.scratch, y=y[:0])
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)


@pytest.mark.parametrize("n", [256, 4096])      # 4096: workgroup-row rotations on both sides
def test_linear_graph_replay_with_changed_inputs(n):
    c = LinearCase("linear", 16, in_features=n, out_features=n)
    y = torch.empty((16, n), device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        c.plan.forward(c.x, c.w, c.scratch, y=y)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        c.plan.forward(c.x, c.w, c.scratch, y=y)
    torch.cuda.synchronize()
    for seed in (11, 12, 13):
        other = make_linear_inputs("linear", tokens=16, seed=seed, in_features=n, out_features=n)
        c.x.copy_(torch.from_numpy(other.x_bf16.view(np.int16).copy()))
        g.replay()
        torch.cuda.synchronize()
        eager = c.plan.forward(c.x, c.w, c.scratch)
        torch.cuda.synchronize()
        assert torch.equal(y, eager)
        c.inp.x_bf16 = other.x_bf16
        assert rel_err(y.cpu().numpy(), c.oracle()) <= TOL_LINEAR
