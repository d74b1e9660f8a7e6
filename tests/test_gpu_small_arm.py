"""The small-batch arm (one persistent launch for the whole layer, plan field smallm_max_tokens)
against the float64 oracle, and against the five-launch path of the same plan geometry."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle_np as O
from gpu_cases import TOL_W4A16, TOL_W4A8_EMU, Case, rel_err, say
from trellis_quantized_moe_tmoe_amd.layer import scratch_view

pytestmark = pytest.mark.gpu


class ArmCase(Case):
    """A case whose plan runs forwards of up to 16 tokens as the single persistent launch."""

    def __init__(self, name, tokens=None, **over):
        super().__init__(name, tokens, **over)
        from trellis_quantized_moe_tmoe_amd import layer as L
        self.plan = L.Plan.for_inputs(self.inp, smallm_max_tokens=16)
        self.scratch = self.plan.alloc_scratch()


def arm_status(c):
    v = c.plan.debug_views(c.inp.tokens, False, c.scratch)
    return int(scratch_view(c.scratch, v.arm_status, (1,), torch.int32).item())


def five_launch(c, w4a8=False):
    from trellis_quantized_moe_tmoe_amd import layer as L
    plan = L.Plan.for_inputs(c.inp, smallm_max_tokens=0)
    scratch = plan.alloc_scratch()
    y = plan.forward(c.x, c.ids, c.w, c.weights, scratch, w4a8=w4a8)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("name,T,over", [
    ("decode", 1, {}), ("decode", 4, {}), ("decode", 16, {}),
    ("tiny", 4, {}), ("tiny", 16, {}),                                 # 2 routes per expert: 16-row tiles
    ("wide", 16, {}),                                                  # H 2560 = 20 x 128, I 320 = 128+128+64
    ("tiny", 8, dict(bits_override=5)), ("tiny", 8, dict(bits_override=6)),
    ("tiny", 16, dict(bits_choices=(2, 3, 4, 5, 6))),
    ("tiny", 2, dict(hidden=1024, inter=128, experts=4, top_k=1)),    # top-1
])
def test_small_arm_w4a16(name, T, over):
    c = ArmCase(name, T, **over)
    assert c.plan.smallm_max_tokens >= T
    y = c.run().cpu().numpy()
    assert arm_status(c) == 0
    err = rel_err(y, c.oracle_w4a16)
    ref5 = five_launch(c).cpu().numpy()
    d5 = rel_err(y, ref5)
    say(f"[result] {c.label} small arm W4A16 rel err {err:.3e} (vs five launches {d5:.3e}, "
        f"bitwise equal: {bool(np.array_equal(y, ref5))})")
    assert err <= TOL_W4A16
    assert d5 <= 2e-3


@pytest.mark.parametrize("T", [1, 8, 16])
def test_small_arm_w4a8(T):
    c = ArmCase("w4a8", T)
    y = c.run(w4a8=True).cpu().numpy()
    assert arm_status(c) == 0
    e8 = rel_err(y, c.oracle_w4a8)
    e16 = rel_err(y, c.oracle_w4a16)
    gap = rel_err(c.oracle_w4a8, c.oracle_w4a16)
    say(f"[result] {c.label} small arm W4A8 rel err vs W4A8 oracle {e8:.3e}, vs W4A16 oracle {e16:.3e}")
    assert e8 <= TOL_W4A8_EMU
    assert e16 <= gap + TOL_W4A8_EMU


def test_small_arm_repeated_calls_are_bitwise_equal():
    c = ArmCase("decode", 16)
    first = c.run().clone()
    for i in range(40):
        y = c.run()
        assert torch.equal(y, first), i
    assert arm_status(c) == 0


def test_small_arm_dropped_ids_and_an_empty_token():
    c = ArmCase("decode", 4)
    ids = c.inp.ids.copy()
    ids[1, 3] = -1
    ids[2, :] = 200                       # every route of token 2 dropped: its row is zero
    c.ids = torch.from_numpy(ids).cuda()
    y = c.run().cpu().numpy()
    w = c.inp.weights.copy()
    w[1, 3] = 0.0
    w[2, :] = 0.0
    fixed = ids.copy()
    fixed[1, 3] = 0
    fixed[2, :] = np.arange(8)
    ref = O.forward(dataclasses.replace(c.inp, ids=fixed, weights=w))
    assert np.all(y[2] == 0.0)
    assert rel_err(y, ref) <= TOL_W4A16
    assert arm_status(c) == 0
    view = c.plan.debug_views(4, False, c.scratch)
    # the dropped-id count of the call sits beside the status word in the arena's scalars
    status = scratch_view(c.scratch, view.arm_status - 16, (1,), torch.int32).item()
    assert status == 9


def test_small_arm_graph_replays_with_changed_inputs():
    from trellis_quantized_moe_tmoe_amd.workloads import make_inputs
    c = ArmCase("decode", 16)
    y = torch.empty((16, c.inp.hidden), device="cuda")
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        c.plan.forward(c.x, c.ids, c.w, c.weights, c.scratch, y=y)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        c.plan.forward(c.x, c.ids, c.w, c.weights, c.scratch, y=y)
    for seed in (21, 22, 23):
        other = make_inputs("decode", tokens=16, seed=seed)
        c.x.copy_(torch.from_numpy(other.x_bf16.view(np.int16)).cuda())
        c.ids.copy_(torch.from_numpy(other.ids).cuda())
        c.w.copy_(torch.from_numpy(other.weights).cuda())
        for _ in range(3):
            g.replay()
            torch.cuda.synchronize()
            eager = c.plan.forward(c.x, c.ids, c.w, c.weights, c.scratch).clone()
            torch.cuda.synchronize()
            assert torch.equal(y, eager)
        ref = O.forward(dataclasses.replace(c.inp, x_bf16=other.x_bf16, ids=other.ids, weights=other.weights))
        assert rel_err(y.cpu().numpy(), ref) <= TOL_W4A16
    assert arm_status(c) == 0


def test_small_arm_two_arenas_interleaved():
    c = ArmCase("decode", 4)
    s2 = c.plan.alloc_scratch()
    y1 = c.plan.forward(c.x, c.ids, c.w, c.weights, c.scratch).clone()
    for _ in range(3):
        ya = c.plan.forward(c.x, c.ids, c.w, c.weights, s2)
        yb = c.plan.forward(c.x, c.ids, c.w, c.weights, c.scratch)
        torch.cuda.synchronize()
        assert torch.equal(ya, y1) and torch.equal(yb, y1)


def test_small_arm_static_scratch_entry_point():
    c = ArmCase("decode", 16)
    y = c.plan.forward_static(c.x, c.ids, c.w, c.weights)
    torch.cuda.synchronize()
    assert rel_err(y.cpu().numpy(), c.oracle_w4a16) <= TOL_W4A16
