"""The entry point without a scratch argument (tmoe_forward_w4a16_static) against the one with
the caller's arena (tmoe_forward_w4a16): two calls in a row through the C ABI, the second with
fewer tokens, both bit-identical to the arena entry point and within the W4A16 bound of the
oracle. The library's array keeps the first call's contents when the second runs."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle_np as O
from gpu_cases import TOL_W4A16, Case, rel_err, say

pytestmark = pytest.mark.gpu


def test_static_scratch_entry_point_matches_arena_entry_point():
    c = Case("decode", 16)
    H = c.inp.hidden
    ref_full = c.oracle_w4a16
    for T in (16, 4, 16):
        x, ids, w = c.x[:T].contiguous(), c.ids[:T].contiguous(), c.w[:T].contiguous()
        y_static = torch.full((T, H), float("nan"), device="cuda")
        y_arena = torch.full((T, H), float("nan"), device="cuda")
        say(f"[case] static scratch entry point, decode T={T} (plan max_tokens 16)")
        c.plan.forward_static(x, ids, w, c.weights, y=y_static)
        torch.cuda.synchronize()
        c.plan.forward(x, ids, w, c.weights, c.scratch, y=y_arena)
        torch.cuda.synchronize()
        assert torch.equal(y_static, y_arena), float((y_static - y_arena).abs().max())
        sub = dataclasses.replace(c.inp, tokens=T, x_bf16=c.inp.x_bf16[:T], ids=c.inp.ids[:T],
                                  weights=c.inp.weights[:T])
        ref = O.forward(sub)
        assert np.array_equal(ref, ref_full[:T])          # rows are independent of the batch
        err = rel_err(y_static.cpu().numpy(), ref)
        say(f"[result] static entry point T={T}: equal to the arena entry point, rel err {err:.3e}")
        assert err <= TOL_W4A16


def test_static_scratch_entry_point_zero_tokens():
    c = Case("tiny", 4)
    y = torch.full((4, c.inp.hidden), 7.0, device="cuda")
    c.plan.forward_static(c.x[:0], c.ids[:0], c.w[:0], c.weights, y=y[:0])
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
