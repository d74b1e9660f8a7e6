"""The Python binding checks tensor shapes, dtypes, layouts and devices before it calls the C ABI
(which sees raw pointers only and cannot check buffer sizes). Every case here must raise ValueError
before any launch; the tensors live on the CPU, so a call that slipped through would be caught by
the final device check rather than reaching a kernel."""
import numpy as np
import pytest
import torch

from trellis_quantized_moe_tmoe_amd import layer as L
from trellis_quantized_moe_tmoe_amd.workloads import make_inputs, make_linear_inputs


def _cpu_case(ids_dtype=torch.int64):
    inp = make_inputs("tiny")
    plan = L.Plan.for_inputs(inp, ids_dtype=ids_dtype)
    weights = L.DeviceWeights.from_inputs(inp, "cpu")
    x, ids, w = L.device_activations(inp, "cpu", ids_dtype=ids_dtype)
    y = torch.empty((inp.tokens, inp.hidden), dtype=torch.float32)
    scratch = torch.empty(plan.scratch_bytes, dtype=torch.uint8)
    return inp, plan, weights, dict(x=x, ids=ids, w=w, y=y, scratch=scratch)


def _call(plan, weights, a, stages=False):
    if stages:
        plan.forward_stages(0, 4, a["x"], a["ids"], a["w"], weights, a["scratch"], a["y"])
    else:
        plan.forward(a["x"], a["ids"], a["w"], weights, a["scratch"], y=a["y"])


def test_valid_cpu_tensors_stop_at_the_device_check():
    _, plan, weights, a = _cpu_case()
    with pytest.raises(ValueError, match="GPU device"):
        _call(plan, weights, a)
    with pytest.raises(ValueError, match="GPU device"):
        _call(plan, weights, a, stages=True)


@pytest.mark.parametrize("field,bad,msg", [
    ("y", lambda a: torch.empty((a["y"].shape[0] - 1, a["y"].shape[1])), "y: shape"),
    ("y", lambda a: torch.empty(a["y"].shape, dtype=torch.float16), "y: dtype"),
    ("y", lambda a: torch.empty((a["y"].shape[1], a["y"].shape[0])).t(), "y: must be contiguous"),
    ("x", lambda a: a["x"][:, :-8], "x: shape"),
    ("x", lambda a: a["x"].float(), "x: dtype"),
    ("x", lambda a: a["x"].reshape(-1), "x: expected a 2-D"),
    ("ids", lambda a: a["ids"].to(torch.int32), "ids: dtype"),
    ("ids", lambda a: a["ids"][:, :1], "ids: shape"),
    ("w", lambda a: a["w"].double(), "w: dtype"),
    ("w", lambda a: a["w"][:-1], "w: shape"),
    ("scratch", lambda a: a["scratch"][:-16], "scratch: .* bytes"),
    ("scratch", lambda a: a["scratch"].view(torch.int32), "scratch: expected"),
])
def test_layer_rejects_mismatched_tensors(field, bad, msg):
    _, plan, weights, a = _cpu_case()
    a[field] = bad(a)
    for stages in (False, True):
        with pytest.raises(ValueError, match=msg):
            _call(plan, weights, a, stages)


def test_layer_rejects_int32_ids_on_an_int64_plan_and_back():
    _, plan, weights, a = _cpu_case(torch.int32)
    a["ids"] = a["ids"].to(torch.int64)
    with pytest.raises(ValueError, match="ids: dtype"):
        _call(plan, weights, a)


def test_layer_rejects_too_many_tokens():
    inp, plan, weights, a = _cpu_case()
    a["x"] = torch.cat([a["x"], a["x"]])
    with pytest.raises(ValueError, match="at most"):
        _call(plan, weights, a)


@pytest.mark.parametrize("name", ["payload", "scale1", "sv2"])
def test_layer_rejects_weights_of_another_shape(name):
    _, plan, weights, a = _cpu_case()
    t = getattr(weights, name)
    setattr(weights, name, t.reshape(-1)[: t.numel() - 2] if name == "payload" else t[:-1])
    with pytest.raises(ValueError, match=name):
        _call(plan, weights, a)


def test_layer_rejects_mixed_devices_before_the_device_type():
    _, plan, weights, a = _cpu_case()
    a["y"] = torch.empty(a["y"].shape, dtype=torch.float32, device="meta")
    with pytest.raises(ValueError, match="different devices"):
        _call(plan, weights, a)


def test_linear_rejects_mismatched_tensors():
    inp = make_linear_inputs("linear", tokens=4, in_features=128, out_features=256)
    plan = L.LinearPlan.for_inputs(inp)
    wts = L.LinearWeightsDev.from_inputs(inp, "cpu")
    x = torch.from_numpy(inp.x_bf16.view(np.int16).copy())
    scratch = torch.empty(plan.scratch_bytes, dtype=torch.uint8)
    y = torch.empty((4, 256), dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU device"):
        plan.forward(x, wts, scratch, y=y)
    with pytest.raises(ValueError, match="y: shape"):
        plan.forward(x, wts, scratch, y=torch.empty((4, 128)))
    with pytest.raises(ValueError, match="x: shape"):
        plan.forward(x[:, :64], wts, scratch, y=y)
    with pytest.raises(ValueError, match="scratch"):
        plan.forward(x, wts, scratch[:-1], y=y)
    wts.sv = wts.sv[:-1]
    with pytest.raises(ValueError, match="sv: shape"):
        plan.forward(x, wts, scratch, y=y)
