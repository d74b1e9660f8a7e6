"""Thin torch-facing wrapper over the C ABI: torch provides device memory and the stream only.

Every step of the layer runs in the HIP kernels of libtmoe.so; this module only passes tensor
pointers, sizes and the current stream."""
from __future__ import annotations

import ctypes
from typing import Optional

import numpy as np
import torch

from . import native
from .native import check, lib


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


# The C ABI sees raw pointers only, so it cannot check buffer sizes: the shapes, dtypes, layouts
# and devices of the tensors are checked here, before any call that would launch a kernel.
_BITS16 = (torch.int16, torch.bfloat16, torch.uint16) if hasattr(torch, "uint16") else (torch.int16, torch.bfloat16)


def _require(t, name: str, shape, dtypes) -> None:
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype}, expected one of {[str(d) for d in dtypes]}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _same_device(named) -> None:
    devs = {t.device for _, t in named}
    if len(devs) != 1:
        raise ValueError("tensors on different devices: " + ", ".join(f"{n}={t.device}" for n, t in named))
    dev = devs.pop()
    if dev.type != "cuda":
        raise ValueError(f"tensors must be on a GPU device, got {dev}")


def _check_scratch(scratch, need: int) -> None:
    if not isinstance(scratch, torch.Tensor) or scratch.dtype != torch.uint8 or scratch.dim() != 1:
        raise ValueError("scratch: expected a 1-D uint8 tensor")
    if not scratch.is_contiguous():
        raise ValueError("scratch: must be contiguous")
    if scratch.numel() < need:
        raise ValueError(f"scratch: {scratch.numel()} bytes, the plan needs {need}")


class DeviceWeights:
    """Device copies of one weight set: trellis payload words, fp16 scales and sign vectors."""

    FIELDS = ("payload", "scale1", "scale2", "su1", "sv1", "su2", "sv2")

    def __init__(self, payload: torch.Tensor, scale1, scale2, su1, sv1, su2, sv2):
        self.payload, self.scale1, self.scale2 = payload, scale1, scale2
        self.su1, self.sv1, self.su2, self.sv2 = su1, sv1, su2, sv2
        self._c = native.Weights(*[t.data_ptr() for t in (payload, scale1, scale2, su1, sv1, su2, sv2)])

    @classmethod
    def from_inputs(cls, inp, device="cuda") -> "DeviceWeights":
        def up(a, dt):
            return torch.from_numpy(np.ascontiguousarray(a).view(dt)).to(device)
        return cls(up(inp.payload, np.int16), *[up(getattr(inp, n), np.float16)
                                                 for n in ("scale1", "scale2", "su1", "sv1", "su2", "sv2")])

    def clone(self) -> "DeviceWeights":
        return DeviceWeights(*[getattr(self, n).clone() for n in self.FIELDS])

    @property
    def c(self) -> native.Weights:
        return self._c


def device_activations(inp, device="cuda", ids_dtype=torch.int64):
    """(x as bf16 bit patterns in an int16 tensor [T, H], ids [T, k], weights fp32 [T, k])."""
    x = torch.from_numpy(np.ascontiguousarray(inp.x_bf16).view(np.int16)).to(device)
    ids = torch.from_numpy(np.ascontiguousarray(inp.ids)).to(ids_dtype).to(device)
    w = torch.from_numpy(np.ascontiguousarray(inp.weights, np.float32)).to(device)
    return x, ids, w


class Plan:
    def __init__(self, hidden: int, inter: int, num_experts: int, top_k: int, max_tokens: int,
                 expert_bits, rotation: str = "hadamard", ids_dtype=torch.int64, block_m: int = 0,
                 smallm_max_tokens: int = 0, fc2_reduce: str = "deterministic"):
        """smallm_max_tokens: forwards with at most this many tokens run as one persistent launch
        (the pages' small-M arm, whose default is 16; here 0 = never by default, as the five-launch
        path is faster on gfx950). fc2_reduce: "deterministic" (route-major epilogue, bitwise
        reproducible) or "atomic" (FP32 atomic sum into y, opt-in)."""
        bits = np.ascontiguousarray(np.asarray(expert_bits, dtype=np.uint8))
        self._bits = bits
        if fc2_reduce not in ("deterministic", "atomic"):
            raise ValueError(f"fc2_reduce: {fc2_reduce!r}")
        self.config = native.Config(hidden, inter, num_experts, top_k, max_tokens,
                                    bits.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)),
                                    native.ROT_IDENTITY if rotation == "identity" else native.ROT_HADAMARD,
                                    native.IDS_I64 if ids_dtype == torch.int64 else native.IDS_I32, block_m,
                                    smallm_max_tokens,
                                    native.FC2_ATOMIC if fc2_reduce == "atomic" else native.FC2_DETERMINISTIC)
        self.smallm_max_tokens, self.fc2_reduce = smallm_max_tokens, fc2_reduce
        self.ids_dtype = ids_dtype
        handle = ctypes.c_void_p()
        sb, pw = ctypes.c_size_t(), ctypes.c_size_t()
        check(lib.tmoe_plan(ctypes.byref(self.config), ctypes.byref(handle), ctypes.byref(sb), ctypes.byref(pw)),
              "tmoe_plan")
        self.handle = handle
        self.scratch_bytes = sb.value
        self.payload_words = pw.value
        self.hidden, self.inter, self.num_experts, self.top_k = hidden, inter, num_experts, top_k
        self.max_tokens = max_tokens

    @classmethod
    def for_inputs(cls, inp, max_tokens: Optional[int] = None, **kw) -> "Plan":
        return cls(inp.hidden, inp.inter, inp.experts, inp.top_k, max_tokens or inp.tokens, inp.bits, **kw)

    def close(self):
        if getattr(self, "handle", None) and self.handle.value:
            lib.tmoe_plan_destroy(self.handle)
            self.handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def info(self) -> native.PlanInfo:
        out = native.PlanInfo()
        check(lib.tmoe_plan_get_info(self.handle, ctypes.byref(out)), "tmoe_plan_get_info")
        return out

    def expert_offset(self, e: int) -> int:
        out = ctypes.c_size_t()
        check(lib.tmoe_plan_expert_offset(self.handle, e, ctypes.byref(out)), "tmoe_plan_expert_offset")
        return out.value

    def alloc_scratch(self, device="cuda") -> torch.Tensor:
        return torch.empty(self.scratch_bytes, dtype=torch.uint8, device=device)

    def forward(self, x: torch.Tensor, ids: torch.Tensor, w: torch.Tensor, weights: DeviceWeights,
                scratch: torch.Tensor, y: Optional[torch.Tensor] = None, w4a8: bool = False) -> torch.Tensor:
        T = x.shape[0] if isinstance(x, torch.Tensor) and x.dim() == 2 else -1
        if y is None and isinstance(x, torch.Tensor):
            y = torch.empty((max(T, 0), self.hidden), dtype=torch.float32, device=x.device)
        self.check_call(x, ids, w, weights, scratch, y)
        fn = lib.tmoe_forward_w4a8 if w4a8 else lib.tmoe_forward_w4a16
        check(fn(self.handle, _ptr(x), _ptr(ids), _ptr(w), T, ctypes.byref(weights.c), _ptr(y), _ptr(scratch),
                 scratch.numel(), _stream(x.device)), "tmoe_forward_w4a8" if w4a8 else "tmoe_forward_w4a16")
        return y

    def forward_static(self, x: torch.Tensor, ids: torch.Tensor, w: torch.Tensor, weights: DeviceWeights,
                       y: Optional[torch.Tensor] = None) -> torch.Tensor:
        """W4A16 forward on the library's own per-GPU scratch array (tmoe_forward_w4a16_static): the
        call allocates nothing when y is given."""
        T = x.shape[0] if isinstance(x, torch.Tensor) and x.dim() == 2 else -1
        if y is None and isinstance(x, torch.Tensor):
            y = torch.empty((max(T, 0), self.hidden), dtype=torch.float32, device=x.device)
        if self.scratch_bytes > native.STATIC_SCRATCH_BYTES:
            raise ValueError(f"plan needs {self.scratch_bytes} scratch bytes, the static arena holds "
                             f"{native.STATIC_SCRATCH_BYTES}")
        self.check_call(x, ids, w, weights, None, y)
        check(lib.tmoe_forward_w4a16_static(self.handle, _ptr(x), _ptr(ids), _ptr(w), T, ctypes.byref(weights.c),
                                            _ptr(y), _stream(x.device)), "tmoe_forward_w4a16_static")
        return y

    def forward_stages(self, first: int, last: int, x: torch.Tensor, ids: torch.Tensor, w: torch.Tensor,
                       weights: DeviceWeights, scratch: torch.Tensor, y: torch.Tensor, w4a8: bool = False) -> None:
        self.check_call(x, ids, w, weights, scratch, y)
        check(lib.tmoe_forward_stages(self.handle, int(w4a8), first, last, _ptr(x), _ptr(ids), _ptr(w), x.shape[0],
                                      ctypes.byref(weights.c), _ptr(y), _ptr(scratch), scratch.numel(),
                                      _stream(x.device)), "tmoe_forward_stages")

    def check_call(self, x, ids, w, weights, scratch, y) -> None:
        """Raise ValueError unless the tensors match what the forward reads and writes: x bf16 bits
        [T, H]; ids [T, k] of the plan's id dtype; w fp32 [T, k]; y fp32 [T, H]; weights of this
        plan's shapes; scratch at least the planned bytes; all contiguous, on one GPU device."""
        if not isinstance(x, torch.Tensor) or x.dim() != 2:
            raise ValueError("x: expected a 2-D tensor [T, H]")
        T = x.shape[0]
        if T > self.max_tokens:
            raise ValueError(f"x: {T} tokens, the plan holds at most {self.max_tokens}")
        H, I, E, k = self.hidden, self.inter, self.num_experts, self.top_k
        _require(x, "x", (T, H), _BITS16)
        _require(ids, "ids", (T, k), (self.ids_dtype,))
        _require(w, "w", (T, k), (torch.float32,))
        _require(y, "y", (T, H), (torch.float32,))
        if not isinstance(weights, DeviceWeights):
            raise ValueError("weights: expected DeviceWeights")
        _require(weights.payload, "payload", (self.payload_words,), (torch.int16,))
        for name, n in (("scale1", 2 * I), ("scale2", H), ("su1", H), ("sv1", 2 * I), ("su2", I), ("sv2", H)):
            _require(getattr(weights, name), name, (E, n), (torch.float16, torch.int16))
        if scratch is not None:
            _check_scratch(scratch, self.scratch_bytes)
        _same_device([("x", x), ("ids", ids), ("w", w), ("y", y)] + ([("scratch", scratch)] if scratch is not None else [])
                     + [(n, getattr(weights, n)) for n in DeviceWeights.FIELDS])

    def forward_status(self, x, ids, w, T, weights, y, scratch, scratch_bytes, w4a8=False, stream=None) -> int:
        """Raw status of a forward call with explicit (possibly invalid) arguments; for tests."""
        fn = lib.tmoe_forward_w4a8 if w4a8 else lib.tmoe_forward_w4a16
        wc = ctypes.byref(weights.c) if isinstance(weights, DeviceWeights) else weights
        return fn(self.handle, x, ids, w, T, wc, y, scratch, scratch_bytes, stream)

    def route_map(self, ids: torch.Tensor, scratch: torch.Tensor) -> native.RouteMap:
        T = ids.shape[0]
        view = native.RouteMap()
        check(lib.tmoe_build_route_map(self.handle, _ptr(ids), T, _ptr(scratch), scratch.numel(),
                                       ctypes.byref(view), _stream(ids.device)), "tmoe_build_route_map")
        return view

    def debug_decode(self, weights: DeviceWeights, expert: int, matrix: int, as_e4m3: bool = False) -> torch.Tensor:
        K, N = (self.hidden, 2 * self.inter) if matrix == 0 else (self.inter, self.hidden)
        dev = weights.payload.device
        out = torch.empty((K, N), dtype=torch.uint8 if as_e4m3 else torch.int16, device=dev)
        check(lib.tmoe_debug_decode(self.handle, ctypes.byref(weights.c), expert, matrix, int(as_e4m3), _ptr(out),
                                    _stream(dev)), "tmoe_debug_decode")
        return out

    def debug_views(self, T: int, w4a8: bool, scratch: torch.Tensor) -> native.DebugViews:
        v = native.DebugViews()
        check(lib.tmoe_debug_get_views(self.handle, T, int(w4a8), _ptr(scratch), scratch.numel(), ctypes.byref(v)),
              "tmoe_debug_get_views")
        return v


def debug_mxfp8(x: torch.Tensor):
    """MXFP8 quantization of an fp32 [rows, cols] device tensor with the forward's quantizer."""
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    e = torch.empty((rows, cols // 32), dtype=torch.uint8, device=x.device)
    check(lib.tmoe_debug_mxfp8(_ptr(x), rows, cols, _ptr(q), _ptr(e), _stream(x.device)), "tmoe_debug_mxfp8")
    return q, e


def debug_rotate(x: torch.Tensor) -> torch.Tensor:
    """Rotation R_n of each row of an fp32 [rows, n] device tensor, in place, with the forward's kernels."""
    rows, n = x.shape
    check(lib.tmoe_debug_rotate(_ptr(x), rows, n, _stream(x.device)), "tmoe_debug_rotate")
    return x


def scratch_view(scratch: torch.Tensor, ptr: int, shape, dtype) -> torch.Tensor:
    """View of `shape` elements of `dtype` at device address `ptr` inside the scratch tensor."""
    off = int(ptr) - scratch.data_ptr()
    n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
    if off < 0 or off + n > scratch.numel():
        raise ValueError("pointer outside the scratch arena")
    return scratch[off:off + n].view(dtype).view(shape)


class LinearWeightsDev:
    """Device copies of one dense trellis matrix: payload words, fp16 output scales and sign vectors."""

    FIELDS = ("payload", "scale", "su", "sv")

    def __init__(self, payload: torch.Tensor, scale, su, sv):
        self.payload, self.scale, self.su, self.sv = payload, scale, su, sv
        self._c = native.LinearWeights(*[t.data_ptr() for t in (payload, scale, su, sv)])

    @classmethod
    def from_inputs(cls, inp, device="cuda") -> "LinearWeightsDev":
        def up(a, dt):
            return torch.from_numpy(np.ascontiguousarray(a).view(dt)).to(device)
        return cls(up(inp.payload, np.int16), *[up(getattr(inp, n), np.float16) for n in ("scale", "su", "sv")])

    def clone(self) -> "LinearWeightsDev":
        return LinearWeightsDev(*[getattr(self, n).clone() for n in self.FIELDS])

    @property
    def c(self) -> native.LinearWeights:
        return self._c


class LinearPlan:
    """Dense trellis linear y = sv * R_N(scale * (C^T R_K(su * x))) (include/tmoe.h)."""

    def __init__(self, in_features: int, out_features: int, bits: int, max_tokens: int, rotation: str = "hadamard"):
        self.config = native.LinearConfig(in_features, out_features, bits, max_tokens,
                                          native.ROT_IDENTITY if rotation == "identity" else native.ROT_HADAMARD)
        handle = ctypes.c_void_p()
        sb, pw = ctypes.c_size_t(), ctypes.c_size_t()
        check(lib.tmoe_linear_plan(ctypes.byref(self.config), ctypes.byref(handle), ctypes.byref(sb),
                                   ctypes.byref(pw)), "tmoe_linear_plan")
        self.handle = handle
        self.scratch_bytes = sb.value
        self.payload_words = pw.value
        self.in_features, self.out_features, self.max_tokens = in_features, out_features, max_tokens

    @classmethod
    def for_inputs(cls, inp, max_tokens: Optional[int] = None, **kw) -> "LinearPlan":
        return cls(inp.in_features, inp.out_features, inp.bits, max_tokens or max(inp.tokens, 1), **kw)

    def close(self):
        if getattr(self, "handle", None) and self.handle.value:
            lib.tmoe_linear_plan_destroy(self.handle)
            self.handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def alloc_scratch(self, device="cuda") -> torch.Tensor:
        return torch.empty(self.scratch_bytes, dtype=torch.uint8, device=device)

    def forward(self, x: torch.Tensor, weights: LinearWeightsDev, scratch: torch.Tensor,
                y: Optional[torch.Tensor] = None) -> torch.Tensor:
        T = x.shape[0] if isinstance(x, torch.Tensor) and x.dim() == 2 else -1
        if y is None and isinstance(x, torch.Tensor):
            y = torch.empty((max(T, 0), self.out_features), dtype=torch.float32, device=x.device)
        self.check_call(x, weights, scratch, y)
        check(lib.tmoe_linear_w4a16(self.handle, _ptr(x), T, ctypes.byref(weights.c), _ptr(y), _ptr(scratch),
                                    scratch.numel(), _stream(x.device)), "tmoe_linear_w4a16")
        return y

    def check_call(self, x, weights, scratch, y) -> None:
        """Raise ValueError unless x is bf16 bits [T, K], y fp32 [T, N], the weights match the plan
        and scratch holds the planned bytes, all contiguous on one GPU device."""
        if not isinstance(x, torch.Tensor) or x.dim() != 2:
            raise ValueError("x: expected a 2-D tensor [T, K]")
        T = x.shape[0]
        if T > self.max_tokens:
            raise ValueError(f"x: {T} tokens, the plan holds at most {self.max_tokens}")
        K, N = self.in_features, self.out_features
        _require(x, "x", (T, K), _BITS16)
        _require(y, "y", (T, N), (torch.float32,))
        if not isinstance(weights, LinearWeightsDev):
            raise ValueError("weights: expected LinearWeightsDev")
        _require(weights.payload, "payload", (self.payload_words,), (torch.int16,))
        for name, n in (("scale", N), ("su", K), ("sv", N)):
            _require(getattr(weights, name), name, (n,), (torch.float16, torch.int16))
        _check_scratch(scratch, self.scratch_bytes)
        _same_device([("x", x), ("y", y), ("scratch", scratch)] +
                     [(n, getattr(weights, n)) for n in LinearWeightsDev.FIELDS])

    def forward_status(self, x, T, weights, y, scratch, scratch_bytes, stream=None) -> int:
        """Raw status of a call with explicit (possibly invalid) arguments; for tests."""
        wc = ctypes.byref(weights.c) if isinstance(weights, LinearWeightsDev) else weights
        return lib.tmoe_linear_w4a16(self.handle, x, T, wc, y, scratch, scratch_bytes, stream)
