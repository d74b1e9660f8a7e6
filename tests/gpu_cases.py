"""Shared set-up for the GPU parity tests: one seeded case on the device plus its oracle."""
from __future__ import annotations

import functools
import sys

import numpy as np
import torch

import oracle_np as O
from trellis_quantized_moe_tmoe_amd.workloads import make_inputs

TOL_W4A16 = 1e-2          # max|y - y_ref| / max|y_ref|, the stated W4A16 bound
TOL_W4A8 = 3e-2           # the stated W4A8 bound against the W4A16 oracle
TOL_W4A8_EMU = 1e-2       # GPU W4A8 against the oracle's W4A8-emulating mode


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def rel_err(y, ref):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(y - ref)) / max(np.max(np.abs(ref)), 1e-30))


class Case:
    def __init__(self, name, tokens=None, ids_dtype=torch.int64, rotation="hadamard", max_tokens=None,
                 identity_signs=False, **over):
        from trellis_quantized_moe_tmoe_amd import layer as L
        self.L = L
        self.inp = make_inputs(name, tokens=tokens, identity_signs=identity_signs, **over)
        self.label = f"{name} T={self.inp.tokens} H={self.inp.hidden} I={self.inp.inter} E={self.inp.experts} " \
                     f"k={self.inp.top_k} seed={self.inp.seed}"
        say(f"[case] {self.label} ids={ids_dtype} rot={rotation}")
        self.plan = L.Plan.for_inputs(self.inp, max_tokens=max_tokens, rotation=rotation, ids_dtype=ids_dtype)
        self.weights = L.DeviceWeights.from_inputs(self.inp)
        self.x, self.ids, self.w = L.device_activations(self.inp, ids_dtype=ids_dtype)
        self.scratch = self.plan.alloc_scratch()
        self.rotation = rotation

    def run(self, w4a8=False, y=None):
        y = self.plan.forward(self.x, self.ids, self.w, self.weights, self.scratch, y=y, w4a8=w4a8)
        torch.cuda.synchronize()
        return y

    @functools.cached_property
    def oracle_w4a16(self):
        return O.forward(self.inp, identity=self.rotation == "identity")

    @functools.cached_property
    def oracle_w4a8(self):
        return O.forward(self.inp, mode="w4a8", identity=self.rotation == "identity")


@functools.lru_cache(maxsize=1)
def e4m3_of_fp16_table():
    """E4M3 byte of every fp16 bit pattern's value (oracle rounding), for vectorised expectations."""
    lib = O.lib()
    t = np.zeros(1 << 16, np.uint8)
    for h in range(1 << 16):
        v = lib.orc_half_to_double(h)
        if np.isfinite(v) and abs(v) <= 448:
            t[h] = lib.orc_double_to_e4m3(v)
    return t
