"""C ABI checks that need no GPU: exported symbols and fail-closed host validation.

Validation happens before any launch (the Summary of 'serve canonical Fruit QSRT atoms' (b12x PR
#129) rejects bad layouts and route maps up front; the description of 'TrellisMX (procedural NPK)
... P8 runtime' (flashinfer PR #69) rejects a short or misaligned arena), so every call below
returns before touching a (fake) device pointer."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    src = open(os.path.join(ROOT, "include", "tmoe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tmoe_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def N():
    from trellis_quantized_moe_tmoe_amd import native
    return native


def test_library_exports_every_declared_symbol(N):
    declared = _declared_symbols()
    assert len(declared) >= 12
    for name in declared:
        assert hasattr(N.lib, name), name
    assert sorted(N.EXPORTS) == declared


def _cfg(N, bits, **kw):
    d = dict(hidden=1024, inter=512, num_experts=len(bits), top_k=8, max_tokens=16, rotation=0, ids_dtype=1,
             block_m=0)
    d.update(kw)
    arr = (ctypes.c_uint8 * len(bits))(*bits)
    c = N.Config(d["hidden"], d["inter"], d["num_experts"], d["top_k"], d["max_tokens"],
                 ctypes.cast(arr, ctypes.POINTER(ctypes.c_uint8)), d["rotation"], d["ids_dtype"], d["block_m"])
    return c, arr


def _plan(N, bits, **kw):
    c, keep = _cfg(N, bits, **kw)
    h = ctypes.c_void_p()
    sb, pw = ctypes.c_size_t(), ctypes.c_size_t()
    st = N.lib.tmoe_plan(ctypes.byref(c), ctypes.byref(h), ctypes.byref(sb), ctypes.byref(pw))
    return st, h, sb.value, pw.value


@pytest.mark.parametrize("kw,status", [
    (dict(hidden=1000), 2), (dict(inter=96), 2), (dict(hidden=8192), 2), (dict(hidden=0), 1),
    (dict(top_k=0), 1), (dict(top_k=33), 2), (dict(max_tokens=0), 1), (dict(rotation=2), 1),
    (dict(ids_dtype=3), 1), (dict(block_m=24), 1), (dict(block_m=48), 0), (dict(hidden=2560, inter=320), 0),
])
def test_plan_validation(N, kw, status):
    st, h, _, _ = _plan(N, [4] * 8, **kw)
    assert st == status
    if st == 0:
        assert N.lib.tmoe_plan_destroy(h) == 0


@pytest.mark.parametrize("bits,status", [([4, 3, 2], 0), ([4, 5], 0), ([6, 5, 2], 0), ([7], 2), ([1], 2),
                                         ([0], 1), ([17], 1)])
def test_plan_bit_widths(N, bits, status):
    assert _plan(N, bits)[0] == status


def test_plan_too_many_experts(N):
    assert _plan(N, [4] * 513)[0] == 2


def test_payload_words_and_offsets(N):
    bits = [4, 3, 2, 4]
    st, h, sb, pw = _plan(N, bits, hidden=2560, inter=320)
    assert st == 0
    per_bit = 3 * 2560 * 320 // 16
    assert pw == per_bit * sum(bits)
    off = ctypes.c_size_t()
    for e, want in enumerate(np.concatenate([[0], np.cumsum(bits)[:-1]]) * per_bit):
        assert N.lib.tmoe_plan_expert_offset(h, e, ctypes.byref(off)) == 0 and off.value == want
    assert N.lib.tmoe_plan_expert_offset(h, 4, ctypes.byref(off)) == 1
    info = N.PlanInfo()
    assert N.lib.tmoe_plan_get_info(h, ctypes.byref(info)) == 0 and info.scratch_bytes == sb
    N.lib.tmoe_plan_destroy(h)


def test_forward_fails_closed_before_any_launch(N):
    st, h, sb, _ = _plan(N, [4] * 8)
    fake = 1 << 20                                # never dereferenced: validation returns first
    w = N.Weights(*([fake] * 7))
    fw = N.lib.tmoe_forward_w4a16
    args = lambda **o: [h, o.get("x", fake), o.get("ids", fake), o.get("w", fake), o.get("T", 4),
                        ctypes.byref(o.get("wt", w)), o.get("y", fake), o.get("scratch", fake),
                        o.get("bytes", sb), None]
    assert fw(*args(T=17)) == 4                   # above capacity
    assert fw(*args(T=-1)) == 1
    assert fw(*args(T=0)) == 0                    # nothing to do, nothing launched
    assert fw(*args(bytes=sb - 1)) == 3           # short arena
    assert fw(*args(scratch=fake + 8)) == 3       # arena not 16-byte aligned
    assert fw(*args(scratch=0)) == 3
    assert fw(*args(ids=0)) == 1
    assert fw(*args(ids=fake + 4)) == 5           # int64 ids need 8-byte alignment
    assert fw(*args(x=0)) == 1
    assert fw(*args(y=fake + 4)) == 5
    assert fw(*args(wt=N.Weights(*([fake] * 6 + [0])))) == 1
    assert N.lib.tmoe_forward_w4a8(*args(T=17)) == 4
    N.lib.tmoe_plan_destroy(h)


def test_w4a8_needs_128_multiples(N):
    st, h, sb, _ = _plan(N, [4] * 8, hidden=2560, inter=320)
    fake = 1 << 20
    w = N.Weights(*([fake] * 7))
    assert N.lib.tmoe_forward_w4a8(h, fake, fake, fake, 2, ctypes.byref(w), fake, fake, sb, None) == 2
    N.lib.tmoe_plan_destroy(h)


def test_route_map_and_debug_validation(N):
    st, h, sb, _ = _plan(N, [4] * 8)
    view = N.RouteMap()
    fake = 1 << 20
    assert N.lib.tmoe_build_route_map(h, fake, 17, fake, sb, ctypes.byref(view), None) == 4
    assert N.lib.tmoe_build_route_map(h, fake, 2, fake, sb - 16, ctypes.byref(view), None) == 3
    assert N.lib.tmoe_build_route_map(h, fake, 2, fake, sb, None, None) == 1
    w = N.Weights(*([fake] * 7))
    assert N.lib.tmoe_debug_decode(h, ctypes.byref(w), 8, 0, 0, fake, None) == 1
    assert N.lib.tmoe_debug_decode(h, ctypes.byref(w), 0, 2, 0, fake, None) == 1
    assert N.lib.tmoe_debug_mxfp8(fake, 4, 48, fake, fake, None) == 1
    assert N.lib.tmoe_debug_rotate(fake, 4, 100, None) == 2
    v = N.DebugViews()
    assert N.lib.tmoe_debug_get_views(h, 17, 0, fake, sb, ctypes.byref(v)) == 4
    assert N.lib.tmoe_debug_get_views(h, 4, 0, fake, sb, ctypes.byref(v)) == 0
    assert v.splits and v.a1 == fake + (v.a1 - fake)
    assert v.a1_pitch >= 1024 and v.b_pitch >= 512
    assert N.lib.tmoe_debug_get_views(h, 4, 1, fake, sb, ctypes.byref(v)) == 0
    assert (v.a1_pitch, v.b_pitch) == (1024, 512)
    assert N.lib.tmoe_status_str(3).decode().startswith("scratch")
    N.lib.tmoe_plan_destroy(h)


def _linear_plan(N, **kw):
    d = dict(in_features=1024, out_features=1024, bits=4, max_tokens=16, rotation=0)
    d.update(kw)
    c = N.LinearConfig(d["in_features"], d["out_features"], d["bits"], d["max_tokens"], d["rotation"])
    h = ctypes.c_void_p()
    sb, pw = ctypes.c_size_t(), ctypes.c_size_t()
    st = N.lib.tmoe_linear_plan(ctypes.byref(c), ctypes.byref(h), ctypes.byref(sb), ctypes.byref(pw))
    return st, h, sb.value, pw.value


@pytest.mark.parametrize("kw,status", [
    (dict(), 0), (dict(in_features=2560, out_features=320, bits=3), 0), (dict(in_features=1000), 2),
    (dict(out_features=48), 2), (dict(out_features=8192), 2), (dict(bits=5), 0), (dict(bits=6), 0),
    (dict(bits=7), 2), (dict(bits=0), 1),
    (dict(bits=17), 1), (dict(max_tokens=0), 1), (dict(rotation=2), 1), (dict(in_features=-64), 1),
])
def test_linear_plan_validation(N, kw, status):
    st, h, sb, pw = _linear_plan(N, **kw)
    assert st == status
    if st == 0:
        K = kw.get("in_features", 1024)
        Nf = kw.get("out_features", 1024)
        assert pw == (K // 16) * (Nf // 16) * 16 * kw.get("bits", 4)
        assert sb > 0
        assert N.lib.tmoe_linear_plan_destroy(h) == 0


def test_linear_fails_closed_before_any_launch(N):
    """Bad arguments return an error before any device pointer (all fake here) is touched."""
    st, h, sb, _ = _linear_plan(N, max_tokens=16)
    assert st == 0
    fake = ctypes.c_void_p(0x1000)
    w = N.LinearWeights(0x1000, 0x1000, 0x1000, 0x1000)
    call = N.lib.tmoe_linear_w4a16
    assert call(h, fake, 17, ctypes.byref(w), fake, fake, sb, None) == 4          # T > max_tokens
    assert call(h, fake, -1, ctypes.byref(w), fake, fake, sb, None) == 1          # T < 0
    assert call(h, fake, 4, ctypes.byref(w), fake, fake, sb - 1, None) == 3       # short arena
    assert call(h, fake, 4, ctypes.byref(w), fake, ctypes.c_void_p(0x1008), sb, None) == 3   # misaligned arena
    assert call(h, fake, 4, None, fake, fake, sb, None) == 1                      # no weights
    assert call(h, ctypes.c_void_p(0x1002), 4, ctypes.byref(w), fake, fake, sb, None) == 5  # x misaligned
    bad = N.LinearWeights(0x1000, 0x1001, 0x1000, 0x1000)
    assert call(h, fake, 4, ctypes.byref(bad), fake, fake, sb, None) == 5         # odd fp16 pointer
    assert call(h, fake, 0, ctypes.byref(w), fake, fake, sb, None) == 0           # T = 0: nothing
    assert call(None, fake, 4, ctypes.byref(w), fake, fake, sb, None) == 1
    assert N.lib.tmoe_linear_plan_destroy(h) == 0


def test_w4a8_rejects_widths_above_four(N):
    """The fp8 path decodes widths 2-4; a plan holding a 5- or 6-bit expert runs W4A16 only."""
    st, h, sb, _ = _plan(N, [4, 5, 4, 6])
    assert st == 0
    fake = 1 << 20
    w = N.Weights(*([fake] * 7))
    args = [h, fake, fake, fake, 4, ctypes.byref(w), fake, fake, sb, None]
    assert N.lib.tmoe_forward_w4a8(*args) == 2
    N.lib.tmoe_plan_destroy(h)


def test_static_entry_point_rejects_plans_beyond_its_arena(N):
    # prefill capacity (2048 tokens, top-8) needs about 184 MiB of scratch: rejected on the host
    # before any HIP call, so this runs without a GPU
    st, h, sb, _ = _plan(N, [4] * 96, max_tokens=2048)
    assert st == 0 and sb > N.STATIC_SCRATCH_BYTES
    w = N.Weights(*([16] * 7))
    assert N.lib.tmoe_forward_w4a16_static(h, 16, 16, 16, 4, ctypes.byref(w), 16, None) == 7
    assert N.lib.tmoe_status_str(7).decode().startswith("plan needs more scratch")
    st2, h2, sb2, _ = _plan(N, [4] * 96, max_tokens=16)
    assert st2 == 0 and sb2 <= N.STATIC_SCRATCH_BYTES
    # T = 0 returns at once, before the device lookup
    assert N.lib.tmoe_forward_w4a16_static(h2, 16, 16, 16, 0, ctypes.byref(w), 16, None) == 0
    assert N.lib.tmoe_plan_destroy(h) == 0 and N.lib.tmoe_plan_destroy(h2) == 0
