"""Trellis decode inside the grouped GEMMs is bit-exact.

The layer's own FC1 (stage 1) and FC2 (stage 3) kernels run on operand rows that are one-hot: row
r of the FC1 input holds 1 at column k_r and 0 elsewhere, so output row r of the GEMM is row k_r
of the expert's decoded matrix, times 1, plus zeros: an exact fp32 sum. The split planes are added
(only one holds a nonzero term per element) and compared bit for bit with the oracle's decoded
fp16 codes (W4A16) or with their E4M3 roundings (W4A8: the one-hot operand is the E4M3 value 256
with the block scale 2^-8, so the product is exactly the weight operand). This grades the decode
as the GEMM kernels perform it -- their LDS-ring offsets, the second staging load of widths 5 and
6, the E4M3 lane mapping -- on every tile shape: 16-, 32- and 64-row wavefront tiles, 128-row
workgroup tiles of 128 and 256 columns, and the scaled-fp8 kernel. The channel scales are set to 1:
where a GEMM finishes its sums in one launch it applies the scale and rounds to fp16, which then
returns the code itself."""
import numpy as np
import pytest
import torch

import oracle_np as O
from gpu_cases import Case, e4m3_of_fp16_table, say
from trellis_quantized_moe_tmoe_amd.layer import scratch_view

pytestmark = pytest.mark.gpu

E4M3_256 = 0x78        # E4M3 encoding of 256.0
E8M0_2M8 = 119         # E8M0 encoding of 2^-8


def _e4m3_value(byte_codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(byte_codes, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float32).numpy()


class Probe:
    def __init__(self, case: Case, w4a8: bool):
        self.c, self.w4a8 = case, w4a8
        inp = case.inp
        self.R = inp.routes
        rm = O.route_map(inp.ids, inp.experts, 16)
        self.valid = int(rm["offsets"][-1])
        self.sorted = rm["sorted_routes"][: self.valid]
        self.flat_ids = inp.ids.reshape(-1)
        self.codes = {}
        self.halves = 0
        self.lut = e4m3_of_fp16_table() if w4a8 else None
        self.y = torch.empty((inp.tokens, inp.hidden), dtype=torch.float32, device="cuda")
        case.weights.scale1.fill_(1.0)
        case.weights.scale2.fill_(1.0)

    def expert(self, e):
        if e not in self.codes:
            self.codes[e] = O.expert_codes(self.c.inp, e)
        return self.codes[e]

    def stage(self, first, last):
        c = self.c
        c.plan.forward_stages(first, last, c.x, c.ids, c.w, c.weights, c.scratch, self.y, w4a8=self.w4a8)

    def _write_onehot(self, ptr, scale_ptr, pitch, K, ks):
        """Row i of the operand (i < R) gets the one-hot vector e_{ks[i]}."""
        c, R = self.c, self.R
        rows = torch.arange(R, device="cuda")
        kcol = torch.from_numpy(ks.astype(np.int64)).cuda()
        if not self.w4a8:
            a = scratch_view(c.scratch, ptr, (R, pitch), torch.float16)
            a.zero_()
            a[rows, kcol] = 1.0
        else:
            q = scratch_view(c.scratch, ptr, (R, K), torch.uint8)
            s = scratch_view(c.scratch, scale_ptr, (R, K // 32), torch.uint8)
            q.zero_()
            s.fill_(127)
            q[rows, kcol] = E4M3_256
            s[rows, kcol // 32] = E8M0_2M8

    def expected_row(self, e, matrix, k):
        codes = self.expert(e)[matrix][k]
        if not self.w4a8:
            return codes.view(np.float16).astype(np.float32)
        # a small negative code rounds to E4M3 -0, which the exact fp32 sum 0 + (-0) * 1 makes +0
        return _e4m3_value(self.lut[codes]) + np.float32(0.0)

    def check(self, matrix: int, salt: int) -> int:
        """FC1 (matrix 0) or FC2 (matrix 1) on one-hot rows; returns the number of rows compared."""
        c, R = self.c, self.R
        inp = c.inp
        H, I = inp.hidden, inp.inter
        K, N = (H, 2 * I) if matrix == 0 else (I, H)
        v = c.plan.debug_views(inp.tokens, self.w4a8, c.scratch)
        self.stage(0, 0)
        torch.cuda.synchronize()
        ks = (np.arange(R, dtype=np.int64) * (7 + 2 * salt) + 13 * salt) % K
        if matrix == 0:
            self._write_onehot(v.a1, v.a1_scale, v.a1_pitch, K, ks)
            self.stage(1, 1)
        else:
            self._write_onehot(v.b, v.b_scale, v.b_pitch, K, ks)
            self.stage(3, 3)
        torch.cuda.synchronize()
        splits = scratch_view(c.scratch, v.splits, (2,), torch.int32).cpu().numpy()
        half = scratch_view(c.scratch, v.half_planes, (2,), torch.int32).cpu().numpy()
        S = int(splits[matrix])
        if half[matrix]:                                # one fp16 plane, times the channel scale 1
            assert S == 1
            out = scratch_view(c.scratch, v.z if matrix == 0 else v.v, (R, N), torch.float16)
            got = out.double().cpu().numpy()
        else:
            out = scratch_view(c.scratch, v.z if matrix == 0 else v.v, (S, R, N), torch.float32)
            got = out.double().sum(0).cpu().numpy()
        self.halves += int(half[matrix])
        for p in range(self.valid):
            r = int(self.sorted[p])
            e = int(self.flat_ids[r])
            k = int(ks[r] if matrix == 0 else ks[p])    # FC1 reads rows by route, FC2 by slot
            want = self.expected_row(e, matrix, k)
            row = got[p].astype(np.float32)
            if not np.array_equal(row.view(np.uint32), want.view(np.uint32)):
                bad = np.nonzero(row != want)[0][:4]
                raise AssertionError(f"FC{matrix + 1} slot {p} route {r} expert {e} (bits {int(inp.bits[e])}) "
                                     f"k {k}: columns {bad.tolist()} got {row[bad]} want {want[bad]}")
        return self.valid


CASES = [
    # name, T, overrides, w4a8                                  kernel (16-row groups per tile)
    ("tiny", 4, dict(), False),                                # wavefront tiles, 16 rows
    ("tiny", 16, dict(), False),                               # 32 rows
    ("tiny", 64, dict(hidden=192, inter=128), False),          # 64 rows (no 128-row tile width)
    ("tiny", 64, dict(), False),                               # 128-row workgroup tiles, 256 columns
    ("tiny", 64, dict(hidden=384, inter=128), False),          # 128-row workgroup tiles, 128 columns
    ("tiny", 4, dict(bits_choices=(2, 3, 4)), False),          # mixed widths 2-4, 16 rows
    ("tiny", 16, dict(bits_choices=(2, 3, 4)), False),
    ("tiny", 64, dict(bits_choices=(2, 3, 4)), False),         # mixed widths, 128-row tiles
    ("tiny", 4, dict(bits_override=2), False),
    ("tiny", 64, dict(bits_override=3), False),
    ("tiny", 4, dict(bits_override=5), False),                 # widths 5 and 6: two staging loads
    ("tiny", 16, dict(bits_override=6), False),
    ("tiny", 64, dict(bits_override=5), False),                # 64-row tiles
    ("tiny", 16, dict(bits_choices=(2, 3, 4, 5, 6)), False),   # mixed widths 2-6
    ("decode", 16, dict(), False),                             # the decode geometry, 4 K splits
    ("prefill", 2048, dict(), False),                          # the prefill geometry, Zipf loads
    ("tiny", 4, dict(), True),                                 # scaled fp8, 16 rows
    ("tiny", 16, dict(), True),                                # 32 rows
    ("tiny", 64, dict(), True),                                # 64 rows
    ("tiny", 16, dict(bits_choices=(2, 3, 4)), True),          # mixed widths
    ("w4a8", 64, dict(), True),                                # the W4A8 geometry
]


@pytest.mark.parametrize("name,T,over,w4a8", CASES)
def test_gemm_decode_bit_exact(name, T, over, w4a8):
    c = Case(name, T, **over)
    pr = Probe(c, w4a8)
    n = 0
    for matrix in (0, 1):
        for salt in (0, 1):
            n += pr.check(matrix, salt)
    say(f"[result] {c.label} {'W4A8' if w4a8 else 'W4A16'} in-GEMM decode: {n} one-hot rows bit-exact "
        f"({pr.halves} of 4 checks on fp16 planes)")
