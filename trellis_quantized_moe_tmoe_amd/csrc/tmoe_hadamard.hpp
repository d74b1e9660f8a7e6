// tmoe_hadamard.hpp -- Walsh-Hadamard transforms of 512- and 1024-value rows on the matrix cores
// (v_mfma_f32_16x16x32_f16 / 16x16x16f16), for the activation and the combine at large batches
// (one fp16 GEMM plane): the same orthonormal rotations the wavefront butterflies of tmoe_device.hpp
// compute, with every stage summing in fp32 and rounding its output once to fp16 for the next stage.
// Where a few wavefronts carry the whole launch (small batches, the route map's rotation) the chain
// of dependent MFMA stages costs more than the butterflies' VALU work, so those keep the butterflies.
#pragma once
#include "tmoe_device.hpp"

namespace tmoe {

// With element i = 32a + b (a < 16, b < 32) the transform is H_16 (x) H_32: Y[a'][b'] = sum over a, b
// of H16[a'][a] H32[b'][b] X[a][b]. Four 16x16 MFMA stages carry it, each taking the previous
// output layout as it stands: a C tile (lane l: rows 4(l/16)+[0,4), column l%16) is a K = 16
// operand over its rows, as the B operand of the next product or, read as rows = its column, as the
// A operand; the constant operands absorb the order of the K values. The forward transform of a row
// in memory contracts b (A = the row, lane l: elements 32(l%16) + 8(l/16) + [0,8)), then a, leaving
// the "C2" layout: tile h, value i of lane l is element 32(4(l/16)+i) + 16h + l%16. A transform of
// values in the C2 layout contracts a (A = the C2 tile), then b, leaving tile h, value i of lane l
// as element 32(l%16) + 16h + 4(l/16) + i. Entries of H are +-1 (exact in fp16); every stage sums
// in fp32 and hands its output to the next stage rounded once to fp16.
namespace hmfma {
constexpr uint32_t hbit(int i, int j) { return (__builtin_popcount(i & j) & 1) ? 0xBC00u : 0x3C00u; }
constexpr int stage4_k(int q, int r) { return r < 4 ? 4 * q + r : 16 + 4 * q + r - 4; }
// per lane, fp16 pairs: [0, 2) H16[l%16][4(l/16)+r] (A of the a-contraction of the forward
// transform, B of the second transform's); [2, 10) H32[16h + l%16][8(l/16)+r] for h = 0, 1 (B of
// the b-contraction of the forward transform); [10, 18) H32[16h + l%16][stage4_k(l/16, r)] (A of the
// second transform's b-contraction, whose K values arrive as rows 4(l/16)+[0,4) of both C tiles)
struct Table {
  uint32_t w[64][20];
};
constexpr Table make_table() {
  Table t{};
  for (int l = 0; l < 64; ++l) {
    const int c = l % 16, q = l / 16;
    for (int pr = 0; pr < 2; ++pr) t.w[l][pr] = hbit(c, 4 * q + 2 * pr) | (hbit(c, 4 * q + 2 * pr + 1) << 16);
    for (int h = 0; h < 2; ++h)
      for (int pr = 0; pr < 4; ++pr) {
        t.w[l][2 + 4 * h + pr] = hbit(16 * h + c, 8 * q + 2 * pr) | (hbit(16 * h + c, 8 * q + 2 * pr + 1) << 16);
        t.w[l][10 + 4 * h + pr] =
            hbit(16 * h + c, stage4_k(q, 2 * pr)) | (hbit(16 * h + c, stage4_k(q, 2 * pr + 1)) << 16);
      }
  }
  return t;
}
__device__ const Table kTable = make_table();

typedef _Float16 half4v __attribute__((ext_vector_type(4)));
typedef uint32_t u2v __attribute__((ext_vector_type(2)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ half4v to_half4(f4 v) {
  return half4v{static_cast<_Float16>(v[0]), static_cast<_Float16>(v[1]), static_cast<_Float16>(v[2]),
                static_cast<_Float16>(v[3])};
}

struct Operands {
  half4v h16;
  half8 h32b[2], h32a[2];
};

__device__ __forceinline__ Operands load_operands(int lane) {
  const u4v* src = reinterpret_cast<const u4v*>(kTable.w[lane]);
  const u4v w0 = src[0], w1 = src[1], w2 = src[2], w3 = src[3], w4 = src[4];
  Operands o;
  o.h16 = __builtin_bit_cast(half4v, u2v{w0[0], w0[1]});
  o.h32b[0] = __builtin_bit_cast(half8, u4v{w0[2], w0[3], w1[0], w1[1]});
  o.h32b[1] = __builtin_bit_cast(half8, u4v{w1[2], w1[3], w2[0], w2[1]});
  o.h32a[0] = __builtin_bit_cast(half8, u4v{w2[2], w2[3], w3[0], w3[1]});
  o.h32a[1] = __builtin_bit_cast(half8, u4v{w3[2], w3[3], w4[0], w4[1]});
  return o;
}

// Forward transform (unscaled) of the row whose A operand the lane holds: out[h] = C2 tile h.
__device__ __forceinline__ void forward(const Operands& o, half8 x, f4 (&out)[2]) {
  const f4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const f4 c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(x, o.h32b[h], z, 0, 0, 0);
    out[h] = __builtin_amdgcn_mfma_f32_16x16x16f16(o.h16, to_half4(c1), z, 0, 0, 0);
  }
}

// 1024-point transform (unscaled) of a row in memory, H_32 (x) H_32 with element i = 32a + b: x[ha]
// holds rows a = 16 ha + l%16, elements 8(l/16) + [0,8) of each; out[ha][hb] is the C tile of rows
// a' = 16 ha + 4(l/16) + [0,4), column b' = 16 hb + l%16 (element 32a' + b').
__device__ __forceinline__ void forward1024(const Operands& o, const half8 (&x)[2], f4 (&out)[2][2]) {
  const f4 z = {0.f, 0.f, 0.f, 0.f};
  f4 c1[2][2];
#pragma unroll
  for (int ha = 0; ha < 2; ++ha)
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) c1[ha][hb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(x[ha], o.h32b[hb], z, 0, 0, 0);
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    // K = a over both row tiles: rows 4(l/16)+[0,4) of tile 0, then of tile 1 (the order h32a assumes)
    const half4v lo = to_half4(c1[0][hb]), hi = to_half4(c1[1][hb]);
    const half8 bk = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
    for (int ha = 0; ha < 2; ++ha) out[ha][hb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(o.h32a[ha], bk, z, 0, 0, 0);
  }
}

// Transform (unscaled) of values in the C2 layout: out[h] = tile h of the second transform's layout.
__device__ __forceinline__ void from_c2(const Operands& o, const f4 (&v)[2], f4 (&out)[2]) {
  const f4 z = {0.f, 0.f, 0.f, 0.f};
  f4 c3[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) c3[h] = __builtin_amdgcn_mfma_f32_16x16x16f16(to_half4(v[h]), o.h16, z, 0, 0, 0);
  const half4v lo = to_half4(c3[0]), hi = to_half4(c3[1]);
  const half8 b = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
  for (int h = 0; h < 2; ++h) out[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(o.h32a[h], b, z, 0, 0, 0);
}

}  // namespace hmfma

}  // namespace tmoe
