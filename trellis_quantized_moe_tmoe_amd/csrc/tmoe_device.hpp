// tmoe_device.hpp -- device building blocks shared by the HIP kernels (gfx950 / CDNA4).
//
//  * trellis window decode: 8 consecutive tile elements per lane, from two aligned 32-bit
//    loads, straight into a register operand (trellis3_t256 tiles, "integrate EXL3 Trellis into
//    the fused W4A16 API", review of prepare.py; codebook constants from the review of
//    intrinsics.py);
//  * fast Walsh-Hadamard butterflies over a wavefront (cross-lane stages via lane shuffles,
//    the rest inside registers), normalised per block (128-point scale 1/sqrt(128) as in the
//    review of kernel.py, _had128_quad);
//  * MXFP8 quantization with the exponent taken from the fp32 bits of amax/448 ("TrellisMX
//    (procedural NPK) ... P8 runtime", Precision notes).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tmoe {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef int i8v __attribute__((ext_vector_type(8)));
typedef short s2v __attribute__((ext_vector_type(2)));

struct ExpertInfo {          // written into scratch by the route-map kernel
  long long word_offset;     // first 16-bit word of the expert's region (FC1 then FC2)
  int bits;                  // 2, 3 or 4
  int pad;
};

// ------------------------------------------------------------------ trellis decode
// Codebook value of a 16-bit state s: m = ((s * 0xCBAC1FED) mod 2^32 & 0x8fff8fff) | 0x3b603b60,
// value = h(lo16(m)) + h(hi16(m)) rounded once to fp16. With s < 2^16 the 32-bit product splits
// into two 16 x 16 products that each fit 32 bits (so they map to the full-rate u24 multiply):
// s*0xCBAC1FED = s*0x1FED + ((s*0xCBAC) << 16) mod 2^32.
__device__ __forceinline__ _Float16 trellis_code(uint32_t s) {
  const uint32_t x = s * 0x1FEDu + ((s * 0xCBACu) << 16);
  const uint32_t m = (x & 0x8fff8fffu) | 0x3b603b60u;
  const _Float16 lo = __builtin_bit_cast(_Float16, static_cast<uint16_t>(m & 0xffffu));
  const _Float16 hi = __builtin_bit_cast(_Float16, static_cast<uint16_t>(m >> 16));
  return lo + hi;
}

// Two little-endian 16-bit words in one 32-bit load, as a big-endian (first word high) bit string.
__device__ __forceinline__ uint32_t be32(uint32_t w) { return (w << 16) | (w >> 16); }

// 32-bit word index j0 (floor((q*BITS - 2) / 4), may be -1) of the 64-bit window that covers the
// states of elements 8q .. 8q+7 of a tile: their bits span [8q*BITS + BITS - 16, 8q*BITS + 8*BITS).
template <int BITS>
__device__ __forceinline__ int window_word(int q) {
  if constexpr (BITS == 4) return q - 1;
  else if constexpr (BITS == 2) return (q - 1) >> 1;
  else return (q * BITS - 2) >> 2;
}

// Load the window of group q of the tile starting at `tile` (8*BITS 32-bit words): hi/lo are the
// big-endian halves of the 64 stream bits [32*j0, 32*j0 + 64), taken modulo the tile length.
template <int BITS>
__device__ __forceinline__ void load_window(const uint32_t* __restrict__ tile, int q, uint32_t& hi,
                                            uint32_t& lo) {
  constexpr int NW = 8 * BITS;
  const int j0 = window_word<BITS>(q);
  const int a = j0 < 0 ? j0 + NW : j0;
  const int b = (j0 + 1 == NW) ? 0 : j0 + 1;
  hi = tile[a];
  lo = tile[b];
}

// Decode elements 8q .. 8q+7 from a loaded window into fp16 codebook values.
template <int BITS>
__device__ __forceinline__ half8 decode8(uint32_t hi_raw, uint32_t lo_raw, int q) {
  const uint32_t hi = be32(hi_raw), lo = be32(lo_raw);
  const int j0 = window_word<BITS>(q);
  half8 r;
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    // the state of element 8q+jj ends at stream bit (8q+jj+1)*BITS; in the window that is
    // bit position end_rel from the top, so the state is (window >> (64 - end_rel)) & 0xffff.
    const int shift = 64 - ((8 * q + jj + 1) * BITS - 32 * j0);
    uint32_t w;
    if constexpr (BITS == 4) {
      w = __builtin_amdgcn_alignbit(hi, lo, 28 - 4 * jj);   // shift = 28 - 4*jj for every q
    } else {
      w = shift >= 32 ? (hi >> (shift - 32)) : __builtin_amdgcn_alignbit(hi, lo, shift);
    }
    r[jj] = trellis_code(w & 0xffffu);
  }
  return r;
}

// fp16 -> E4M3 (round to nearest even) of two values, packed in the low 16 bits.
__device__ __forceinline__ uint32_t fp8x2_from_half2(half2v v) {
  s2v old = {0, 0};
  s2v r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(old, v, 1.0f, false);
  return static_cast<uint32_t>(static_cast<uint16_t>(r[0]));
}

// fp32 -> E4M3 (round to nearest even) of two values, packed in the low 16 bits.
__device__ __forceinline__ uint32_t fp8x2_from_f32(float a, float b) {
  s2v old = {0, 0};
  s2v r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(old, a, b, 1.0f, false);
  return static_cast<uint32_t>(static_cast<uint16_t>(r[0]));
}

// Eight fp16 codes -> eight E4M3 bytes (two 32-bit words).
__device__ __forceinline__ void fp8x8_from_half8(half8 h, uint32_t& w0, uint32_t& w1) {
  half2v p0 = {h[0], h[1]}, p1 = {h[2], h[3]}, p2 = {h[4], h[5]}, p3 = {h[6], h[7]};
  w0 = fp8x2_from_half2(p0) | (fp8x2_from_half2(p1) << 16);
  w1 = fp8x2_from_half2(p2) | (fp8x2_from_half2(p3) << 16);
}

// ------------------------------------------------------------------ conversions
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ float h2f(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// ------------------------------------------------------------------ wavefront FWHT
// A row segment of 64*EPL values lives in a wavefront with element e = i*64 + lane in v[i].
// The butterflies of the Walsh-Hadamard transform in natural order commute, so the cross-lane
// strides 1..32 and the in-register strides 64..32*EPL can run in any order.
template <int EPL>
__device__ __forceinline__ void fwht_segment(float (&v)[EPL], int lane) {
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const float p = __shfl_xor(v[i], s, 64);
      v[i] = (lane & s) ? (p - v[i]) : (v[i] + p);
    }
  }
#pragma unroll
  for (int t = 1; t < EPL; t <<= 1) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      if ((i & t) == 0) {
        const float a = v[i], b = v[i | t];
        v[i] = a + b;
        v[i | t] = a - b;
      }
    }
  }
  // 1/sqrt(64*EPL), rounded once to fp32 from the exact value
  constexpr float kScale = (EPL == 1) ? 0.125f : (EPL == 2) ? 0.08838834764831845f
                         : (EPL == 4) ? 0.0625f : (EPL == 8) ? 0.04419417382415922f
                         : (EPL == 16) ? 0.03125f : (EPL == 32) ? 0.02209708691207961f
                         : 0.015625f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) v[i] *= kScale;
}

// ------------------------------------------------------------------ MXFP8
// E8M0 exponent of a block with maximum magnitude amax: ceil(log2(fp32(amax / 448))) from the
// quotient's bits, -127 for a zero or subnormal quotient, clamped to [-127, 127].
__device__ __forceinline__ int mx_exponent(float amax) {
  const float q = amax / 448.0f;
  const uint32_t u = __float_as_uint(q);
  const int field = static_cast<int>((u >> 23) & 0xffu);
  if (field == 0) return -127;
  int e = field - 127 + ((u & 0x7fffffu) != 0 ? 1 : 0);
  return e > 127 ? 127 : e;
}

// Maximum of |v| over the 32-lane half of the wavefront this lane belongs to.
__device__ __forceinline__ float half_wave_amax(float v) {
  float a = fabsf(v);
#pragma unroll
  for (int s = 1; s < 32; s <<= 1) a = fmaxf(a, __shfl_xor(a, s, 64));
  return a;
}

}  // namespace tmoe
