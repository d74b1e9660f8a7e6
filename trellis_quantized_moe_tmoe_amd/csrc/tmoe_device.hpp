// tmoe_device.hpp -- device building blocks shared by the HIP kernels (gfx950 / CDNA4).
//
//  * trellis window decode: 8 consecutive tile elements per lane, from two or three aligned 32-bit
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
  int bits;                  // 2..6
  int pad;
};

// ------------------------------------------------------------------ trellis decode
// Codebook value of a 16-bit state s: m = ((s * 0xCBAC1FED) mod 2^32 & 0x8fff8fff) | 0x3b603b60,
// value = h(lo16(m)) + h(hi16(m)) rounded once to fp16 (round to nearest even). The multiply is a
// full-rate v_mul_lo_u32 on gfx950; mask and OR are one v_and_or_b32; the half + half sum is one
// SDWA add that reads both halves of m and writes straight into one half of a packed operand.
constexpr uint32_t kMcgMul = 0xCBAC1FEDu;
constexpr uint32_t kMcgMask = 0x8fff8fffu;
constexpr uint32_t kMcgOr = 0x3b603b60u;

__device__ __forceinline__ uint32_t mcg_bits(uint32_t s, uint32_t mask, uint32_t orv) {
  const uint32_t x = s * kMcgMul;
  uint32_t m;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(m) : "v"(x), "v"(mask), "s"(orv));
  return m;
}

// Two codebook values from their m words, packed as (value of ma) | (value of mb) << 16.
__device__ __forceinline__ uint32_t code_pair(uint32_t ma, uint32_t mb) {
  uint32_t r;
  asm("v_add_f16_sdwa %0, %1, %1 dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:WORD_0 src1_sel:WORD_1\n\t"
      "v_add_f16_sdwa %0, %2, %2 dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:WORD_0 src1_sel:WORD_1"
      : "=&v"(r)
      : "v"(ma), "v"(mb));
  return r;
}

// Codebook value of one state (scalar path, used where a single value is needed).
__device__ __forceinline__ _Float16 trellis_code(uint32_t s) {
  const uint32_t m = ((s * kMcgMul) & kMcgMask) | kMcgOr;
  const _Float16 lo = __builtin_bit_cast(_Float16, static_cast<uint16_t>(m & 0xffffu));
  const _Float16 hi = __builtin_bit_cast(_Float16, static_cast<uint16_t>(m >> 16));
  return lo + hi;
}

// Two little-endian 16-bit words in one 32-bit load, as a big-endian (first word high) bit string.
__device__ __forceinline__ uint32_t be32(uint32_t w) { return __builtin_amdgcn_alignbit(w, w, 16); }

// ---- state windows
// The states of elements 8q .. 8q+7 of a tile (group q) are the 16-bit stream fields starting at
// bits s0 + jj*BITS, jj = 0..7, with s0 = 8q*BITS + BITS - 16 (taken modulo the tile's 256*BITS
// bits). A lane reads the 32-bit words j0 .. j0 + dec_words - 1 (modulo the tile) that hold them.
//  * 4 bits: j0 = q - 1 (the fields then end at fixed offsets of two words; see prep_window4);
//  * other widths: j0 = floor((s0 - 1) / 32). The lane shifts the words once into a window that
//    starts at s0 itself (a funnel shift by dec_shift, the same for every step of the lane), so
//    every field sits at a fixed offset jj*BITS of the window and takes one bit-field extract. The
//    window spans 64 bits (three words; two for width 2, whose fields span 30 bits), and the 8
//    fields span 7*BITS + 16 <= 58 bits of it.
template <int BITS>
constexpr int dec_words() { return BITS == 4 || BITS == 2 ? 2 : 3; }

template <int BITS>
__device__ __forceinline__ int dec_first_word(int q) {
  if constexpr (BITS == 4) return q - 1;
  else return (8 * q * BITS + BITS - 17) >> 5;       // arithmetic shift: floor, -1 for q = 0
}

// Right-shift amount of the funnel shift that starts the window at s0 (0..31; unused at 4 bits).
template <int BITS>
__device__ __forceinline__ uint32_t dec_shift(int q) {
  const int s0 = 8 * q * BITS + BITS - 16;
  return static_cast<uint32_t>(32 - (s0 - 32 * dec_first_word<BITS>(q)));
}

// Read group q's words from a tile of 8*BITS 32-bit words (raw, as stored).
template <int BITS>
__device__ __forceinline__ void load_dec_words(const uint32_t* __restrict__ tile, int q,
                                               uint32_t (&w)[dec_words<BITS>()]) {
  constexpr int NW = 8 * BITS;
  const int j0 = dec_first_word<BITS>(q);
#pragma unroll
  for (int i = 0; i < dec_words<BITS>(); ++i) w[i] = tile[(j0 + i + NW) % NW];
}

// 4 bits: the big-endian strings X = w[2q-1]:w[2q] and L = w[2q]:w[2q+1] plus the raw low word.
struct Window4 {
  uint32_t x, l, raw_lo;
};

__device__ __forceinline__ Window4 prep_window4(uint32_t hi_raw, uint32_t lo_raw) {
  // words: hi_raw = w[2q-2] | w[2q-1] << 16, lo_raw = w[2q] | w[2q+1] << 16 (little endian)
  Window4 w;
  w.x = __builtin_amdgcn_perm(hi_raw, lo_raw, 0x07060100u);   // bytes: lo.0 lo.1 hi.2 hi.3
  w.l = be32(lo_raw);
  w.raw_lo = lo_raw;
  return w;
}

// The 16-bit states of group q from its words (raw, as stored); sh = dec_shift<BITS>(q).
template <int BITS>
__device__ __forceinline__ void group_states(const uint32_t (&w)[dec_words<BITS>()], uint32_t sh, uint32_t (&st)[8]) {
  if constexpr (BITS == 4) {
    // the state of element 8q+j is the 16 stream bits ending at 4(8q+j+1): X >> (12-4j) for j < 3,
    // L >> (28-4j) for 4 <= j < 7, and the raw half-words for j = 3 and 7
    const Window4 v = prep_window4(w[0], w[1]);
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      if (jj == 3) st[jj] = v.raw_lo & 0xffffu;
      else if (jj == 7) st[jj] = v.raw_lo >> 16;
      else st[jj] = jj < 3 ? __builtin_amdgcn_ubfe(v.x, 12 - 4 * jj, 16) : __builtin_amdgcn_ubfe(v.l, 28 - 4 * jj, 16);
    }
  } else {
    // window bits [0, 32) in X, [32, 64) in L, [16, 48) in M (bit 0 = the window's first stream bit,
    // held in bit 31 of X); field jj starts at window bit o = jj*BITS
    const uint32_t w0 = be32(w[0]), w1 = be32(w[1]);
    const uint32_t X = __builtin_amdgcn_alignbit(w0, w1, sh);
    uint32_t L = 0, M = 0;
    if constexpr (dec_words<BITS>() == 3) {
      L = __builtin_amdgcn_alignbit(w1, be32(w[2]), sh);
      M = __builtin_amdgcn_alignbit(X, L, 16);
    }
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int o = jj * BITS;
      if (o <= 16) st[jj] = __builtin_amdgcn_ubfe(X, 16 - o, 16);
      else if (o <= 32) st[jj] = __builtin_amdgcn_ubfe(M, 32 - o, 16);
      else st[jj] = __builtin_amdgcn_ubfe(L, 48 - o, 16);
    }
  }
}

// Decode group q into four packed fp16 pairs (element 8q+2i in the low half of p[i]).
template <int BITS>
__device__ __forceinline__ void decode8_pairs(const uint32_t (&w)[dec_words<BITS>()], uint32_t sh, uint32_t mask,
                                              uint32_t orv, uint32_t (&p)[4]) {
  uint32_t st[8];
  group_states<BITS>(w, sh, st);
  uint32_t m[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) m[j] = mcg_bits(st[j], mask, orv);
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = code_pair(m[2 * i], m[2 * i + 1]);
}

template <int BITS>
__device__ __forceinline__ half8 decode8(const uint32_t (&w)[dec_words<BITS>()], uint32_t sh, uint32_t mask,
                                         uint32_t orv) {
  uint32_t p[4];
  decode8_pairs<BITS>(w, sh, mask, orv, p);
  typedef uint32_t u4v __attribute__((ext_vector_type(4)));
  const u4v v = {p[0], p[1], p[2], p[3]};
  return __builtin_bit_cast(half8, v);
}

// The mask and OR constants live in registers for v_and_or_b32 (no 32-bit literal in VOP3 here);
// loading them through an opaque move keeps them from being folded back into two instructions.
__device__ __forceinline__ uint32_t vreg_const(uint32_t c) {
  uint32_t r;
  asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(c));
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

// Two packed fp16 pairs -> four E4M3 bytes in one word (pa's values in bytes 0-1, pb's in 2-3);
// the second conversion writes the high half and keeps the low one. The first starts from pa's own
// bits (its high half is overwritten), so no register has to be cleared for it.
__device__ __forceinline__ uint32_t fp8x4_from_pairs(uint32_t pa, uint32_t pb) {
  s2v r = __builtin_bit_cast(s2v, pa);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(r, __builtin_bit_cast(half2v, pa), 1.0f, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(r, __builtin_bit_cast(half2v, pb), 1.0f, true);
  return __builtin_bit_cast(uint32_t, r);
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
// strides 1..32 and the in-register strides 64..32*EPL can run in any order. Cross-lane partners
// come from DPP (strides 1, 2, 8), ds_swizzle (4, 16) and one lane permute (32). A lane stage
// computes own + sign * partner (sign = -1 on the lane holding the upper element), which is the
// butterfly's lower output on the lower lane and the negated upper output on the upper lane; the
// partner is the multiplicand, so a DPP partner folds into the fused multiply-add (one instruction
// per value). After the six lane stages lane l holds (-1)^popcount(l) times its true values (a sign
// that passes unchanged through the in-register stages, which are linear), and the final scale
// carries that sign. Every value has the same bits as the plain butterflies give: each add or
// subtract is the same one, up to an exact negation.
template <int S>
__device__ __forceinline__ float lane_partner(float v) {
  const int x = __float_as_int(v);
  int r;
  if constexpr (S == 1) r = __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, true);        // quad_perm 1,0,3,2
  else if constexpr (S == 2) r = __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, true);   // quad_perm 2,3,0,1
  else if constexpr (S == 4) r = __builtin_amdgcn_ds_swizzle(x, 0x1F | (4 << 10));          // lane ^ 4
  else if constexpr (S == 8) r = __builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, true);  // row_ror 8
  else if constexpr (S == 16) r = __builtin_amdgcn_ds_swizzle(x, 0x1F | (16 << 10));        // lane ^ 16
  else r = __shfl_xor(x, 32, 64);
  return __int_as_float(r);
}

// v[i] += (v[i] of the DPP partner lane) * sg for N values, one v_fmac_f32 with a DPP source each
// (the compiler keeps the DPP move separate). The leading s_nop gives the two wait states a DPP read
// needs after a VALU write of its source register; every source is written before the statement.
#define TMOE_FMAC_DPP(I, N, CTRL) "v_fmac_f32_dpp %" #I ", %" #I ", %" #N " " CTRL " row_mask:0xf bank_mask:0xf\n"
#define TMOE_DPP_STAGE(CTRL)                                                                             \
  do {                                                                                                   \
    if constexpr (N == 8) {                                                                              \
      asm("s_nop 1\n" TMOE_FMAC_DPP(0, 8, CTRL) TMOE_FMAC_DPP(1, 8, CTRL) TMOE_FMAC_DPP(2, 8, CTRL)      \
              TMOE_FMAC_DPP(3, 8, CTRL) TMOE_FMAC_DPP(4, 8, CTRL) TMOE_FMAC_DPP(5, 8, CTRL)              \
                  TMOE_FMAC_DPP(6, 8, CTRL) TMOE_FMAC_DPP(7, 8, CTRL)                                    \
          : "+v"(v[B]), "+v"(v[B + 1]), "+v"(v[B + 2]), "+v"(v[B + 3]), "+v"(v[B + 4]), "+v"(v[B + 5]), \
            "+v"(v[B + 6]), "+v"(v[B + 7])                                                               \
          : "v"(sg));                                                                                    \
    } else if constexpr (N == 4) {                                                                       \
      asm("s_nop 1\n" TMOE_FMAC_DPP(0, 4, CTRL) TMOE_FMAC_DPP(1, 4, CTRL) TMOE_FMAC_DPP(2, 4, CTRL)      \
              TMOE_FMAC_DPP(3, 4, CTRL)                                                                  \
          : "+v"(v[B]), "+v"(v[B + 1]), "+v"(v[B + 2]), "+v"(v[B + 3])                                   \
          : "v"(sg));                                                                                    \
    } else if constexpr (N == 2) {                                                                       \
      asm("s_nop 1\n" TMOE_FMAC_DPP(0, 2, CTRL) TMOE_FMAC_DPP(1, 2, CTRL) : "+v"(v[B]), "+v"(v[B + 1]) \
          : "v"(sg));                                                                                    \
    } else {                                                                                             \
      asm("s_nop 1\n" TMOE_FMAC_DPP(0, 1, CTRL) : "+v"(v[B]) : "v"(sg));                                \
    }                                                                                                    \
  } while (0)

template <int S, int B, int N, int EPL>
__device__ __forceinline__ void fmac_dpp(float (&v)[EPL], float sg) {
  if constexpr (S == 1) TMOE_DPP_STAGE("quad_perm:[1,0,3,2]");
  else if constexpr (S == 2) TMOE_DPP_STAGE("quad_perm:[2,3,0,1]");
  else TMOE_DPP_STAGE("row_ror:8");
}
#undef TMOE_DPP_STAGE
#undef TMOE_FMAC_DPP

template <int S, int EPL, int B = 0>
__device__ __forceinline__ void fmac_dpp_all(float (&v)[EPL], float sg) {
  if constexpr (B < EPL) {
    constexpr int N = EPL - B >= 8 ? 8 : EPL - B;
    fmac_dpp<S, B, N>(v, sg);
    fmac_dpp_all<S, EPL, B + N>(v, sg);
  }
}

template <int S, int EPL>
__device__ __forceinline__ void fwht_lane_stage(float (&v)[EPL], int lane) {
  const float sg = (lane & S) ? -1.0f : 1.0f;
  if constexpr (S == 1 || S == 2 || S == 8) {
    fmac_dpp_all<S>(v, sg);
  } else {
    float p[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) p[i] = lane_partner<S>(v[i]);
#pragma unroll
    for (int i = 0; i < EPL; ++i) v[i] = fmaf(p[i], sg, v[i]);
  }
}

template <int EPL>
__device__ __forceinline__ void fwht_segment(float (&v)[EPL], int lane) {
  fwht_lane_stage<1>(v, lane);
  fwht_lane_stage<2>(v, lane);
  fwht_lane_stage<4>(v, lane);
  fwht_lane_stage<8>(v, lane);
  fwht_lane_stage<16>(v, lane);
  fwht_lane_stage<32>(v, lane);
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
  const float fs = (__builtin_popcount(lane & 63) & 1) ? -kScale : kScale;
#pragma unroll
  for (int i = 0; i < EPL; ++i) v[i] *= fs;
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

// Maximum of |v| over the 32-lane half of the wavefront this lane belongs to: a butterfly over the
// lane bits 0-4 by DPP and swizzle exchanges (the rotation by 8 inside a 16-lane row pairs the two
// 8-lane groups as an exchange of bit 3 would); max is exact, so the order does not matter.
__device__ __forceinline__ float half_wave_amax(float v) {
  float a = fabsf(v);
  a = fmaxf(a, lane_partner<1>(a));
  a = fmaxf(a, lane_partner<2>(a));
  a = fmaxf(a, lane_partner<4>(a));
  a = fmaxf(a, lane_partner<8>(a));
  a = fmaxf(a, lane_partner<16>(a));
  return a;
}

}  // namespace tmoe
