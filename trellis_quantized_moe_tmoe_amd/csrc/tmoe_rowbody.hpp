// tmoe_rowbody.hpp -- row helpers shared by the route-map launch (input rotation) and the
// activation / combine kernels: rotation-block traversal, MXFP8 stores, the input rotation body.
#pragma once
#include "tmoe_device.hpp"
#include "tmoe_internal.hpp"

namespace tmoe {

__device__ __forceinline__ long long route_expert(const void* ids, int ids64, int r) {
  return ids64 ? static_cast<const long long*>(ids)[r] : static_cast<long long>(static_cast<const int*>(ids)[r]);
}

// Visit the rotation blocks of a row: one power-of-two segment of EPL values per lane, or (EPL = 0)
// 128-point blocks (2 per lane) followed by an optional 64-point block (1 per lane).
template <int EPL, class Body>
__device__ __forceinline__ void for_segments(const RowRot& rot, Body& body) {
  if constexpr (EPL > 0) {
    body.template run<EPL>(0);
  } else {
    for (int b = 0; b < rot.nblk128; ++b) body.template run<2>(b * 128);
    if (rot.tail64) body.template run<1>(rot.nblk128 * 128);
  }
}

// Segments of a row that rotate independently: the whole row for a power-of-two length, else its
// 128-value blocks and the 64-value tail. Row kernels give each segment a wavefront of its own, so a
// long non-power-of-two row is not walked block after block by one wavefront.
__host__ __device__ inline int row_segments(const RowRot& rot) { return rot.pow2 ? 1 : rot.nblk128 + rot.tail64; }

// Run body on segment seg of the row (EPL > 0: the whole row, EPL values per lane; EPL = 0: block
// seg, 2 values per lane, or the 64-value tail, 1 per lane).
template <int EPL, class Body>
__device__ __forceinline__ void run_segment(const RowRot& rot, int seg, Body& body) {
  if constexpr (EPL > 0) {
    body.template run<EPL>(0);
  } else {
    if (seg < rot.nblk128) body.template run<2>(seg * 128);
    else body.template run<1>(rot.nblk128 * 128);
  }
}

// MXFP8 of one value per lane; each 32-lane half of the wavefront is one 32-value block.
__device__ __forceinline__ void mx_store(float v, int lane, uint8_t* q_row, uint8_t* s_row, int idx) {
  const float amax = half_wave_amax(v);
  const int e = mx_exponent(amax);
  float sv = ldexpf(v, -e);
  sv = fminf(fmaxf(sv, -448.0f), 448.0f);     // saturating E4M3 (only a subnormal quotient can exceed)
  q_row[idx] = static_cast<uint8_t>(fp8x2_from_f32(sv, 0.0f) & 0xffu);
  if ((lane & 31) == 0) s_row[idx >> 5] = static_cast<uint8_t>(e + 127);
}

// Input rotation of one route (token t, expert e): a = R_H(su1_e * x_t) into operand row p.
// The butterflies of fwht_segment act on every bit of the element index, so the transform is the
// same whether a lane holds elements off + 64 i + lane (strided) or off + S lane + i (blocked); the
// fp16 path with 8 or more values per lane and the MXFP8 path with 8 or 16 use the blocked layout,
// whose loads and stores are 8 or 16 bytes wide (other MXFP8 rows keep the strided one, where a
// 32-value block is a half-wavefront).
template <bool MX>
struct RotateBody {
  const RotateArgs& a;
  int lane, p, t, e, H;     // p: operand row (the route index)
  template <int S>
  __device__ __forceinline__ void run(int off) {
    float v[S];
    // (the signs need only 2-byte alignment by contract; x and the arena are 16-byte aligned)
    if constexpr (MX && (S == 8 || S == 16)) {
      if ((reinterpret_cast<uintptr_t>(a.su1) & 15) == 0) {
        run_mx_blocked<S>(off);
        return;
      }
    }
    if constexpr (!MX && S >= 8) {
      if ((reinterpret_cast<uintptr_t>(a.su1) & 15) == 0) {
        typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
        typedef _Float16 h8 __attribute__((ext_vector_type(8)));
        const u16x8* xr = reinterpret_cast<const u16x8*>(a.x + static_cast<size_t>(t) * H + off + S * lane);
        const u16x8* sr = reinterpret_cast<const u16x8*>(a.su1 + static_cast<size_t>(e) * H + off + S * lane);
#pragma unroll
        for (int c = 0; c < S / 8; ++c) {
          const u16x8 xv = xr[c], sv = sr[c];
#pragma unroll
          for (int i = 0; i < 8; ++i) v[8 * c + i] = bf16_to_f32(xv[i]) * h2f(sv[i]);
        }
        if (!a.rot.identity) fwht_segment<S>(v, lane);
        h8* out = reinterpret_cast<h8*>(static_cast<_Float16*>(a.a1) + static_cast<size_t>(p) * a.lda + off + S * lane);
#pragma unroll
        for (int c = 0; c < S / 8; ++c) {
          h8 o;
#pragma unroll
          for (int i = 0; i < 8; ++i) o[i] = static_cast<_Float16>(v[8 * c + i]);
          out[c] = o;
        }
        return;
      }
    }
    const uint16_t* xr = a.x + static_cast<size_t>(t) * H + off + lane;
    const uint16_t* sr = a.su1 + static_cast<size_t>(e) * H + off + lane;
#pragma unroll
    for (int i = 0; i < S; ++i) v[i] = bf16_to_f32(xr[64 * i]) * h2f(sr[64 * i]);
    finish<S>(v, off);
  }
  // MXFP8 in the blocked layout (element off + S lane + i in v[i]): a 32-value block is 32 / S
  // adjacent lanes, so its maximum is the lane's own S values and one (S = 16) or two (S = 8) lane
  // exchanges, and the lane writes its S codes with one 16- or 8-byte store.
  template <int S>
  __device__ __forceinline__ void run_mx_blocked(int off) {
    typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
    float v[S];
    const u16x8* xr = reinterpret_cast<const u16x8*>(a.x + static_cast<size_t>(t) * H + off + S * lane);
    const u16x8* sr = reinterpret_cast<const u16x8*>(a.su1 + static_cast<size_t>(e) * H + off + S * lane);
#pragma unroll
    for (int c = 0; c < S / 8; ++c) {
      const u16x8 xv = xr[c], sv = sr[c];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[8 * c + i] = bf16_to_f32(xv[i]) * h2f(sv[i]);
    }
    if (!a.rot.identity) fwht_segment<S>(v, lane);
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < S; ++i) m = fmaxf(m, fabsf(v[i]));
    m = fmaxf(m, lane_partner<1>(m));
    if constexpr (S == 8) m = fmaxf(m, lane_partner<2>(m));
    const int ex = mx_exponent(m);
    uint32_t w[S / 4];
#pragma unroll
    for (int k = 0; k < S / 4; ++k) {
      float q4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) q4[j] = fminf(fmaxf(ldexpf(v[4 * k + j], -ex), -448.0f), 448.0f);
      w[k] = fp8x2_from_f32(q4[0], q4[1]) | (fp8x2_from_f32(q4[2], q4[3]) << 16);
    }
    uint8_t* q = static_cast<uint8_t*>(a.a1) + static_cast<size_t>(p) * H + off + S * lane;
    if constexpr (S == 16) *reinterpret_cast<uint4*>(q) = make_uint4(w[0], w[1], w[2], w[3]);
    else *reinterpret_cast<uint2*>(q) = make_uint2(w[0], w[1]);
    if ((lane & (32 / S - 1)) == 0)
      a.a1_scale[static_cast<size_t>(p) * (H / 32) + ((off + S * lane) >> 5)] = static_cast<uint8_t>(ex + 127);
  }
  // NB consecutive 128-blocks from element off: every block's loads are issued before the first
  // block is rotated (a long non-power-of-two row would otherwise wait on each block in turn).
  template <int NB>
  __device__ __forceinline__ void run_blocks128(int off) {
    const uint16_t* xr = a.x + static_cast<size_t>(t) * H + off + lane;
    const uint16_t* sr = a.su1 + static_cast<size_t>(e) * H + off + lane;
    uint16_t xv[NB][2], sv[NB][2];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        xv[nb][i] = xr[128 * nb + 64 * i];
        sv[nb][i] = sr[128 * nb + 64 * i];
      }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float v[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) v[i] = bf16_to_f32(xv[nb][i]) * h2f(sv[nb][i]);
      finish<2>(v, off + 128 * nb);
    }
  }
  // Rotation and store of one segment held strided (element off + 64 i + lane in v[i]).
  template <int S>
  __device__ __forceinline__ void finish(float (&v)[S], int off) {
    if (!a.rot.identity) fwht_segment<S>(v, lane);
    if constexpr (!MX) {
      _Float16* out = static_cast<_Float16*>(a.a1) + static_cast<size_t>(p) * a.lda + off + lane;
#pragma unroll
      for (int i = 0; i < S; ++i) out[64 * i] = static_cast<_Float16>(v[i]);
    } else {
      uint8_t* q = static_cast<uint8_t*>(a.a1) + static_cast<size_t>(p) * H;
      uint8_t* sc = a.a1_scale + static_cast<size_t>(p) * (H / 32);
#pragma unroll
      for (int i = 0; i < S; ++i) mx_store(v[i], lane, q, sc, off + 64 * i + lane);
    }
  }
};

// Host: call f with the rotation's values per lane as a compile-time constant (0 = 128/64 blocks).
template <class F>
void dispatch_epl(const RowRot& rot, F&& f) {
  if (!rot.pow2) { f(std::integral_constant<int, 0>{}); return; }
  switch (rot.n / 64) {
    case 1: f(std::integral_constant<int, 1>{}); break;
    case 2: f(std::integral_constant<int, 2>{}); break;
    case 4: f(std::integral_constant<int, 4>{}); break;
    case 8: f(std::integral_constant<int, 8>{}); break;
    case 16: f(std::integral_constant<int, 16>{}); break;
    case 32: f(std::integral_constant<int, 32>{}); break;
    default: f(std::integral_constant<int, 64>{}); break;
  }
}

// Items of the input rotation: routes, or (route, row segment) pairs when the host splits rows (few
// routes with long non-power-of-two rows).
__host__ __device__ inline int rotate_items_per_route(const RotateArgs& a) {
  return a.split_segments ? row_segments(a.rot) : 1;
}

// One rotation item of operand row p (token t's x with expert e's signs): segment seg of the row
// when rows are split into `per` items, else the whole row.
template <int EPL, bool MX>
__device__ __forceinline__ void rotate_item(const RotateArgs& a, int p, int t, int e, int seg, int per) {
  const int lane = threadIdx.x & 63;
  RotateBody<MX> body{a, lane, p, t, e, a.rot.n};
  if (per > 1) {
    run_segment<EPL>(a.rot, seg, body);
  } else if constexpr (EPL > 0) {
    body.template run<EPL>(0);
  } else {                          // the whole row: its 128-blocks four at a time, then the tail
    int b = 0;
    for (; b + 4 <= a.rot.nblk128; b += 4) body.template run_blocks128<4>(b * 128);
    for (; b < a.rot.nblk128; ++b) body.template run_blocks128<1>(b * 128);
    if (a.rot.tail64) body.template run<1>(a.rot.nblk128 * 128);
  }
}

// Workgroup-level input rotation, one item per wavefront: item first + wave. Used by the route-map
// launch for its extra workgroups (the rotation does not depend on the route map).
template <int EPL, bool MX>
__device__ __forceinline__ void rotate_routes(const RotateArgs& a, int first) {
  const int per = EPL > 0 ? 1 : rotate_items_per_route(a);
  const int item = first + static_cast<int>(threadIdx.x >> 6);
  const int r = item / per, seg = item - r * per;
  if (r >= a.routes) return;
  const long long e = route_expert(a.ids, a.ids64, r);
  if (e < 0 || e >= a.num_experts) return;         // dropped route: its row is never read
  rotate_item<EPL, MX>(a, r, r / a.top_k, static_cast<int>(e), seg, per);
}

}  // namespace tmoe
