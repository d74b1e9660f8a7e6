// k_rowops.hip -- per-row kernels around the two trellis GEMMs, one wavefront per row.
//
//  k_rotate : a = R_H(su1_e * x_t) for every route slot, stored as fp16 or MXFP8 (E4M3 values
//             with one E8M0 scale per 32). One fused launch for rotation and quantization, as in
//             "serve canonical Fruit QSRT atoms", Hot path.
//  k_act    : the activation epilogue between FC1 and FC2 in the pages' order
//             R_I -> svh -> silu(gate) * up -> suh_down -> R_I ("integrate EXL3 Trellis into the
//             fused W4A16 API", review of kernel.py), with the FC1 channel scales applied first.
//  k_out_rotate + k_topk_sum: y_t = sum over j ascending of w[t,j] * sv2_e * R_H(scale2_e * v), the
//             output rotation with exact top-k weighting. The rotation runs per route (one wavefront
//             each), the sum per token and column in a fixed j order with no atomics, so repeated
//             calls are bitwise identical.
#include "tmoe_device.hpp"
#include "tmoe_internal.hpp"

namespace tmoe {

namespace {

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

// MXFP8 of one value per lane; each 32-lane half of the wavefront is one 32-value block.
__device__ __forceinline__ void mx_store(float v, int lane, uint8_t* q_row, uint8_t* s_row, int idx) {
  const float amax = half_wave_amax(v);
  const int e = mx_exponent(amax);
  float sv = ldexpf(v, -e);
  sv = fminf(fmaxf(sv, -448.0f), 448.0f);     // saturating E4M3 (only a subnormal quotient can exceed)
  q_row[idx] = static_cast<uint8_t>(fp8x2_from_f32(sv, 0.0f) & 0xffu);
  if ((lane & 31) == 0) s_row[idx >> 5] = static_cast<uint8_t>(e + 127);
}

template <bool MX>
struct RotateBody {
  const RotateArgs& a;
  int lane, p, t, e, H;
  template <int S>
  __device__ __forceinline__ void run(int off) {
    float v[S];
    const uint16_t* xr = a.x + static_cast<size_t>(t) * H + off + lane;
    const uint16_t* sr = a.su1 + static_cast<size_t>(e) * H + off + lane;
#pragma unroll
    for (int i = 0; i < S; ++i) v[i] = bf16_to_f32(xr[64 * i]) * h2f(sr[64 * i]);
    if (!a.rot.identity) fwht_segment<S>(v, lane);
    if constexpr (!MX) {
      _Float16* out = static_cast<_Float16*>(a.a1) + static_cast<size_t>(p) * H + off + lane;
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

template <int EPL, bool MX>
__global__ __launch_bounds__(256) void k_rotate(RotateArgs a) {
  const int lane = threadIdx.x & 63;
  const int p = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (p >= a.routes || p >= a.offsets[a.num_experts]) return;   // whole wavefront leaves together
  const int r = a.sorted_routes[p];
  const int t = r / a.top_k;
  const int e = static_cast<int>(route_expert(a.ids, a.ids64, r));
  RotateBody<MX> body{a, lane, p, t, e, a.rot.n};
  for_segments<EPL>(a.rot, body);
}

template <bool MX>
struct ActBody {
  const ActArgs& a;
  int lane, p, e, I, splits;
  template <int S>
  __device__ __forceinline__ void run(int off) {
    float zg[S], zu[S];
    const size_t plane = static_cast<size_t>(a.routes) * 2 * I;
    const float* zr = a.z + static_cast<size_t>(p) * 2 * I + off + lane;
    const uint16_t* c1 = a.scale1 + static_cast<size_t>(e) * 2 * I + off + lane;
#pragma unroll
    for (int i = 0; i < S; ++i) {
      float sg = 0.0f, su = 0.0f;
      for (int s = 0; s < splits; ++s) {
        sg += zr[s * plane + 64 * i];
        su += zr[s * plane + I + 64 * i];
      }
      zg[i] = sg * h2f(c1[64 * i]);
      zu[i] = su * h2f(c1[I + 64 * i]);
    }
    if (!a.rot.identity) {
      fwht_segment<S>(zg, lane);
      fwht_segment<S>(zu, lane);
    }
    const uint16_t* s1 = a.sv1 + static_cast<size_t>(e) * 2 * I + off + lane;
    const uint16_t* s2 = a.su2 + static_cast<size_t>(e) * I + off + lane;
    float bb[S];
#pragma unroll
    for (int i = 0; i < S; ++i) {
      const float g = zg[i] * h2f(s1[64 * i]);
      const float u = zu[i] * h2f(s1[I + 64 * i]);
      const float h = g / (1.0f + expf(-g)) * u;
      bb[i] = h * h2f(s2[64 * i]);
    }
    if (!a.rot.identity) fwht_segment<S>(bb, lane);
    if constexpr (!MX) {
      _Float16* out = static_cast<_Float16*>(a.b) + static_cast<size_t>(p) * I + off + lane;
#pragma unroll
      for (int i = 0; i < S; ++i) out[64 * i] = static_cast<_Float16>(bb[i]);
    } else {
      uint8_t* q = static_cast<uint8_t*>(a.b) + static_cast<size_t>(p) * I;
      uint8_t* sc = a.b_scale + static_cast<size_t>(p) * (I / 32);
#pragma unroll
      for (int i = 0; i < S; ++i) mx_store(bb[i], lane, q, sc, off + 64 * i + lane);
    }
  }
};

template <int EPL, bool MX>
__global__ __launch_bounds__(256) void k_act(ActArgs a) {
  const int lane = threadIdx.x & 63;
  const int p = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (p >= a.routes || p >= a.offsets[a.num_experts]) return;
  const int r = a.sorted_routes[p];
  const int e = static_cast<int>(route_expert(a.ids, a.ids64, r));
  ActBody<MX> body{a, lane, p, e, a.rot.n, *a.splits};
  for_segments<EPL>(a.rot, body);
}

// Per route slot: o = w[r] * sv2_e * R_H(scale2_e * sum_s v_s), written over split plane 0 of the
// same slot (each slot is read completely before it is written, by the same wavefront).
struct OutRotBody {
  const CombineArgs& a;
  int lane, p, e, H, splits;
  float wt;
  template <int S>
  __device__ __forceinline__ void run(int off) {
    const size_t plane = static_cast<size_t>(a.routes) * H;
    float* vr = a.v + static_cast<size_t>(p) * H + off + lane;
    const uint16_t* c2 = a.scale2 + static_cast<size_t>(e) * H + off + lane;
    float vv[S];
#pragma unroll
    for (int i = 0; i < S; ++i) {
      float acc = 0.0f;
      for (int sp = 0; sp < splits; ++sp) acc += vr[sp * plane + 64 * i];
      vv[i] = acc * h2f(c2[64 * i]);
    }
    if (!a.rot.identity) fwht_segment<S>(vv, lane);
    const uint16_t* sg = a.sv2 + static_cast<size_t>(e) * H + off + lane;
#pragma unroll
    for (int i = 0; i < S; ++i) vr[64 * i] = wt * (vv[i] * h2f(sg[64 * i]));
  }
};

template <int EPL>
__global__ __launch_bounds__(256) void k_out_rotate(CombineArgs a) {
  const int lane = threadIdx.x & 63;
  const int p = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (p >= a.routes || p >= a.offsets[a.num_experts]) return;
  const int r = a.sorted_routes[p];
  const int e = static_cast<int>(route_expert(a.ids, a.ids64, r));
  OutRotBody body{a, lane, p, e, a.rot.n, *a.splits, a.w[r]};
  for_segments<EPL>(a.rot, body);
}

// y_t = sum over j ascending of o[slot(t, j)]; dropped routes add nothing. Four columns per thread.
__global__ __launch_bounds__(256) void k_topk_sum(CombineArgs a) {
  const int H4 = a.rot.n >> 2;
  const long long idx = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<long long>(a.tokens) * H4) return;
  const int t = static_cast<int>(idx / H4), c = static_cast<int>(idx % H4);
  const float4* o = reinterpret_cast<const float4*>(a.v);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < a.top_k; ++j) {
    const int p = a.route_slot[t * a.top_k + j];
    if (p >= 0) {
      const float4 x = o[static_cast<size_t>(p) * H4 + c];
      acc.x += x.x;
      acc.y += x.y;
      acc.z += x.z;
      acc.w += x.w;
    }
  }
  reinterpret_cast<float4*>(a.y)[static_cast<size_t>(t) * H4 + c] = acc;
}

struct DebugRotateBody {
  float* row;
  const RowRot& rot;
  int lane;
  template <int S>
  __device__ __forceinline__ void run(int off) {
    float v[S];
#pragma unroll
    for (int i = 0; i < S; ++i) v[i] = row[off + 64 * i + lane];
    if (!rot.identity) fwht_segment<S>(v, lane);
#pragma unroll
    for (int i = 0; i < S; ++i) row[off + 64 * i + lane] = v[i];
  }
};

template <int EPL>
__global__ __launch_bounds__(256) void k_debug_rotate(float* data, long long rows, RowRot rot) {
  const int lane = threadIdx.x & 63;
  const long long r = static_cast<long long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  DebugRotateBody body{data + r * rot.n, rot, lane};
  for_segments<EPL>(rot, body);
}

__global__ __launch_bounds__(256) void k_debug_mxfp8(const float* in, long long rows, int cols, uint8_t* q,
                                                     uint8_t* e8m0) {
  const int lane = threadIdx.x & 63;
  const long long r = static_cast<long long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const float* row = in + r * cols;
  uint8_t* qr = q + r * cols;
  uint8_t* sr = e8m0 + r * (cols / 32);
  for (int c = 0; c < cols; c += 64) {
    const int idx = c + lane;
    const bool ok = idx < cols;               // cols is a multiple of 32: whole halves are in or out
    const float v = ok ? row[idx] : 0.0f;
    const float amax = half_wave_amax(v);
    const int e = mx_exponent(amax);
    float sv = ldexpf(v, -e);
    sv = fminf(fmaxf(sv, -448.0f), 448.0f);
    if (ok) {
      qr[idx] = static_cast<uint8_t>(fp8x2_from_f32(sv, 0.0f) & 0xffu);
      if ((lane & 31) == 0) sr[idx >> 5] = static_cast<uint8_t>(e + 127);
    }
  }
}

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

inline unsigned blocks_for(long long rows) { return static_cast<unsigned>((rows + 3) / 4); }

}  // namespace

void launch_rotate(const RotateArgs& a, bool mx, hipStream_t s) {
  dispatch_epl(a.rot, [&](auto epl) {
    constexpr int E = decltype(epl)::value;
    if (mx) hipLaunchKernelGGL((k_rotate<E, true>), dim3(blocks_for(a.routes)), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_rotate<E, false>), dim3(blocks_for(a.routes)), dim3(256), 0, s, a);
  });
}

void launch_act(const ActArgs& a, bool mx, hipStream_t s) {
  dispatch_epl(a.rot, [&](auto epl) {
    constexpr int E = decltype(epl)::value;
    if (mx) hipLaunchKernelGGL((k_act<E, true>), dim3(blocks_for(a.routes)), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_act<E, false>), dim3(blocks_for(a.routes)), dim3(256), 0, s, a);
  });
}

void launch_combine(const CombineArgs& a, hipStream_t s) {
  dispatch_epl(a.rot, [&](auto epl) {
    constexpr int E = decltype(epl)::value;
    hipLaunchKernelGGL((k_out_rotate<E>), dim3(blocks_for(a.routes)), dim3(256), 0, s, a);
  });
  const long long n = static_cast<long long>(a.tokens) * (a.rot.n / 4);
  hipLaunchKernelGGL(k_topk_sum, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, a);
}

void launch_debug_rotate(float* data, long long rows, const RowRot& rot, hipStream_t s) {
  dispatch_epl(rot, [&](auto epl) {
    constexpr int E = decltype(epl)::value;
    hipLaunchKernelGGL((k_debug_rotate<E>), dim3(blocks_for(rows)), dim3(256), 0, s, data, rows, rot);
  });
}

void launch_debug_mxfp8(const float* in, long long rows, int cols, uint8_t* q, uint8_t* e8m0, hipStream_t s) {
  hipLaunchKernelGGL(k_debug_mxfp8, dim3(blocks_for(rows)), dim3(256), 0, s, in, rows, cols, q, e8m0);
}

}  // namespace tmoe
