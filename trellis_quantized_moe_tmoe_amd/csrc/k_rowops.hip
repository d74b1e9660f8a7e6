// k_rowops.hip -- per-row kernels around the two trellis GEMMs.
//
//  (the input rotation runs in the route-map launch, k_route_map.hip)
//  k_act    : the activation epilogue between FC1 and FC2 in the pages' order
//             R_I -> svh -> silu(gate) * up -> suh_down -> R_I ("integrate EXL3 Trellis into the
//             fused W4A16 API", review of kernel.py), with the FC1 channel scales applied first;
//             one wavefront per slot, or per (slot, 128-block) for rows rotated in blocks.
//  k_combine: y_t = sum over j ascending of w[t,j] * sv2_e * R_H(scale2_e * v), the output rotation
//             with exact top-k weighting. One workgroup per token (or per (token, 128-block)): each
//             wavefront rotates one of the token's routes into LDS, then every column is summed in
//             ascending j with no atomics, so repeated calls are bitwise identical.
//
// The FC1/FC2 GEMMs leave up to 8 K-split partial planes; every reader sums them in ascending split
// order, with all loads of a row issued before the first add so one memory latency covers them.
// With one K split the 128-row-tile GEMMs instead leave one fp16 plane with the channel scale
// already applied; the readers take it as template split count SMAX = 0.
#include "tmoe_device.hpp"
#include "tmoe_internal.hpp"
#include "tmoe_hadamard.hpp"
#include "tmoe_rowbody.hpp"

namespace tmoe {

namespace {

// out[i] = sum over s < splits, ascending, of src[s * plane + 64 * i] for i < S, with splits <= SMAX
// (the kernels here pass splits = SMAX, the host's split count). Planes are loaded SU at a time;
// when SU = SMAX the single round re-reads the last plane for s >= splits (in bounds, cached) and
// adds it as nothing, so every load goes out before the first add with no branch between them.
template <int S, int SMAX, int SU>
__device__ __forceinline__ void sum_splits(const float* __restrict__ src, size_t plane, int splits, float (&out)[S]) {
#pragma unroll
  for (int i = 0; i < S; ++i) out[i] = 0.0f;
  auto round = [&](int s0) {
    float t[SU][S];
#pragma unroll
    for (int u = 0; u < SU; ++u) {
      const int sp = s0 + u < splits ? s0 + u : splits - 1;
#pragma unroll
      for (int i = 0; i < S; ++i) t[u][i] = src[sp * plane + 64 * i];
    }
#pragma unroll
    for (int u = 0; u < SU; ++u)
#pragma unroll
      for (int i = 0; i < S; ++i) out[i] += s0 + u < splits ? t[u][i] : 0.0f;
  };
  if constexpr (SU == SMAX) {
    round(0);
  } else {
#pragma unroll 1
    for (int s0 = 0; s0 < splits; s0 += SU) round(s0);
  }
}

template <int S, int SMAX>
constexpr int splits_unroll(int rows) {   // planes loaded per round: about 64 loads in flight per lane
  return SMAX * S * rows <= 64 ? SMAX : (64 / (S * rows) >= 1 ? 64 / (S * rows) : 1);
}

// Values of a lane: elements off + 64 i + lane (strided), or for fp16 rows with 8 or more values per
// lane whose scale and sign vectors are 16-byte aligned, off + S lane + i (blocked: 16-byte loads and
// stores; the butterflies cover every index bit either way).
template <int S>
__device__ __forceinline__ void load_f16_blocked(const uint16_t* src, float (&out)[S]) {
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
#pragma unroll
  for (int c = 0; c < S / 8; ++c) {
    const h8 v = reinterpret_cast<const h8*>(src)[c];
#pragma unroll
    for (int i = 0; i < 8; ++i) out[8 * c + i] = static_cast<float>(v[i]);
  }
}

// sum_splits for the blocked layout of the activation: out[i] = sum over s < SMAX, ascending, of
// src[s * plane + i] (src already at the lane's S values, 16-byte aligned).
template <int S, int SMAX, int SU>
__device__ __forceinline__ void sum_splits_blocked(const float* __restrict__ src, size_t plane, float (&out)[S]) {
  static_assert(SMAX % SU == 0, "split rounds");
#pragma unroll
  for (int i = 0; i < S; ++i) out[i] = 0.0f;
#pragma unroll 1
  for (int s0 = 0; s0 < SMAX; s0 += SU) {
    float4 t[SU][S / 4];
#pragma unroll
    for (int u = 0; u < SU; ++u)
#pragma unroll
      for (int c = 0; c < S / 4; ++c) t[u][c] = reinterpret_cast<const float4*>(src + (s0 + u) * plane)[c];
#pragma unroll
    for (int u = 0; u < SU; ++u)
#pragma unroll
      for (int c = 0; c < S / 4; ++c) {
        out[4 * c] += t[u][c].x;
        out[4 * c + 1] += t[u][c].y;
        out[4 * c + 2] += t[u][c].z;
        out[4 * c + 3] += t[u][c].w;
      }
  }
}

// out[i] = scale[64 i] * (sum of the split planes at src[64 i]), or with SMAX = 0 the fp16 plane's
// value h[64 i], which holds that product already (src, h and scale at the lane's first value).
template <int S, int SMAX, int SU>
__device__ __forceinline__ void scaled_values(const float* __restrict__ src, const uint16_t* __restrict__ h,
                                              size_t plane, int splits, const uint16_t* scale, float (&out)[S]) {
  if constexpr (SMAX == 0) {
#pragma unroll
    for (int i = 0; i < S; ++i) out[i] = h2f(h[64 * i]);
  } else {
    sum_splits<S, SMAX, SU>(src, plane, splits, out);
#pragma unroll
    for (int i = 0; i < S; ++i) out[i] *= h2f(scale[64 * i]);
  }
}

__device__ __forceinline__ bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

template <bool MX, int SMAX>
struct ActBody {
  const ActArgs& a;
  int lane, p, e, I, splits;
  template <int S>
  __device__ __forceinline__ void run(int off) {
    if constexpr (!MX && S >= 8) {
      if (aligned16(a.scale1) && aligned16(a.sv1) && aligned16(a.su2)) {
        run_blocked<S>(off);
        return;
      }
    }
    float zg[S], zu[S];
    const size_t plane = static_cast<size_t>(a.routes) * 2 * I;
    const size_t zo = static_cast<size_t>(p) * 2 * I + off + lane;
    const uint16_t* c1 = a.scale1 + static_cast<size_t>(e) * 2 * I + off + lane;
    constexpr int SU = SMAX > 0 ? splits_unroll<S, SMAX>(2) : 1;
    scaled_values<S, SMAX, SU>(a.z + zo, a.z16 + zo, plane, splits, c1, zg);
    scaled_values<S, SMAX, SU>(a.z + zo + I, a.z16 + zo + I, plane, splits, c1 + I, zu);
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
      const float h = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;   // SiLU(g) * u
      bb[i] = h * h2f(s2[64 * i]);
    }
    if (!a.rot.identity) fwht_segment<S>(bb, lane);
    if constexpr (!MX) {
      _Float16* out = static_cast<_Float16*>(a.b) + static_cast<size_t>(p) * a.ldb + off + lane;
#pragma unroll
      for (int i = 0; i < S; ++i) out[64 * i] = static_cast<_Float16>(bb[i]);
    } else {
      uint8_t* q = static_cast<uint8_t*>(a.b) + static_cast<size_t>(p) * I;
      uint8_t* sc = a.b_scale + static_cast<size_t>(p) * (I / 32);
#pragma unroll
      for (int i = 0; i < S; ++i) mx_store(bb[i], lane, q, sc, off + 64 * i + lane);
    }
  }
  template <int S>
  __device__ __forceinline__ void run_blocked(int off) {
    const size_t plane = static_cast<size_t>(a.routes) * 2 * I;
    const size_t zo = static_cast<size_t>(p) * 2 * I + off + S * lane;
    const size_t erow = static_cast<size_t>(e) * 2 * I + off + S * lane;
    float zg[S], zu[S], sg[S], su[S], s2[S];
    if constexpr (SMAX == 0) {                 // one fp16 plane, scale1 applied
      load_f16_blocked<S>(a.z16 + zo, zg);
      load_f16_blocked<S>(a.z16 + zo + I, zu);
    } else {
      sum_splits_blocked<S, SMAX, splits_unroll<S, SMAX>(2)>(a.z + zo, plane, zg);
      sum_splits_blocked<S, SMAX, splits_unroll<S, SMAX>(2)>(a.z + zo + I, plane, zu);
    }
    load_f16_blocked<S>(a.sv1 + erow, sg);
    load_f16_blocked<S>(a.sv1 + erow + I, su);
    load_f16_blocked<S>(a.su2 + static_cast<size_t>(e) * I + off + S * lane, s2);
    if constexpr (SMAX > 0) {
      float cg[S], cu[S];
      load_f16_blocked<S>(a.scale1 + erow, cg);
      load_f16_blocked<S>(a.scale1 + erow + I, cu);
#pragma unroll
      for (int i = 0; i < S; ++i) {
        zg[i] *= cg[i];
        zu[i] *= cu[i];
      }
    }
    if (!a.rot.identity) {
      fwht_segment<S>(zg, lane);
      fwht_segment<S>(zu, lane);
    }
    float bb[S];
#pragma unroll
    for (int i = 0; i < S; ++i) {
      const float g = zg[i] * sg[i];
      const float u = zu[i] * su[i];
      const float h = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;   // SiLU(g) * u
      bb[i] = h * s2[i];
    }
    if (!a.rot.identity) fwht_segment<S>(bb, lane);
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    h8* out = reinterpret_cast<h8*>(static_cast<_Float16*>(a.b) + static_cast<size_t>(p) * a.ldb + off + S * lane);
#pragma unroll
    for (int c = 0; c < S / 8; ++c) {
      h8 o;
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = static_cast<_Float16>(bb[8 * c + i]);
      out[c] = o;
    }
  }
};


// The activation of kActSlots consecutive slots from p0 with I = 512 and one fp16 FC1 plane (scale1
// applied), their three rotations on the matrix cores: g and u are forward transforms of the plane's
// halves, the product is transformed from the C2 layout and stored from the second transform's
// layout. Slots are grouped by expert, so the sign rows are read again only where the expert
// changes, and the next slot's FC1 row is requested before the current one is transformed. Filled
// slots are contiguous: the first slot of expert -1 ends the wavefront's work.
constexpr int kActSlots = 4;
__device__ __forceinline__ void act_rows_mfma(const ActArgs& a, int p0, int lane) {
  constexpr int I = 512;
  constexpr float kScale = 0.04419417382415922f;   // 1/sqrt(512), rounded once to fp32
  const int c = lane & 15, q = lane >> 4;
  auto row = [&](int p) {
    return reinterpret_cast<const _Float16*>(a.z16) + static_cast<size_t>(p) * 2 * I + 32 * c + 8 * q;
  };
  int p = p0;
  int e = a.slot_expert[p];                       // (p0 < routes)
  if (e < 0) return;
  half8 xg = *reinterpret_cast<const half8*>(row(p));
  half8 xu = *reinterpret_cast<const half8*>(row(p) + I);
  const hmfma::Operands o = hmfma::load_operands(lane);
  float sg[2][4], su[2][4], sd[2][4];
  int e_signs = -1;
  for (int k = 0; k < kActSlots; ++k) {
    const int pn = p + 1;
    const bool more = k + 1 < kActSlots && pn < a.routes;
    const int en = more ? a.slot_expert[pn] : -1;
    const _Float16* rn = row(more ? pn : p);       // (a repeat of the current row when there is none)
    const half8 ng = *reinterpret_cast<const half8*>(rn);
    const half8 nu = *reinterpret_cast<const half8*>(rn + I);
    f4 g[2], u[2], v[2];
    hmfma::forward(o, xg, g);
    hmfma::forward(o, xu, u);
    if (e != e_signs) {
      // signs at the C2 positions 32(4q+i) + 16h + c
      const uint16_t* s1 = a.sv1 + static_cast<size_t>(e) * 2 * I + 128 * q + c;
      const uint16_t* s2 = a.su2 + static_cast<size_t>(e) * I + 128 * q + c;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sg[h][i] = h2f(s1[32 * i + 16 * h]);
          su[h][i] = h2f(s1[I + 32 * i + 16 * h]);
          sd[h][i] = h2f(s2[32 * i + 16 * h]);
        }
      e_signs = e;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float gg = (g[h][i] * kScale) * sg[h][i];
        const float uu = (u[h][i] * kScale) * su[h][i];
        v[h][i] = gg * __builtin_amdgcn_rcpf(1.0f + __expf(-gg)) * uu * sd[h][i];   // SiLU(g) * u * su2
      }
    f4 y[2];
    hmfma::from_c2(o, v, y);
    _Float16* out = static_cast<_Float16*>(a.b) + static_cast<size_t>(p) * a.ldb + 32 * c + 4 * q;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const hmfma::half4v r = {static_cast<_Float16>(y[h][0] * kScale), static_cast<_Float16>(y[h][1] * kScale),
                               static_cast<_Float16>(y[h][2] * kScale), static_cast<_Float16>(y[h][3] * kScale)};
      *reinterpret_cast<hmfma::half4v*>(out + 16 * h) = r;
    }
    if (en < 0) break;
    p = pn;
    e = en;
    xg = ng;
    xu = nu;
  }
}

// One wavefront per (slot, row segment): every step of the epilogue (rotations, SiLU, scales) stays
// inside one segment of the intermediate row.
template <int EPL, bool MX, int SMAX>
__global__ __launch_bounds__(256) void k_act(ActArgs a) {
  if (static_cast<int>(blockIdx.x) >= a.act_blocks) {      // zero y for the atomic FC2 reduction
    const long long i0 = (static_cast<long long>(blockIdx.x) - a.act_blocks) * 256 * 4 + 4 * threadIdx.x;
    if (i0 + 3 < a.y_count) {
      *reinterpret_cast<float4*>(a.y_zero + i0) = make_float4(0.f, 0.f, 0.f, 0.f);
    } else {
      for (long long i = i0; i < a.y_count; ++i) a.y_zero[i] = 0.0f;
    }
    return;
  }
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if constexpr (EPL == 8 && !MX && SMAX == 0) {
    if (!a.rot.identity) {                       // kActSlots slots per wavefront (launch_act)
      if (item * kActSlots < a.routes) act_rows_mfma(a, item * kActSlots, lane);
      return;
    }
  }
  const int nseg = EPL > 0 ? 1 : row_segments(a.rot);
  const int p = item / nseg, seg = item - p * nseg;
  if (p >= a.routes) return;
  const int e = a.slot_expert[p];                // -1 past the filled slots (dropped routes)
  if (e < 0) return;
  ActBody<MX, SMAX> body{a, lane, p, e, a.rot.n, SMAX};
  run_segment<EPL>(a.rot, seg, body);
}

// Few slots with I = 512 and fp32 K-split planes: one workgroup of four wavefronts per slot, so the
// chain of dependent instructions each wavefront runs is about a quarter of a whole-row wavefront's
// (at small batches that chain, not the chip's throughput, sets the kernel's time). Wavefront w holds
// elements 128 w + lane and 128 w + 64 + lane; with i = 128 w + j the rotation is H_4 (x) H_128: the
// 128-point transform inside each wavefront (its butterflies, scale 1/sqrt(128)), then H_4 across
// the four wavefronts through LDS, in ascending order of the source wavefront, times 1/2. MX: the
// product goes out as MXFP8; each 32-lane half of a wavefront holds 32 consecutive elements, one
// E8M0 block.
template <bool MX, int SMAX>
__global__ __launch_bounds__(256) void k_act_split(ActArgs a) {
  constexpr int I = 512;
  __shared__ float xs[3][4][128];               // gate, up, then the product, per wavefront
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int p = blockIdx.x;                     // the grid is one workgroup per slot
  const int e = a.slot_expert[p];               // -1 past the filled slots: the whole workgroup leaves
  if (e < 0) return;
  const bool rot = !a.rot.identity;
  const int i0 = 128 * w + lane, i1 = i0 + 64;
  const size_t plane = static_cast<size_t>(a.routes) * 2 * I;
  const float* zr = a.z + static_cast<size_t>(p) * 2 * I;
  float t[SMAX][4];
#pragma unroll
  for (int sp = 0; sp < SMAX; ++sp) {
    t[sp][0] = zr[sp * plane + i0];
    t[sp][1] = zr[sp * plane + i1];
    t[sp][2] = zr[sp * plane + I + i0];
    t[sp][3] = zr[sp * plane + I + i1];
  }
  const uint16_t* c1 = a.scale1 + static_cast<size_t>(e) * 2 * I;
  const uint16_t* s1 = a.sv1 + static_cast<size_t>(e) * 2 * I;
  const uint16_t* s2 = a.su2 + static_cast<size_t>(e) * I;
  const float cg0 = h2f(c1[i0]), cg1 = h2f(c1[i1]), cu0 = h2f(c1[I + i0]), cu1 = h2f(c1[I + i1]);
  const float sg0 = h2f(s1[i0]), sg1 = h2f(s1[i1]), su0 = h2f(s1[I + i0]), su1 = h2f(s1[I + i1]);
  const float sd0 = h2f(s2[i0]), sd1 = h2f(s2[i1]);
  float g[2] = {0.f, 0.f}, u[2] = {0.f, 0.f};
#pragma unroll
  for (int sp = 0; sp < SMAX; ++sp) {           // split planes in ascending order
    g[0] += t[sp][0];
    g[1] += t[sp][1];
    u[0] += t[sp][2];
    u[1] += t[sp][3];
  }
  g[0] *= cg0;
  g[1] *= cg1;
  u[0] *= cu0;
  u[1] *= cu1;
  // H_4 across the wavefronts: value j of wavefront w becomes (1/2) sum over v of (-1)^popcount(w & v)
  // times value j of wavefront v
  auto across = [&](int k, float (&v)[2]) {
    xs[k][w][lane] = v[0];
    xs[k][w][64 + lane] = v[1];
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float acc = xs[k][0][64 * h + lane];
#pragma unroll
      for (int src = 1; src < 4; ++src) {
        const float x = xs[k][src][64 * h + lane];
        acc = (__builtin_popcount(w & src) & 1) ? acc - x : acc + x;
      }
      v[h] = 0.5f * acc;
    }
  };
  if (rot) {
    fwht_segment<2>(g, lane);
    fwht_segment<2>(u, lane);
    // gate and up cross in one exchange (one barrier)
    xs[0][w][lane] = g[0];
    xs[0][w][64 + lane] = g[1];
    xs[1][w][lane] = u[0];
    xs[1][w][64 + lane] = u[1];
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float ag = xs[0][0][64 * h + lane], au = xs[1][0][64 * h + lane];
#pragma unroll
      for (int src = 1; src < 4; ++src) {
        const float xg = xs[0][src][64 * h + lane], xu = xs[1][src][64 * h + lane];
        const bool neg = __builtin_popcount(w & src) & 1;
        ag = neg ? ag - xg : ag + xg;
        au = neg ? au - xu : au + xu;
      }
      g[h] = 0.5f * ag;
      u[h] = 0.5f * au;
    }
  }
  float b[2];
  {
    const float gg0 = g[0] * sg0, uu0 = u[0] * su0, gg1 = g[1] * sg1, uu1 = u[1] * su1;
    b[0] = gg0 * __builtin_amdgcn_rcpf(1.0f + __expf(-gg0)) * uu0 * sd0;   // SiLU(g) * u * su2
    b[1] = gg1 * __builtin_amdgcn_rcpf(1.0f + __expf(-gg1)) * uu1 * sd1;
  }
  if (rot) {
    fwht_segment<2>(b, lane);
    across(2, b);
  }
  if constexpr (MX) {
    uint8_t* q = static_cast<uint8_t*>(a.b) + static_cast<size_t>(p) * I;
    uint8_t* sc = a.b_scale + static_cast<size_t>(p) * (I / 32);
    mx_store(b[0], lane, q, sc, i0);
    mx_store(b[1], lane, q, sc, i1);
  } else {
    _Float16* out = static_cast<_Float16*>(a.b) + static_cast<size_t>(p) * a.ldb;
    out[i0] = static_cast<_Float16>(b[0]);
    out[i1] = static_cast<_Float16>(b[1]);
  }
}

// Rotates one route's row held in LDS in place: o = wt * sv2_e * R_H(row).
struct CombineRotBody {
  const CombineArgs& a;
  float* row;
  int lane, e;
  float wt;
  template <int S>
  __device__ __forceinline__ void run(int off) {
    float vv[S];
#pragma unroll
    for (int i = 0; i < S; ++i) vv[i] = row[off + 64 * i + lane];
    if (!a.rot.identity) fwht_segment<S>(vv, lane);
    const uint16_t* sg = a.sv2 + static_cast<size_t>(e) * a.rot.n + off + lane;
#pragma unroll
    for (int i = 0; i < S; ++i) row[off + 64 * i + lane] = wt * (vv[i] * h2f(sg[64 * i]));
  }
};

// One workgroup of W wavefronts per token t (power-of-two rows, EPL > 0), or per (token, row segment)
// for few tokens with a long non-power-of-two row (EPL = 0): one 128-value block or the 64-value
// tail, as the rotation never crosses a segment (many tokens with such rows use k_combine_blocks).
// Round it handles routes j = it * W + w (wavefront w): the split sum of v times scale2, rotated,
// times sv2 and the route's weight, goes to the wavefront's LDS row (in registers up to 16 values
// per lane; longer rows are staged in LDS and rotated there); after a barrier every thread adds its
// columns of the W rows in ascending j onto a running sum kept in LDS (the last round writes y
// instead). Dropped routes add nothing. LDS: (W + 1) * L floats plus W flags, L the segment length.
template <int EPL, int SMAX>
__global__ __launch_bounds__(EPL >= 64 ? 256 : 1024) void k_combine(CombineArgs a) {
  extern __shared__ float lds[];
  const int H = a.rot.n, K = a.top_k;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, W = blockDim.x >> 6;
  const int t = blockIdx.x, seg = blockIdx.y;
  constexpr bool split = EPL == 0;
  const int off = split ? seg * 128 : 0;
  const int L = !split ? H : (seg < a.rot.nblk128 ? 128 : 64);
  float* acc = lds;                         // [L]
  float* rows = lds + L;                    // [W][L]
  int* live = reinterpret_cast<int*>(rows + static_cast<size_t>(W) * L);   // [W]
  float* row = rows + static_cast<size_t>(wv) * L;
  const int splits = SMAX;
  const size_t plane = static_cast<size_t>(a.routes) * H;
  const int rounds = (K + W - 1) / W;
  for (int it = 0; it < rounds; ++it) {
    const int j = it * W + wv;
    const int r = t * K + j;
    // the route's expert and weight do not depend on its slot, so their loads go out with the slot's
    const bool jk = j < K;
    const int p = jk ? a.route_slot[r] : -1;
    const int e_r = jk ? static_cast<int>(route_expert(a.ids, a.ids64, r)) : 0;
    const float w_r = jk ? a.w[r] : 0.0f;
    if (lane == 0) live[wv] = p >= 0;
    if (p >= 0) {
      const int e = e_r;
      // S values per lane in registers: split sum, scale, rotation, sign and weight, one LDS write
      auto in_registers = [&](auto s_const) {
        constexpr int S = decltype(s_const)::value;
        const float wt = w_r;
        float vv[S];
        const size_t vo = static_cast<size_t>(p) * H + off + lane;
        const uint16_t* c2 = a.scale2 + static_cast<size_t>(e) * H + off + lane;
        const uint16_t* sg = a.sv2 + static_cast<size_t>(e) * H + off + lane;
        scaled_values<S, SMAX, (SMAX > 0 ? splits_unroll<S, SMAX>(1) : 1)>(a.v + vo, a.v16 + vo, plane, splits, c2, vv);
        if (!a.rot.identity) fwht_segment<S>(vv, lane);
#pragma unroll
        for (int i = 0; i < S; ++i) row[64 * i + lane] = wt * (vv[i] * h2f(sg[64 * i]));
      };
      if constexpr (split) {
        if (L == 128) in_registers(std::integral_constant<int, 2>{});
        else in_registers(std::integral_constant<int, 1>{});
      } else if constexpr (EPL == 16 && SMAX == 0) {
        if (a.rot.identity) {
          in_registers(std::integral_constant<int, EPL>{});
        } else {
          // one fp16 plane (scale2 applied): R_H on the matrix cores, then sign and weight (1/32
          // folded into the weight exactly) into the route's LDS row at the natural positions
          const int c = lane & 15, q = lane >> 4;
          const _Float16* vr = reinterpret_cast<const _Float16*>(a.v16) + static_cast<size_t>(p) * H + 32 * c + 8 * q;
          const half8 x[2] = {*reinterpret_cast<const half8*>(vr), *reinterpret_cast<const half8*>(vr + 512)};
          const hmfma::Operands o = hmfma::load_operands(lane);
          f4 y[2][2];
          hmfma::forward1024(o, x, y);
          // the signs are read after the products (held beside the operands they would cost the
          // kernel a wavefront per SIMD)
          __builtin_amdgcn_sched_barrier(0);
          const uint16_t* sg = a.sv2 + static_cast<size_t>(e_r) * H + 128 * q + c;
          float sv[2][2][4];
#pragma unroll
          for (int ha = 0; ha < 2; ++ha)
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
#pragma unroll
              for (int i = 0; i < 4; ++i) sv[ha][hb][i] = h2f(sg[512 * ha + 32 * i + 16 * hb]);
          const float wt = w_r * 0.03125f;
          float* rr = row + 128 * q + c;
#pragma unroll
          for (int ha = 0; ha < 2; ++ha)
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
#pragma unroll
              for (int i = 0; i < 4; ++i) rr[512 * ha + 32 * i + 16 * hb] = wt * (y[ha][hb][i] * sv[ha][hb][i]);
        }
      } else if constexpr (EPL <= 16) {
        in_registers(std::integral_constant<int, EPL>{});
      } else {
        const size_t vo = static_cast<size_t>(p) * H + lane;
        const uint16_t* c2 = a.scale2 + static_cast<size_t>(e) * H + lane;
        constexpr int U = 8;
        // (here EPL >= 32: the row is one block of 64 * EPL values, a multiple of 512); unrolled,
        // so every chunk's loads can be in flight before the first LDS write
#pragma unroll
        for (int base = 0; base < 64 * EPL; base += 64 * U) {
          float sum[U];
          scaled_values<U, SMAX, (SMAX > 0 ? splits_unroll<U, SMAX>(1) : 1)>(a.v + vo + base, a.v16 + vo + base, plane,
                                                                          splits, c2 + base, sum);
#pragma unroll
          for (int i = 0; i < U; ++i) row[base + 64 * i + lane] = sum[i];
        }
        CombineRotBody body{a, row, lane, e, w_r};
        for_segments<EPL>(a.rot, body);
      }
    }
    __syncthreads();
    const int L4 = L >> 2;
    const bool last = it + 1 == rounds;
    const int nw = K - it * W < W ? K - it * W : W;
    for (int c = threadIdx.x; c < L4; c += blockDim.x) {
      float4 s4 = it == 0 ? make_float4(0.f, 0.f, 0.f, 0.f) : reinterpret_cast<const float4*>(acc)[c];
      for (int w = 0; w < nw; ++w) {
        if (!live[w]) continue;
        const float4 x = reinterpret_cast<const float4*>(rows + static_cast<size_t>(w) * L)[c];
        s4.x += x.x;
        s4.y += x.y;
        s4.z += x.z;
        s4.w += x.w;
      }
      if (last) reinterpret_cast<float4*>(a.y + static_cast<size_t>(t) * H + off)[c] = s4;
      else reinterpret_cast<float4*>(acc)[c] = s4;
    }
    __syncthreads();
  }
}

// Large batches with rows of a non-power-of-two length: one wavefront per (token t, rotation block),
// which holds the block's S values per lane (S = 2: a 128-block; S = 1: the 64-value tail) through
// all k routes: y_t[block] = sum over j ascending of w[t,j] * (sv2_e * R(scale2_e * v_slot[block])),
// the same operations in the same order as the workgroup combine (no contraction into FMAs, so both
// give the same bits). Lane j < k loads route j's slot, expert and weight once; routes are then taken
// JB at a time with all of a batch's loads issued before the first is used. Dropped routes add
// nothing. No LDS, no barrier.
template <int S, int SMAX>
__device__ __forceinline__ void combine_block(const CombineArgs& a, int t, int off, int lane) {
#pragma clang fp contract(off)
  constexpr int JB = SMAX > 0 ? 16 / SMAX : 16;
  const int H = a.rot.n, K = a.top_k;         // K <= 32
  const size_t plane = static_cast<size_t>(a.routes) * H;
  const int rl = t * K + (lane < K ? lane : K - 1);
  const int p_l = lane < K ? a.route_slot[rl] : -1;
  // expert and weight loads do not wait for the slot's (a dropped route's are never used)
  const int e_l = lane < K ? static_cast<int>(route_expert(a.ids, a.ids64, rl)) : 0;
  const float w_l = lane < K ? a.w[rl] : 0.0f;
  float acc[S];
#pragma unroll
  for (int i = 0; i < S; ++i) acc[i] = 0.0f;
  for (int j0 = 0; j0 < K; j0 += JB) {
    int p[JB];
    float vv[JB][S], c2[JB][S], sg[JB][S];
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) {
      const int j = j0 + jb < K ? j0 + jb : K - 1;
      p[jb] = j0 + jb < K ? __builtin_amdgcn_readlane(p_l, j) : -1;
      const int e = p[jb] >= 0 ? __builtin_amdgcn_readlane(e_l, j) : 0;   // a dropped route's id may be invalid
      const int pp = p[jb] >= 0 ? p[jb] : 0;
      const size_t vo = static_cast<size_t>(pp) * H + off + lane;
      const uint16_t* cs = a.scale2 + static_cast<size_t>(e) * H + off + lane;
      const uint16_t* ss = a.sv2 + static_cast<size_t>(e) * H + off + lane;
      if constexpr (SMAX == 0) {               // one fp16 plane, scale2 applied
#pragma unroll
        for (int i = 0; i < S; ++i) vv[jb][i] = h2f(a.v16[vo + 64 * i]);
      } else {
        sum_splits<S, SMAX, SMAX>(a.v + vo, plane, SMAX, vv[jb]);
#pragma unroll
        for (int i = 0; i < S; ++i) c2[jb][i] = h2f(cs[64 * i]);
      }
#pragma unroll
      for (int i = 0; i < S; ++i) sg[jb][i] = h2f(ss[64 * i]);
    }
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) {
      if (p[jb] < 0) continue;
      const float wt = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w_l), j0 + jb));
      if constexpr (SMAX > 0) {
#pragma unroll
        for (int i = 0; i < S; ++i) vv[jb][i] *= c2[jb][i];
      }
      if (!a.rot.identity) fwht_segment<S>(vv[jb], lane);
#pragma unroll
      for (int i = 0; i < S; ++i) acc[i] += wt * (vv[jb][i] * sg[jb][i]);
    }
  }
  float* out = a.y + static_cast<size_t>(t) * H + off + lane;
#pragma unroll
  for (int i = 0; i < S; ++i) out[64 * i] = acc[i];
}

template <int SMAX>
__global__ __launch_bounds__(256) void k_combine_blocks(CombineArgs a) {
  const int lane = threadIdx.x & 63;
  const int nseg = a.rot.nblk128 + a.rot.tail64;
  const int item = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x * 4 + (threadIdx.x >> 6)));
  const int t = item / nseg, seg = item - t * nseg;
  if (t >= a.tokens) return;
  if (seg < a.rot.nblk128) combine_block<2, SMAX>(a, t, seg * 128, lane);
  else combine_block<1, SMAX>(a, t, seg * 128, lane);
}

// Dense trellis linear, before its GEMM: workgroups [0, rot_blocks) rotate the tokens' rows, one
// item per wavefront (a whole row, or one 128-block of a long non-power-of-two row while tokens are
// few); the others write the GEMM tiles of the single expert and the combine's route tables.
template <int EPL>
__global__ __launch_bounds__(256) void k_linear_prep(LinearPrepArgs a) {
  if (static_cast<int>(blockIdx.x) < a.rot_blocks) {
    const int per = EPL > 0 ? 1 : rotate_items_per_route(a.rot);
    const int item = static_cast<int>(blockIdx.x * 4 + (threadIdx.x >> 6));
    const int t = item / per, seg = item - t * per;
    if (t < a.tokens) rotate_item<EPL, false>(a.rot, t, t, 0, seg, per);
    return;
  }
  const int i0 = (static_cast<int>(blockIdx.x) - a.rot_blocks) * 256 + static_cast<int>(threadIdx.x);
  const int stride = (static_cast<int>(gridDim.x) - a.rot_blocks) * 256;
  for (int i = i0; i < a.tokens; i += stride) {
    a.slot[i] = i;
    a.ids[i] = 0;
    a.w[i] = 1.0f;
  }
  const int nt = (a.tokens + a.tile_rows - 1) / a.tile_rows;
  for (int i = i0; i < nt; i += stride)
    a.gtiles[i] = make_int4(a.bits << 24, i * a.tile_rows, min(a.tile_rows, a.tokens - i * a.tile_rows), 0);
  if (i0 == 0) *a.num_gtiles = nt;
}

// Long power-of-two rows (n = 256 B with B = 4, 8, 16, i.e. 1024-4096 values) split over a workgroup
// of n/4 threads: wavefront w first transforms its contiguous 256 values (4 per lane; index bits 0-7,
// fwht_segment<4>), the block goes through LDS, and 256 threads then each hold the B values that
// share index bits 0-7 and transform index bits 8 and up in registers. The two passes cover every
// index bit once, so this is the same n-point Walsh-Hadamard transform, with 1/sqrt(n) applied as
// 1/16 and then 1/sqrt(B). A wavefront per row would walk 64 values per lane through twelve stages.
template <int B>
__device__ __forceinline__ void fwht_across_blocks(float (&u)[B]) {
#pragma unroll
  for (int h = 1; h < B; h <<= 1)
#pragma unroll
    for (int m = 0; m < B; ++m)
      if ((m & h) == 0) {
        const float x0 = u[m], x1 = u[m | h];
        u[m] = x0 + x1;
        u[m | h] = x0 - x1;
      }
  constexpr float kScale = B == 4 ? 0.5f : B == 8 ? 0.35355339059327373f : 0.25f;   // 1/sqrt(B)
#pragma unroll
  for (int m = 0; m < B; ++m) u[m] *= kScale;
}

// Dense linear input rotation with workgroup rows: workgroups [0, tokens) rotate row t (operand row
// t, sign vector su); the rest write the GEMM tiles and the combine's route tables.
template <int B>
__global__ __launch_bounds__(64 * B) void k_linear_prep_wide(LinearPrepArgs a) {
  __shared__ float row[256 * B];
  const RotateArgs& r = a.rot;
  if (static_cast<int>(blockIdx.x) < a.tokens) {
    const int t = blockIdx.x, n = 256 * B;
    const int lane = threadIdx.x & 63, off = static_cast<int>(threadIdx.x >> 6) * 256 + lane;
    const uint16_t* xr = r.x + static_cast<size_t>(t) * n + off;
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = bf16_to_f32(xr[64 * i]) * h2f(r.su1[off + 64 * i]);
    if (!r.rot.identity) fwht_segment<4>(v, lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) row[off + 64 * i] = v[i];
    __syncthreads();
    if (threadIdx.x < 256) {
      float u[B];
#pragma unroll
      for (int m = 0; m < B; ++m) u[m] = row[threadIdx.x + 256 * m];
      if (!r.rot.identity) fwht_across_blocks<B>(u);
      _Float16* o = static_cast<_Float16*>(r.a1) + static_cast<size_t>(t) * r.lda + threadIdx.x;
#pragma unroll
      for (int m = 0; m < B; ++m) o[256 * m] = static_cast<_Float16>(u[m]);
    }
    return;
  }
  const int i0 = (static_cast<int>(blockIdx.x) - a.tokens) * static_cast<int>(blockDim.x) + static_cast<int>(threadIdx.x);
  const int stride = (static_cast<int>(gridDim.x) - a.tokens) * static_cast<int>(blockDim.x);
  for (int i = i0; i < a.tokens; i += stride) {
    a.slot[i] = i;
    a.ids[i] = 0;
    a.w[i] = 1.0f;
  }
  const int nt = (a.tokens + a.tile_rows - 1) / a.tile_rows;
  for (int i = i0; i < nt; i += stride)
    a.gtiles[i] = make_int4(a.bits << 24, i * a.tile_rows, min(a.tile_rows, a.tokens - i * a.tile_rows), 0);
  if (i0 == 0) *a.num_gtiles = nt;
}

// Combine of one route per token (top-k = 1, the dense linear's case) with workgroup rows:
// y_t = w[t] * sv2_e * R_n(scale2_e * v_slot), or zeros for a dropped route; one workgroup per token.
template <int B, int SMAX>
__global__ __launch_bounds__(64 * B) void k_combine_one_wide(CombineArgs a) {
  __shared__ float row[256 * B];
  const int t = blockIdx.x, n = 256 * B;
  const int lane = threadIdx.x & 63, off = static_cast<int>(threadIdx.x >> 6) * 256 + lane;
  const int p = a.route_slot[t];
  const long long id = route_expert(a.ids, a.ids64, t);
  const float wt = a.w[t];
  const int e = p >= 0 ? static_cast<int>(id) : 0;
  float v[4];
  if (p >= 0) {
    const size_t plane = static_cast<size_t>(a.routes) * n;
    const size_t vo = static_cast<size_t>(p) * n + off;
    const uint16_t* c2 = a.scale2 + static_cast<size_t>(e) * n + off;
    scaled_values<4, SMAX, (SMAX > 0 ? splits_unroll<4, SMAX>(1) : 1)>(a.v + vo, a.v16 + vo, plane, SMAX, c2, v);
    if (!a.rot.identity) fwht_segment<4>(v, lane);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = 0.0f;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) row[off + 64 * i] = v[i];
  __syncthreads();
  if (threadIdx.x < 256) {
    float u[B];
#pragma unroll
    for (int m = 0; m < B; ++m) u[m] = row[threadIdx.x + 256 * m];
    if (p >= 0 && !a.rot.identity) fwht_across_blocks<B>(u);
    const uint16_t* sg = a.sv2 + static_cast<size_t>(e) * n + threadIdx.x;
    float* y = a.y + static_cast<size_t>(t) * n + threadIdx.x;
#pragma unroll
    for (int m = 0; m < B; ++m) y[256 * m] = p >= 0 ? wt * (u[m] * h2f(sg[256 * m])) : 0.0f;
  }
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

inline unsigned blocks_for(long long rows) { return static_cast<unsigned>((rows + 3) / 4); }

// most = 0: one fp16 plane with the channel scale applied
template <class F>
void dispatch_smax(int most, F&& f) {
  switch (most) {
    case 0: f(std::integral_constant<int, 0>{}); break;
    case 1: f(std::integral_constant<int, 1>{}); break;
    case 2: f(std::integral_constant<int, 2>{}); break;
    case 4: f(std::integral_constant<int, 4>{}); break;
    default: f(std::integral_constant<int, 8>{}); break;
  }
}

constexpr size_t kCombineLdsBytes = 65536;
constexpr int kActSplitMaxSlots = 2048;   // slots up to which the activation takes a workgroup per slot

// Wavefronts per combine workgroup: at most 16, at most top_k, and LDS within kCombineLdsBytes
// (which keeps H = 4096 at 3, inside that kernel's 256-thread bound).
int combine_waves(int hidden, int top_k) {
  int w = kCombineLdsBytes / (4 * hidden) - 1;     // (W + 1) rows of H floats, plus W flags
  while (w > 1 && static_cast<size_t>(w + 1) * hidden * 4 + 4 * w > kCombineLdsBytes) --w;
  w = w < top_k ? w : top_k;
  w = w < 16 ? w : 16;
  return w < 1 ? 1 : w;
}

}  // namespace

void launch_act(const ActArgs& a_in, bool mx, hipStream_t s) {
  ActArgs a = a_in;
  // (rows of 512 values from one fp16 plane, rotated: kActSlots slots per wavefront, see k_act; a
  // plane is launched as k_act<E, false, 0> whatever mx says)
  const bool grouped = a.z16 && a.rot.pow2 && a.rot.n == 512 && !a.rot.identity;
  a.act_blocks = grouped ? static_cast<int>(blocks_for((static_cast<long long>(a.routes) + kActSlots - 1) / kActSlots))
                         : static_cast<int>(blocks_for(static_cast<long long>(a.routes) * row_segments(a.rot)));
  const long long zero_blocks = a.y_zero ? (a.y_count + 1023) / 1024 : 0;
  const unsigned grid = static_cast<unsigned>(a.act_blocks + zero_blocks);
  // few slots of 512 values from fp32 planes (y not zeroed here): a workgroup per slot
  if (!a.z16 && a.rot.pow2 && a.rot.n == 512 && !a.y_zero && a.routes <= kActSplitMaxSlots) {
    dispatch_smax(a.nsplit, [&](auto sm) {
      constexpr int SM = decltype(sm)::value;
      if constexpr (SM > 0) {
        if (mx) hipLaunchKernelGGL((k_act_split<true, SM>), dim3(a.routes), dim3(256), 0, s, a);
        else hipLaunchKernelGGL((k_act_split<false, SM>), dim3(a.routes), dim3(256), 0, s, a);
      }
    });
    return;
  }
  dispatch_epl(a.rot, [&](auto epl) {
    dispatch_smax(a.z16 ? 0 : a.nsplit, [&](auto sm) {
      constexpr int E = decltype(epl)::value, SM = decltype(sm)::value;
      if constexpr (SM == 0) {
        hipLaunchKernelGGL((k_act<E, false, 0>), dim3(grid), dim3(256), 0, s, a);   // fp16 operands only
      } else {
        if (mx) hipLaunchKernelGGL((k_act<E, true, SM>), dim3(grid), dim3(256), 0, s, a);
        else hipLaunchKernelGGL((k_act<E, false, SM>), dim3(grid), dim3(256), 0, s, a);
      }
    });
  });
}

// Rows split over a workgroup: power-of-two rows of 1024 to 4096 values (B = n / 256).
static int wide_rows_b(const RowRot& r) { return r.pow2 && r.n >= 1024 && r.n <= 4096 ? r.n / 256 : 0; }

void launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.top_k == 1 && wide_rows_b(a.rot) != 0) {
    dispatch_smax(a.v16 ? 0 : a.nsplit, [&](auto sm) {
      constexpr int SM = decltype(sm)::value;
      switch (wide_rows_b(a.rot)) {
        case 4: hipLaunchKernelGGL((k_combine_one_wide<4, SM>), dim3(a.tokens), dim3(256), 0, s, a); break;
        case 8: hipLaunchKernelGGL((k_combine_one_wide<8, SM>), dim3(a.tokens), dim3(512), 0, s, a); break;
        default: hipLaunchKernelGGL((k_combine_one_wide<16, SM>), dim3(a.tokens), dim3(1024), 0, s, a); break;
      }
    });
    return;
  }
  if (!a.rot.pow2 && !a.split_segments) {
    const unsigned grid = blocks_for(static_cast<long long>(a.tokens) * row_segments(a.rot));
    dispatch_smax(a.v16 ? 0 : a.nsplit, [&](auto sm) {
      hipLaunchKernelGGL((k_combine_blocks<decltype(sm)::value>), dim3(grid), dim3(256), 0, s, a);
    });
    return;
  }
  const bool split = !a.rot.pow2;                // few tokens: one workgroup per (token, segment)
  const int L = split ? 128 : a.rot.n;           // longest segment a workgroup combines
  const int W = combine_waves(L, a.top_k);
  const size_t lds = static_cast<size_t>(W + 1) * L * 4 + 4 * W;
  const dim3 grid(a.tokens, split ? row_segments(a.rot) : 1);
  dispatch_epl(a.rot, [&](auto epl) {
    dispatch_smax(a.v16 ? 0 : a.nsplit, [&](auto sm) {
      constexpr int E = decltype(epl)::value, SM = decltype(sm)::value;
      hipLaunchKernelGGL((k_combine<E, SM>), grid, dim3(64 * W), lds, s, a);
    });
  });
}

void launch_linear_prep(const LinearPrepArgs& a, hipStream_t s) {
  if (const int b = wide_rows_b(a.rot.rot)) {
    const int meta = std::max(1, std::min(64, (a.tokens + 64 * b - 1) / (64 * b)));
    const dim3 grid(a.tokens + meta);
    if (b == 4) hipLaunchKernelGGL((k_linear_prep_wide<4>), grid, dim3(256), 0, s, a);
    else if (b == 8) hipLaunchKernelGGL((k_linear_prep_wide<8>), grid, dim3(512), 0, s, a);
    else hipLaunchKernelGGL((k_linear_prep_wide<16>), grid, dim3(1024), 0, s, a);
    return;
  }
  const int meta = std::max(1, std::min(64, (a.tokens + 255) / 256));
  const dim3 grid(a.rot_blocks + meta);
  dispatch_epl(a.rot.rot, [&](auto epl) {
    hipLaunchKernelGGL((k_linear_prep<decltype(epl)::value>), grid, dim3(256), 0, s, a);
  });
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
