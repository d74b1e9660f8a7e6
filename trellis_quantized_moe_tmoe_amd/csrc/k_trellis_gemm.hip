// k_trellis_gemm.hip -- grouped GEMMs over the route map with trellis weights decoded in registers.
//
// Weights are never expanded in HBM: each wavefront streams the packed trellis words of its
// tiles, decodes them straight into MFMA operands ("W4A8 decode expands fixed-stride trellis
// payload directly into E4M3 MMA operands", "serve canonical Fruit QSRT atoms", Hot path) and
// multiplies them with the route rows of one expert. Output is route-major in slot order, one
// plane per K split, summed in a fixed order by the consumer kernel (deterministic; no atomics).
//
// Work unit of one wavefront: (GEMM tile = expert + up to 16*MG slots, 64 output columns, one K
// split). Units are dealt round-robin to a persistent grid whose size is fixed on the host, so the
// launch is graph-capturable although the tile count is only known on the device.
//
// Operand layouts (gfx950, checked on hardware):
//  * v_mfma_f32_16x16x32_f16: A lane l = row l%16, k = 8*(l/16)+[0,8); B lane l = column l%16,
//    k = 8*(l/16)+[0,8); C lane l = rows 4*(l/16)+[0,4), column l%16. With the tile element order
//    i = 16n + k, a B lane holds 8 consecutive elements of one trellis tile column.
//  * v_mfma_scale_f32_16x16x128_f8f6f4: lane l = row/column l%16; bytes 0-15 hold
//    k = 16*(l/16)+[0,16), bytes 16-31 hold k = 64+16*(l/16)+[0,16); the E8M0 scale of 32-wide
//    K block b of a row is read from lane 16*b + row.
#include "tmoe_device.hpp"
#include "tmoe_internal.hpp"

namespace tmoe {

namespace {

constexpr int NS = 4;   // 16-column strips per wavefront unit (64 columns)

template <int BITS, int MG>
__device__ __forceinline__ void unit_f16(const GemmArgs& a, const int4 t, int ng, int s, int lane) {
  constexpr int TW = 8 * BITS;                         // 32-bit words per 16x16 tile
  const ExpertInfo info = a.einfo[t.x];
  const uint32_t* mat = reinterpret_cast<const uint32_t*>(a.payload + info.word_offset +
                                                          a.fc2_words_per_bit * BITS);
  const int row0 = t.y, rows = t.z;
  const int NT = a.N >> 4;
  const int col = lane & 15, grp = lane >> 4;
  const int q = 2 * col + (grp & 1);                   // 8-element group inside the tile
  const int kt_off = grp >> 1;
  const int ksteps = (a.K >> 5) / a.splits;
  const int ks0 = s * ksteps, ks1 = ks0 + ksteps;
  const int nt0 = ng * NS;
  const _Float16* A = static_cast<const _Float16*>(a.a);

  const _Float16* arow[MG];
  bool aok[MG];
#pragma unroll
  for (int mg = 0; mg < MG; ++mg) {
    const int r = 16 * mg + col;
    aok[mg] = r < rows;
    arow[mg] = A + static_cast<size_t>(row0 + (aok[mg] ? r : 0)) * a.K + 8 * grp;
  }
  f4 acc[MG][NS];
#pragma unroll
  for (int mg = 0; mg < MG; ++mg)
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) acc[mg][ns] = f4{0.f, 0.f, 0.f, 0.f};

  uint32_t hi[NS], lo[NS];
  auto load = [&](int ks, uint32_t(&h)[NS], uint32_t(&l)[NS]) {
    const uint32_t* trow = mat + static_cast<size_t>((2 * ks + kt_off) * NT + nt0) * TW;
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) load_window<BITS>(trow + ns * TW, q, h[ns], l[ns]);
  };
  load(ks0, hi, lo);
  for (int ks = ks0; ks < ks1; ++ks) {
    uint32_t nhi[NS], nlo[NS];
    load(ks + 1 < ks1 ? ks + 1 : ks, nhi, nlo);       // prefetch the next step (in bounds)
    half8 b[NS];
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) b[ns] = decode8<BITS>(hi[ns], lo[ns], q);
#pragma unroll
    for (int mg = 0; mg < MG; ++mg) {
      half8 av = *reinterpret_cast<const half8*>(arow[mg] + 32 * ks);
      if (!aok[mg]) av = half8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int ns = 0; ns < NS; ++ns)
        acc[mg][ns] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, b[ns], acc[mg][ns], 0, 0, 0);
    }
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
      hi[ns] = nhi[ns];
      lo[ns] = nlo[ns];
    }
  }
  float* o = a.out + (static_cast<size_t>(s) * a.routes + row0) * a.N + nt0 * 16 + col;
#pragma unroll
  for (int mg = 0; mg < MG; ++mg)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * mg + 4 * grp + i;
      if (r < rows) {
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) o[static_cast<size_t>(r) * a.N + 16 * ns] = acc[mg][ns][i];
      }
    }
}

template <int MG>
__global__ __launch_bounds__(256) void k_gemm_f16(GemmArgs a) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int W = gridDim.x * 4;
  const int NG = a.N / (16 * NS);
  const int units = *a.num_gtiles * NG * a.splits;
  for (int u = gw; u < units; u += W) {
    const int s = u % a.splits;
    const int rest = u / a.splits;
    const int ng = rest % NG;
    const int4 t = a.gtiles[rest / NG];
    const int bits = a.einfo[t.x].bits;
    if (bits == 4) unit_f16<4, MG>(a, t, ng, s, lane);
    else if (bits == 3) unit_f16<3, MG>(a, t, ng, s, lane);
    else unit_f16<2, MG>(a, t, ng, s, lane);
  }
}

// 32 E4M3 weights of one lane for one 128-deep K step: tiles kt0 (bytes 0-15) and kt0+4
// (bytes 16-31) of one column, 16 consecutive elements of each.
template <int BITS>
__device__ __forceinline__ i8v decode_b_f8(const uint32_t* tile0, const uint32_t* tile1, int col) {
  uint32_t h0, l0, h1, l1, h2, l2, h3, l3;
  load_window<BITS>(tile0, 2 * col, h0, l0);
  load_window<BITS>(tile0, 2 * col + 1, h1, l1);
  load_window<BITS>(tile1, 2 * col, h2, l2);
  load_window<BITS>(tile1, 2 * col + 1, h3, l3);
  i8v b;
  uint32_t w0, w1;
  fp8x8_from_half8(decode8<BITS>(h0, l0, 2 * col), w0, w1);
  b[0] = static_cast<int>(w0); b[1] = static_cast<int>(w1);
  fp8x8_from_half8(decode8<BITS>(h1, l1, 2 * col + 1), w0, w1);
  b[2] = static_cast<int>(w0); b[3] = static_cast<int>(w1);
  fp8x8_from_half8(decode8<BITS>(h2, l2, 2 * col), w0, w1);
  b[4] = static_cast<int>(w0); b[5] = static_cast<int>(w1);
  fp8x8_from_half8(decode8<BITS>(h3, l3, 2 * col + 1), w0, w1);
  b[6] = static_cast<int>(w0); b[7] = static_cast<int>(w1);
  return b;
}

template <int BITS, int MG>
__device__ __forceinline__ void unit_f8(const GemmArgs& a, const int4 t, int ng, int s, int lane) {
  constexpr int TW = 8 * BITS;
  const ExpertInfo info = a.einfo[t.x];
  const uint32_t* mat = reinterpret_cast<const uint32_t*>(a.payload + info.word_offset +
                                                          a.fc2_words_per_bit * BITS);
  const int row0 = t.y, rows = t.z;
  const int NT = a.N >> 4;
  const int col = lane & 15, grp = lane >> 4;
  const int ksteps = (a.K >> 7) / a.splits;
  const int ks0 = s * ksteps, ks1 = ks0 + ksteps;
  const int nt0 = ng * NS;
  const uint8_t* A = static_cast<const uint8_t*>(a.a);
  const int kblocks = a.K >> 5;

  const uint8_t* arow[MG];
  const uint8_t* srow[MG];
  bool aok[MG];
#pragma unroll
  for (int mg = 0; mg < MG; ++mg) {
    const int r = 16 * mg + col;
    aok[mg] = r < rows;
    const size_t rr = static_cast<size_t>(row0 + (aok[mg] ? r : 0));
    arow[mg] = A + rr * a.K + 16 * grp;
    srow[mg] = a.a_scale + rr * kblocks + grp;
  }
  f4 acc[MG][NS];
#pragma unroll
  for (int mg = 0; mg < MG; ++mg)
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) acc[mg][ns] = f4{0.f, 0.f, 0.f, 0.f};

  for (int ks = ks0; ks < ks1; ++ks) {
    const int kt0 = 8 * ks + grp;
    const uint32_t* r0 = mat + static_cast<size_t>(kt0 * NT + nt0) * TW;
    const uint32_t* r1 = mat + static_cast<size_t>((kt0 + 4) * NT + nt0) * TW;
    i8v b[NS];
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) b[ns] = decode_b_f8<BITS>(r0 + ns * TW, r1 + ns * TW, col);
#pragma unroll
    for (int mg = 0; mg < MG; ++mg) {
      const uint4 lo = *reinterpret_cast<const uint4*>(arow[mg] + 128 * ks);
      const uint4 hi = *reinterpret_cast<const uint4*>(arow[mg] + 128 * ks + 64);
      i8v av = {static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z), static_cast<int>(lo.w),
                static_cast<int>(hi.x), static_cast<int>(hi.y), static_cast<int>(hi.z), static_cast<int>(hi.w)};
      int sa = srow[mg][4 * ks];
      if (!aok[mg]) {
        av = i8v{0, 0, 0, 0, 0, 0, 0, 0};
        sa = 127;
      }
#pragma unroll
      for (int ns = 0; ns < NS; ++ns)
        acc[mg][ns] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, b[ns], acc[mg][ns], 0, 0, 0, sa,
                                                                      0, 127);
    }
  }
  float* o = a.out + (static_cast<size_t>(s) * a.routes + row0) * a.N + nt0 * 16 + col;
#pragma unroll
  for (int mg = 0; mg < MG; ++mg)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * mg + 4 * grp + i;
      if (r < rows) {
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) o[static_cast<size_t>(r) * a.N + 16 * ns] = acc[mg][ns][i];
      }
    }
}

template <int MG>
__global__ __launch_bounds__(256) void k_gemm_f8(GemmArgs a) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int W = gridDim.x * 4;
  const int NG = a.N / (16 * NS);
  const int units = *a.num_gtiles * NG * a.splits;
  for (int u = gw; u < units; u += W) {
    const int s = u % a.splits;
    const int rest = u / a.splits;
    const int ng = rest % NG;
    const int4 t = a.gtiles[rest / NG];
    const int bits = a.einfo[t.x].bits;
    if (bits == 4) unit_f8<4, MG>(a, t, ng, s, lane);
    else if (bits == 3) unit_f8<3, MG>(a, t, ng, s, lane);
    else unit_f8<2, MG>(a, t, ng, s, lane);
  }
}

// Dense decode of one K x N matrix with the GEMM's own lane mapping (test hook).
template <int BITS>
__global__ __launch_bounds__(256) void k_debug_decode(const uint16_t* words, int K, int N, int as_e4m3,
                                                      void* out) {
  constexpr int TW = 8 * BITS;
  const int lane = threadIdx.x & 63;
  const int unit = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int NT = N >> 4;
  if (unit >= (K >> 5) * NT) return;
  const int kp = unit / NT, nt = unit % NT;
  const int col = lane & 15, grp = lane >> 4;
  const int q = 2 * col + (grp & 1);
  const int kt = 2 * kp + (grp >> 1);
  const uint32_t* tile = reinterpret_cast<const uint32_t*>(words) + static_cast<size_t>(kt * NT + nt) * TW;
  uint32_t hi, lo;
  load_window<BITS>(tile, q, hi, lo);
  const half8 h = decode8<BITS>(hi, lo, q);
  const int k0 = 16 * kt + 8 * (grp & 1);
  const int n = 16 * nt + col;
  if (!as_e4m3) {
    _Float16* o = static_cast<_Float16*>(out);
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) o[static_cast<size_t>(k0 + jj) * N + n] = h[jj];
  } else {
    uint32_t w0, w1;
    fp8x8_from_half8(h, w0, w1);
    uint8_t* o = static_cast<uint8_t*>(out);
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const uint32_t w = jj < 4 ? w0 : w1;
      o[static_cast<size_t>(k0 + jj) * N + n] = static_cast<uint8_t>((w >> (8 * (jj & 3))) & 0xffu);
    }
  }
}

}  // namespace

void launch_gemm_f16(const GemmArgs& a, int mg, int waves, hipStream_t s) {
  const dim3 grid((waves + 3) / 4), block(256);
  if (mg >= 4) hipLaunchKernelGGL(k_gemm_f16<4>, grid, block, 0, s, a);
  else if (mg == 2) hipLaunchKernelGGL(k_gemm_f16<2>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(k_gemm_f16<1>, grid, block, 0, s, a);
}

void launch_gemm_f8(const GemmArgs& a, int mg, int waves, hipStream_t s) {
  const dim3 grid((waves + 3) / 4), block(256);
  if (mg >= 4) hipLaunchKernelGGL(k_gemm_f8<4>, grid, block, 0, s, a);
  else if (mg == 2) hipLaunchKernelGGL(k_gemm_f8<2>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(k_gemm_f8<1>, grid, block, 0, s, a);
}

void launch_debug_decode(const uint16_t* matrix_words, int bits, int K, int N, int as_e4m3, void* out,
                         hipStream_t s) {
  const int units = (K / 32) * (N / 16);
  const dim3 grid((units + 3) / 4), block(256);
  if (bits == 4) hipLaunchKernelGGL(k_debug_decode<4>, grid, block, 0, s, matrix_words, K, N, as_e4m3, out);
  else if (bits == 3) hipLaunchKernelGGL(k_debug_decode<3>, grid, block, 0, s, matrix_words, K, N, as_e4m3, out);
  else hipLaunchKernelGGL(k_debug_decode<2>, grid, block, 0, s, matrix_words, K, N, as_e4m3, out);
}

}  // namespace tmoe
