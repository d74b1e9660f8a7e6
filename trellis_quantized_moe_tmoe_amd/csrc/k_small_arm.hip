// k_small_arm.hip -- the small-batch arm: the whole layer in one persistent launch.
//
// The small-M arm of "b12x fused MoE: TrellisMX (procedural NPK) source format with an in-tree P8
// runtime" (flashinfer PR #69, description: smallm_max_tokens, 16 by default) exists because at a
// few tokens the weights take a microsecond to stream and the layer's time goes to launches and
// to the dependent loads between its steps. On gfx950 a grid-wide barrier costs several
// microseconds (an L2 write-back per workgroup, then a single contended counter), more than a
// kernel boundary inside a graph, so this kernel has no grid barrier: each step hands its output
// to the next by data flow.
//
//  * Every workgroup builds the route map itself, in LDS, from the ids (at most kArmMaxRoutes
//    routes): the same stable token-major map as the route-map launch, so all workgroups agree.
//  * Each route's input rotation is done once, by one wavefront, which then raises the route's
//    ready flag. An FC1 unit (tile of up to 16 slots, 64 columns, one K split) first puts its
//    trellis words in flight, then waits for the flags of its rows and loads their operand rows.
//  * The wavefront that finishes the last FC1 unit of a tile (a per-tile counter) runs the
//    activation of the tile's rows and raises the tile's flag; FC2 units of the tile wait for it.
//  * The wavefront that finishes the last FC2 unit of a tile rotates, signs and weights the tile's
//    rows (the combine launch's per-route work), and the wavefront that completes the last route of
//    a token (a per-token counter) adds the token's k rows in ascending j and writes y.
//
// Hand-offs between workgroups use device-scope loads and stores (the sc1 cache policy), which
// the per-XCD L2 does not hold back, plus relaxed device-scope flags and counters published after
// the stores have completed (s_waitcnt vmcnt(0)); no L2 write-back or invalidate is issued.
//
// Flags and counters live in a library-owned device array, zero at load, one slot per scratch
// arena. A launch reads the slot's epoch once; flags are set to epoch + 1, counters carry epoch + 1
// in their high word (an atomic max installs it before a unit adds to the low word), and the
// launch that finishes the last token stores the new epoch. So nothing is cleared between calls,
// and stale values of earlier calls never match. Every wait is bounded: a wait that gives up
// marks the call failed in the arena's arm status word, poisons the slot (later calls on it then
// report failure instead of running) and ends its wavefront; every wavefront reaches the end.
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "tmoe_device.hpp"
#include "tmoe_internal.hpp"
#include "tmoe_rowbody.hpp"
#include "tmoe_routemap.hpp"

namespace tmoe {

struct ArmSlot {
  uint32_t epoch;                          // epoch of the last launch that completed
  uint32_t poisoned;                       // a launch gave up a wait: the flags are not trusted
  uint32_t pad0[62];
  unsigned long long tokens_done;          // (epoch << 32) | tokens whose row of y is written
  unsigned long long pad1[31];
  uint32_t route_ready[kArmMaxRoutes];     // = epoch once route r's FC1 operand row is stored
  uint32_t tile_ready[kArmMaxRoutes];      // = epoch once tile i's FC2 operand rows are stored
  unsigned long long tile_done[kArmMaxRoutes];    // (epoch << 32) | FC1 units of tile i done
  unsigned long long tile2_done[kArmMaxRoutes];   // (epoch << 32) | FC2 units of tile i done
  unsigned long long token_done[kArmMaxRoutes];   // (epoch << 32) | routes of token t rotated and weighted
};

}  // namespace tmoe

// One slot per scratch arena (registered on the host); zero when the code object is loaded.
static __device__ __align__(256) tmoe::ArmSlot arm_slots[tmoe::kArmSlots];

namespace tmoe {

namespace {

constexpr int kArmExperts = 512;
constexpr unsigned kArmSpin = 1u << 20;   // polls of one wait (about a second: each poll reads memory)
constexpr int ADF = 2;                    // K steps in flight per wavefront (fp16 units)
constexpr int ANS = 4;                    // 16-column strips per unit (64 columns)

// ------------------------------------------------------------------ device-scope hand-off
__device__ __forceinline__ void st_f32(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_f32(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_u16(uint16_t* p, uint16_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_u8(uint8_t* p, uint8_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint8_t ld_u8(const uint8_t* p) {
  return __hip_atomic_load(const_cast<uint8_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long ld_u64(const void* p) {
  return __hip_atomic_load(reinterpret_cast<unsigned long long*>(const_cast<void*>(p)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_flag(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_flag(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void ctr_open(unsigned long long* c, uint32_t ep) {
  __hip_atomic_fetch_max(c, static_cast<unsigned long long>(ep) << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Adds one arrival; true for the arrival that makes the count `target` (the counter was opened for
// this epoch by the same wavefront earlier, and the stores it publishes have completed).
__device__ __forceinline__ bool ctr_arrive(unsigned long long* c, uint32_t ep, uint32_t target) {
  const unsigned long long old = __hip_atomic_fetch_add(c, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return static_cast<uint32_t>(old >> 32) == ep && static_cast<uint32_t>(old) + 1u == target;
}
__device__ __forceinline__ void stores_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// A value the compiler must treat as computed here: lane-derived addresses of one step are then
// formed inside that step instead of being hoisted out of the persistent loops, where they would
// stay live through the other steps and their registers.
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

struct ArmLds {
  int cnt[4 * kArmExperts];      // per-wave counts while the map is built
  int sorted[kArmMaxRoutes];     // slot -> route
  int slot_e[kArmMaxRoutes];     // slot -> expert
  int rslot[kArmMaxRoutes];      // route -> slot, or -1 for a dropped route
  int off[kArmExperts + 1];      // first slot of expert e
  int toff[kArmExperts + 1];     // first 16-row tile of expert e
  int boff[kArmExperts + 1];     // payload bits of the experts before e
  short tile_e[kArmMaxRoutes];   // tile -> expert
  int4 scan[4];
  int bad[4];
  int ntiles, nvalid, ep, stop;
};

__device__ __forceinline__ int width_of(const ArmArgs& a, int e) {
  return static_cast<int>((a.packed_bits[e >> 3] >> (4 * (e & 7))) & 15u);
}

// Exclusive scan of one int4 per thread over the 256 threads; totals in *total.
__device__ __forceinline__ int4 scan256(int4 v, int4* smem, int4* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int4 x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y0 = __shfl_up(x.x, d, 64), y1 = __shfl_up(x.y, d, 64);
    const int y2 = __shfl_up(x.z, d, 64), y3 = __shfl_up(x.w, d, 64);
    if (lane >= d) {
      x.x += y0;
      x.y += y1;
      x.z += y2;
      x.w += y3;
    }
  }
  if (lane == 63) smem[w] = x;
  __syncthreads();
  int4 pre = make_int4(0, 0, 0, 0);
  for (int i = 0; i < w; ++i) {
    pre.x += smem[i].x;
    pre.y += smem[i].y;
    pre.z += smem[i].z;
    pre.w += smem[i].w;
  }
  int4 tot = make_int4(0, 0, 0, 0);
  for (int i = 0; i < 4; ++i) {
    tot.x += smem[i].x;
    tot.y += smem[i].y;
    tot.z += smem[i].z;
    tot.w += smem[i].w;
  }
  *total = tot;
  __syncthreads();
  return make_int4(pre.x + x.x - v.x, pre.y + x.y - v.y, pre.z + x.z - v.z, pre.w + x.w - v.w);
}

// The stable token-major route map of the call, in this workgroup's LDS (every workgroup builds
// the same one): four wavefronts count and place a quarter of the routes each.
__device__ __forceinline__ void arm_route_map(const ArmArgs& a, ArmLds& L) {
  const int tid = threadIdx.x, w = tid >> 6, E = a.E, R = a.R;
  for (int i = tid; i < 4 * E; i += 256) L.cnt[i] = 0;
  if (tid < 4) L.bad[tid] = 0;
  __syncthreads();
  RouteMapArgs ra{};
  ra.ids = a.ids;
  ra.ids64 = a.ids64;
  ra.routes = R;
  ra.num_experts = E;
  ra.sorted_routes = L.sorted;
  ra.slot_expert = L.slot_e;
  ra.route_slot = L.rslot;
  const int nbits = 32 - __clz(E);
  const int seg = (R + 3) / 4;                          // <= 128 routes: two chunks per wave
  const int beg = min(R, w * seg), end = min(R, beg + seg);
  int kept[kKeep];
  count_segment(ra, beg, end, nbits, L.cnt + w * E, L.bad + w, kept);
  __syncthreads();
  // experts 2 tid and 2 tid + 1: totals, 16-row tiles and widths, scanned across the workgroup
  int tot[2] = {0, 0}, til[2] = {0, 0}, bts[2] = {0, 0};
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int e = 2 * tid + q;
    if (e < E) {
      for (int ww = 0; ww < 4; ++ww) tot[q] += L.cnt[ww * E + e];
      til[q] = (tot[q] + 15) >> 4;
      bts[q] = width_of(a, e);
    }
  }
  int4 total;
  const int4 ex = scan256(make_int4(tot[0] + tot[1], til[0] + til[1], bts[0] + bts[1], 0), L.scan, &total);
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int e = 2 * tid + q;
    if (e < E) {
      L.off[e] = ex.x + (q ? tot[0] : 0);
      L.toff[e] = ex.y + (q ? til[0] : 0);
      L.boff[e] = ex.z + (q ? bts[0] : 0);
      int acc = L.off[e];
      for (int ww = 0; ww < 4; ++ww) {                   // per-wave starting slots
        const int c = L.cnt[ww * E + e];
        L.cnt[ww * E + e] = acc;
        acc += c;
      }
      for (int i = 0; i < til[q]; ++i) L.tile_e[L.toff[e] + i] = static_cast<short>(e);
    }
  }
  if (tid == 0) {
    L.off[E] = total.x;
    L.toff[E] = total.y;
    L.boff[E] = total.z;
    L.ntiles = total.y;
    L.nvalid = total.x;
  }
  __syncthreads();
  place_segment(ra, beg, end, nbits, L.cnt + w * E, kept);
  __syncthreads();
}

// A bounded wait gave up: mark the call failed, poison the slot and stop this wavefront.
__device__ __forceinline__ void arm_fail(const ArmArgs& a) {
  if ((threadIdx.x & 63) == 0) {
    atomicOr(reinterpret_cast<unsigned*>(a.arm_status), 1u);
    st_flag(&a.slot->poisoned, 1u);
  }
}

// Wait until flag[idx] == ep for every lane with want set (idx per lane); false if it gave up.
__device__ __forceinline__ bool wait_flags(const uint32_t* flags, int idx, bool want, uint32_t ep) {
  bool ok = !want || ld_flag(flags + idx) == ep;
  unsigned it = 0;
  while (!__all(ok)) {
    if (++it >= kArmSpin) return false;
    __builtin_amdgcn_s_sleep(2);
    if (!ok) ok = ld_flag(flags + idx) == ep;
  }
  return true;
}

// Runtime values per lane of a rotation row -> compile-time constant (0: 128/64 blocks).
template <class F>
__device__ __forceinline__ void with_epl(const RowRot& r, F&& f) {
  if (!r.pow2) {
    f(std::integral_constant<int, 0>{});
    return;
  }
  switch (r.n >> 6) {
    case 2: f(std::integral_constant<int, 2>{}); break;
    case 4: f(std::integral_constant<int, 4>{}); break;
    case 8: f(std::integral_constant<int, 8>{}); break;
    default: f(std::integral_constant<int, 16>{}); break;
  }
}

// Call f(S, off) for every rotation segment of a row (one power-of-two block of EPL values per
// lane, or 128-blocks and a 64-block).
template <int EPL, class F>
__device__ __forceinline__ void each_segment(const RowRot& r, F&& f) {
  if constexpr (EPL > 0) {
    f(std::integral_constant<int, EPL>{}, 0);
  } else {
    for (int b = 0; b < r.nblk128; ++b) f(std::integral_constant<int, 2>{}, b * 128);
    if (r.tail64) f(std::integral_constant<int, 1>{}, r.nblk128 * 128);
  }
}

// MXFP8 of one value per lane (each 32-lane half is one block), stored device-scope.
__device__ __forceinline__ void mx_store_dev(float v, int lane, uint8_t* q_row, uint8_t* s_row, int idx) {
  const float amax = half_wave_amax(v);
  const int e = mx_exponent(amax);
  float sv = ldexpf(v, -e);
  sv = fminf(fmaxf(sv, -448.0f), 448.0f);
  st_u8(q_row + idx, static_cast<uint8_t>(fp8x2_from_f32(sv, 0.0f) & 0xffu));
  if ((lane & 31) == 0) st_u8(s_row + (idx >> 5), static_cast<uint8_t>(e + 127));
}

__device__ __forceinline__ uint16_t f16_bits(float v) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
}

// out[i] += sum over split planes s < splits, ascending, of src[s * plane + 64 i] (device scope),
// with up to 64 loads in flight per lane before the adds of a round.
template <int S>
__device__ __forceinline__ void split_sum_dev(const float* src, size_t plane, int splits, float (&out)[S]) {
  constexpr int SU = S >= 16 ? 2 : S >= 8 ? 4 : 8;
#pragma unroll
  for (int i = 0; i < S; ++i) out[i] = 0.0f;
  for (int s0 = 0; s0 < splits; s0 += SU) {
    float t[SU][S];
#pragma unroll
    for (int u = 0; u < SU; ++u)
      if (s0 + u < splits)
#pragma unroll
        for (int i = 0; i < S; ++i) t[u][i] = ld_f32(src + (s0 + u) * plane + 64 * i);
#pragma unroll
    for (int u = 0; u < SU; ++u)
      if (s0 + u < splits)
#pragma unroll
        for (int i = 0; i < S; ++i) out[i] += t[u][i];
  }
}

// S consecutive fp16 values (16-byte aligned) as floats.
template <int S>
__device__ __forceinline__ void ld_h16_blocked(const uint16_t* src, float (&out)[S]) {
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
#pragma unroll
  for (int c = 0; c < S / 8; ++c) {
    const h8 v = reinterpret_cast<const h8*>(src)[c];
#pragma unroll
    for (int i = 0; i < 8; ++i) out[8 * c + i] = static_cast<float>(v[i]);
  }
}

// S consecutive values as fp16, device scope, four per 64-bit store.
template <int S>
__device__ __forceinline__ void st_h16_blocked(uint16_t* dst, const float (&v)[S]) {
#pragma unroll
  for (int c = 0; c < S / 4; ++c) {
    const unsigned long long w = static_cast<unsigned long long>(f16_bits(v[4 * c])) |
                                 static_cast<unsigned long long>(f16_bits(v[4 * c + 1])) << 16 |
                                 static_cast<unsigned long long>(f16_bits(v[4 * c + 2])) << 32 |
                                 static_cast<unsigned long long>(f16_bits(v[4 * c + 3])) << 48;
    __hip_atomic_store(reinterpret_cast<unsigned long long*>(dst) + c, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// out[i] = sum over split planes s < splits, ascending, of src[s * plane + i] for S consecutive
// floats per lane (8-byte aligned), device scope.
template <int S>
__device__ __forceinline__ void split_sum_blocked_dev(const float* src, size_t plane, int splits, float (&out)[S]) {
  constexpr int SU = S >= 16 ? 2 : 4;
#pragma unroll
  for (int i = 0; i < S; ++i) out[i] = 0.0f;
  for (int s0 = 0; s0 < splits; s0 += SU) {
    float t[SU][S];
#pragma unroll
    for (int u = 0; u < SU; ++u)
      if (s0 + u < splits)
#pragma unroll
        for (int c = 0; c < S / 2; ++c) {
          const unsigned long long w = ld_u64(src + (s0 + u) * plane + 2 * c);
          t[u][2 * c] = __uint_as_float(static_cast<uint32_t>(w));
          t[u][2 * c + 1] = __uint_as_float(static_cast<uint32_t>(w >> 32));
        }
#pragma unroll
    for (int u = 0; u < SU; ++u)
      if (s0 + u < splits)
#pragma unroll
        for (int i = 0; i < S; ++i) out[i] += t[u][i];
  }
}

__device__ __forceinline__ bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// ------------------------------------------------------------------ row steps
// Input rotation of route r (token t, expert e): a = R_H(su1_e * x_t) into operand row r.
template <bool MX, int EPL>
__device__ __forceinline__ void arm_rotate(const ArmArgs& a, int r, int t, int e, int lane_in) {
  const int lane = opaque(lane_in);
  const int H = a.H;
  each_segment<EPL>(a.rot_h, [&](auto s_c, int off) {
    constexpr int S = decltype(s_c)::value;
    float v[S];
    if constexpr (!MX && S >= 8) {
      // blocked: element off + S lane + i, 16-byte loads (the rotation launch's layout and order)
      if (aligned16(a.su1)) {
        typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
        const u16x8* xr = reinterpret_cast<const u16x8*>(a.x + static_cast<size_t>(t) * H + off + S * lane);
        const u16x8* sr = reinterpret_cast<const u16x8*>(a.su1 + static_cast<size_t>(e) * H + off + S * lane);
#pragma unroll
        for (int c = 0; c < S / 8; ++c) {
          const u16x8 xv = xr[c], sv = sr[c];
#pragma unroll
          for (int i = 0; i < 8; ++i) v[8 * c + i] = bf16_to_f32(xv[i]) * h2f(sv[i]);
        }
        if (!a.rot_h.identity) fwht_segment<S>(v, lane);
        st_h16_blocked<S>(reinterpret_cast<uint16_t*>(a.a1) + static_cast<size_t>(r) * a.lda + off + S * lane, v);
        return;
      }
    }
    const uint16_t* xr = a.x + static_cast<size_t>(t) * H + off + lane;
    const uint16_t* sr = a.su1 + static_cast<size_t>(e) * H + off + lane;
#pragma unroll
    for (int i = 0; i < S; ++i) v[i] = bf16_to_f32(xr[64 * i]) * h2f(sr[64 * i]);
    if (!a.rot_h.identity) fwht_segment<S>(v, lane);
    if constexpr (!MX) {
      uint16_t* o = reinterpret_cast<uint16_t*>(a.a1) + static_cast<size_t>(r) * a.lda + off + lane;
#pragma unroll
      for (int i = 0; i < S; ++i) st_u16(o + 64 * i, f16_bits(v[i]));
    } else {
      uint8_t* q = a.a1 + static_cast<size_t>(r) * H;
      uint8_t* sc = a.a1s + static_cast<size_t>(r) * (H / 32);
#pragma unroll
      for (int i = 0; i < S; ++i) mx_store_dev(v[i], lane, q, sc, off + 64 * i + lane);
    }
  });
}

// Activation of slot p (expert e): b = R_I(su2 * silu(sv1g * R_I(c1g * zg)) * (sv1u * R_I(c1u * zu))).
// Gate, then up, then their product: scheduling barriers keep each part's loads from being
// hoisted over the others (every value of a row segment is live in registers).
template <bool MX, int EPL>
__device__ __forceinline__ void arm_act(const ArmArgs& a, int p, int e, int lane_in) {
  const int lane = opaque(lane_in);
  const int I = a.I;
  const size_t plane = static_cast<size_t>(a.R) * 2 * I;
  each_segment<EPL>(a.rot_i, [&](auto s_c, int off) {
    constexpr int S = decltype(s_c)::value;
    if constexpr (!MX && S >= 8) {
      // blocked: element off + S lane + i, as the activation launch lays out and orders it; gate,
      // then up, then their product (scheduling barriers keep the parts' loads apart)
      if (aligned16(a.scale1) && aligned16(a.sv1) && aligned16(a.su2)) {
        const size_t erow = static_cast<size_t>(e) * 2 * I + off + S * lane;
        const float* zr = a.z + static_cast<size_t>(p) * 2 * I + off + S * lane;
        float zg[S], zu[S];
        auto half_row = [&](float (&v)[S], int h) {     // h = 0: gate, I: up
          float c[S], sgn[S];
          ld_h16_blocked<S>(a.scale1 + erow + h, c);
          ld_h16_blocked<S>(a.sv1 + erow + h, sgn);
          split_sum_blocked_dev<S>(zr + h, plane, a.s1, v);
#pragma unroll
          for (int i = 0; i < S; ++i) v[i] *= c[i];
          if (!a.rot_i.identity) fwht_segment<S>(v, lane);
#pragma unroll
          for (int i = 0; i < S; ++i) v[i] *= sgn[i];
          __builtin_amdgcn_sched_barrier(0);
        };
        half_row(zg, 0);
        half_row(zu, I);
        float s2[S];
        ld_h16_blocked<S>(a.su2 + static_cast<size_t>(e) * I + off + S * lane, s2);
        float bb[S];
#pragma unroll
        for (int i = 0; i < S; ++i) {
          const float g = zg[i], u = zu[i];
          const float h = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;   // SiLU(g) * u
          bb[i] = h * s2[i];
        }
        if (!a.rot_i.identity) fwht_segment<S>(bb, lane);
        st_h16_blocked<S>(reinterpret_cast<uint16_t*>(a.b) + static_cast<size_t>(p) * a.ldb + off + S * lane, bb);
        return;
      }
    }
    const float* zr = a.z + static_cast<size_t>(p) * 2 * I + off + lane;
    const uint16_t* c1 = a.scale1 + static_cast<size_t>(e) * 2 * I + off + lane;
    const uint16_t* s1 = a.sv1 + static_cast<size_t>(e) * 2 * I + off + lane;
    const uint16_t* s2 = a.su2 + static_cast<size_t>(e) * I + off + lane;
    float g[S], u[S];
    auto half_row = [&](float (&v)[S], int h) {      // h = 0: gate, I: up
      split_sum_dev<S>(zr + h, plane, a.s1, v);
#pragma unroll
      for (int i = 0; i < S; ++i) v[i] *= h2f(c1[h + 64 * i]);
      if (!a.rot_i.identity) fwht_segment<S>(v, lane);
#pragma unroll
      for (int i = 0; i < S; ++i) v[i] *= h2f(s1[h + 64 * i]);
      __builtin_amdgcn_sched_barrier(0);
    };
    half_row(g, 0);
    half_row(u, I);
#pragma unroll
    for (int i = 0; i < S; ++i) {
      const float h = g[i] * __builtin_amdgcn_rcpf(1.0f + __expf(-g[i])) * u[i];   // SiLU(g) * u
      g[i] = h * h2f(s2[64 * i]);
    }
    if (!a.rot_i.identity) fwht_segment<S>(g, lane);
    if constexpr (!MX) {
      uint16_t* o = reinterpret_cast<uint16_t*>(a.b) + static_cast<size_t>(p) * a.ldb + off + lane;
#pragma unroll
      for (int i = 0; i < S; ++i) st_u16(o + 64 * i, f16_bits(g[i]));
    } else {
      uint8_t* q = a.b + static_cast<size_t>(p) * I;
      uint8_t* sc = a.bs + static_cast<size_t>(p) * (I / 32);
#pragma unroll
      for (int i = 0; i < S; ++i) mx_store_dev(g[i], lane, q, sc, off + 64 * i + lane);
    }
  });
}

// The combine launch's per-route work for slot p (route r, expert e): o = w[r] * sv2_e *
// R_H(scale2_e * v_p), same operations and order, stored device-scope over the slot's row of the
// first split plane of v (every plane of the row is read before it is overwritten).
template <int EPL>
__device__ __forceinline__ void arm_route_out(const ArmArgs& a, const ArmLds& L, int p, int lane_in) {
  const int lane = opaque(lane_in);
  const int H = a.H;
  const size_t plane = static_cast<size_t>(a.R) * H;
  const int r = L.sorted[p], e = L.slot_e[p];
  const float wt = a.w[r];
  each_segment<EPL>(a.rot_h, [&](auto s_c, int off) {
    constexpr int S = decltype(s_c)::value;
    float* vr = a.v + static_cast<size_t>(p) * H + off + lane;
    float vv[S];
    split_sum_dev<S>(vr, plane, a.s2, vv);
    const uint16_t* c2 = a.scale2 + static_cast<size_t>(e) * H + off + lane;
    const uint16_t* sg = a.sv2 + static_cast<size_t>(e) * H + off + lane;
#pragma unroll
    for (int i = 0; i < S; ++i) vv[i] *= h2f(c2[64 * i]);
    if (!a.rot_h.identity) fwht_segment<S>(vv, lane);
#pragma unroll
    for (int i = 0; i < S; ++i) st_f32(vr + 64 * i, wt * (vv[i] * h2f(sg[64 * i])));
  });
}

// y_t = sum over j ascending of the rows arm_route_out left for token t's routes (dropped routes
// add nothing): the combine launch's sum, in its order; the rows of JB routes are loaded at once.
template <int EPL>
__device__ __forceinline__ void arm_token_sum(const ArmArgs& a, const ArmLds& L, int t, int lane_in) {
  const int lane = opaque(lane_in);
  const int H = a.H, K = a.K;
  each_segment<EPL>(a.rot_h, [&](auto s_c, int off) {
    constexpr int S = decltype(s_c)::value;
    constexpr int JB = S >= 16 ? 4 : 8;
    float acc[S];
#pragma unroll
    for (int i = 0; i < S; ++i) acc[i] = 0.0f;
    for (int j0 = 0; j0 < K; j0 += JB) {
      float o[JB][S];
      int pj[JB];
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) {
        pj[jb] = j0 + jb < K ? L.rslot[t * K + j0 + jb] : -1;
        if (pj[jb] >= 0)
#pragma unroll
          for (int i = 0; i < S; ++i) o[jb][i] = ld_f32(a.v + static_cast<size_t>(pj[jb]) * H + off + lane + 64 * i);
      }
#pragma unroll
      for (int jb = 0; jb < JB; ++jb)
        if (pj[jb] >= 0)
#pragma unroll
          for (int i = 0; i < S; ++i) acc[i] += o[jb][i];
    }
    float* out = a.y + static_cast<size_t>(t) * H + off + lane;
#pragma unroll
    for (int i = 0; i < S; ++i) out[64 * i] = acc[i];
  });
}

// One more finished token; the launch that finishes the last one publishes its epoch.
__device__ __forceinline__ void token_finished(const ArmArgs& a, uint32_t ep) {
  stores_done();
  if ((threadIdx.x & 63) == 0) {
    ctr_open(&a.slot->tokens_done, ep);
    stores_done();
    if (ctr_arrive(&a.slot->tokens_done, ep, static_cast<uint32_t>(a.T))) st_flag(&a.slot->epoch, ep);
  }
}

// ------------------------------------------------------------------ GEMM units
template <class T>
using gptr = const T __attribute__((address_space(1)))*;

template <class T>
__device__ __forceinline__ gptr<T> uniform_ptr(const T* p) {
  const unsigned long long v = reinterpret_cast<unsigned long long>(p);
  const unsigned lo = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(v));
  const unsigned hi = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(v >> 32));
  return reinterpret_cast<gptr<T>>((static_cast<unsigned long long>(hi) << 32) | lo);
}

template <int BITS>
constexpr int arm_ring_tile_bits() { return BITS == kMixedWide ? 6 : (BITS > 4 ? BITS : 4); }
template <int BITS>
constexpr int arm_ring_words() { return ADF * (2 * ANS * 8 * arm_ring_tile_bits<BITS>() + 256); }

struct UnitGeom {            // one GEMM unit: (tile rows, 64 columns, K split)
  int e, row0, rows, ng, s;
  long long woff;            // first payload word of the expert
};

// fp16 unit: trellis words and A fragments arrive with direct global->LDS loads into the
// wavefront's LDS ring (ADF steps deep). The trellis words of the first steps are issued before
// the unit waits for its operand rows; the operand rows are then read device-scope (sc1).
template <int BITS, int FC, class Wait>
__device__ __forceinline__ bool arm_unit_f16(const ArmArgs& a, const ArmLds& L, const UnitGeom& g, int lane_in, uint32_t* ring,
                             uint32_t mask, uint32_t orv, Wait&& wait) {
  const int lane = opaque(lane_in);
  constexpr int TW = 8 * BITS;
  constexpr int BW = 2 * ANS * TW;
  constexpr int AOFF = 2 * ANS * 8 * arm_ring_tile_bits<BITS>();
  constexpr int STAGE = AOFF + 256;
  constexpr int CPT = TW / 4;
  constexpr int NL = BW / 4 > 64 ? 2 : 1;
  const int K = FC == 1 ? a.H : a.I, N = FC == 1 ? 2 * a.I : a.H;
  const int splits = FC == 1 ? a.s1 : a.s2;
  const int NT = N >> 4;
  const int col = lane & 15, grp = lane >> 4;
  const int q = 2 * col + (grp & 1);
  const int ksteps = (K >> 5) / splits;
  const int ks0 = g.s * ksteps, ks1 = ks0 + ksteps;
  const int nt0 = g.ng * ANS;
  const long long fc_off = FC == 2 ? a.fc2_words_per_bit * BITS : 0;
  const gptr<uint32_t> mat = uniform_ptr(reinterpret_cast<const uint32_t*>(a.payload + g.woff + fc_off) +
                                         static_cast<size_t>(nt0) * TW);
  const gptr<_Float16> Abase = uniform_ptr(reinterpret_cast<const _Float16*>(FC == 1 ? a.a1 : a.b));
  const int lda = FC == 1 ? a.lda : a.ldb;
  const bool stager = lane < BW / 4;
  const int st_tile = lane / (ANS * CPT), st_strip = (lane / CPT) % ANS, st_chunk = lane % CPT;
  const int st_off = (st_tile * NT + st_strip) * TW + 4 * st_chunk;
  const int c2 = 64 + lane;
  const bool stager2 = NL == 2 && c2 < BW / 4;
  const int st2_off = ((c2 / (ANS * CPT)) * NT + (c2 / CPT) % ANS) * TW + 4 * (c2 % CPT);
  const int kstride = 2 * NT * TW;
  constexpr int NWW = dec_words<BITS>();
  const uint32_t dsh = dec_shift<BITS>(q);
  int rd[NWW];
#pragma unroll
  for (int i = 0; i < NWW; ++i) rd[i] = (grp >> 1) * ANS * TW + (dec_first_word<BITS>(q) + i + TW) % TW;
  const int slot_row = g.row0 + min(col, g.rows - 1);
  const long long arow = FC == 1 ? L.sorted[slot_row] : slot_row;
  const long long aoff = arow * lda + 8 * grp;
  const bool a_live = col < g.rows;

  f4 acc[ANS];
#pragma unroll
  for (int ns = 0; ns < ANS; ++ns) acc[ns] = f4{0.f, 0.f, 0.f, 0.f};

  auto issue_w = [&](int ks, int d) {
    uint32_t* slot = ring + d * STAGE;
    if (stager)
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(mat + static_cast<size_t>(ks) * kstride + st_off),
                                       (void __attribute__((address_space(3)))*)(slot), 16, 0, 0);
    if constexpr (NL == 2) {
      if (stager2)
        __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(mat + static_cast<size_t>(ks) * kstride + st2_off),
                                         (void __attribute__((address_space(3)))*)(slot + 256), 16, 0, 0);
    }
  };
  auto issue_a = [&](int ks, int d) {
    uint32_t* slot = ring + d * STAGE;
    if (a_live)     // device scope (sc1): the rows were stored by other workgroups in this launch
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(Abase + aoff + 32 * ks),
                                       (void __attribute__((address_space(3)))*)(slot + AOFF), 16, 0, 16);
  };
  auto step = [&](int d, int next, auto first) {
    if constexpr (decltype(first)::value)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(ADF - 1) : "memory");            // later steps' A loads
    else
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"((ADF - 1) * (NL + 1)) : "memory");
    const uint32_t* slot = ring + d * STAGE;
    uint32_t w[ANS][NWW];
#pragma unroll
    for (int ns = 0; ns < ANS; ++ns)
#pragma unroll
      for (int i = 0; i < NWW; ++i) w[ns][i] = slot[rd[i] + ns * TW];
    const half8 av = *reinterpret_cast<const half8*>(slot + AOFF + 4 * lane);
    half8 b[ANS];
#pragma unroll
    for (int ns = 0; ns < ANS; ++ns) b[ns] = decode8<BITS>(w[ns], dsh, mask, orv);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    issue_w(next, d);
    issue_a(next, d);
#pragma unroll
    for (int ns = 0; ns < ANS; ++ns) acc[ns] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, b[ns], acc[ns], 0, 0, 0);
  };
#pragma unroll
  for (int d = 0; d < ADF; ++d) issue_w(min(ks0 + d, ks1 - 1), d);
  const bool ok = wait();
#pragma unroll
  for (int d = 0; d < ADF; ++d) issue_a(min(ks0 + d, ks1 - 1), d);
  if (ok) {
    step(0, min(ks0 + ADF, ks1 - 1), std::true_type{});
    for (int ks = ks0 + 1; ks < ks1; ++ks) step((ks - ks0) & (ADF - 1), min(ks + ADF, ks1 - 1), std::false_type{});
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (!ok) return false;
  float* o = (FC == 1 ? a.z : a.v) + (static_cast<size_t>(g.s) * a.R + g.row0) * N + nt0 * 16 + col;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * grp + i;
    if (r < g.rows) {
#pragma unroll
      for (int ns = 0; ns < ANS; ++ns) st_f32(o + static_cast<size_t>(r) * N + 16 * ns, acc[ns][i]);
    }
  }
  return true;
}

// 32 E4M3 weights of one lane for one 128-deep K step (as the scaled-fp8 GEMM launch).
template <int BITS>
__device__ __forceinline__ i8v arm_decode_b_f8(const uint32_t (&w)[4][dec_words<BITS>()], const uint32_t (&sh)[2],
                                               uint32_t mask, uint32_t orv) {
  i8v b;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    uint32_t p[4];
    decode8_pairs<BITS>(w[g], sh[g & 1], mask, orv, p);
    b[2 * g] = static_cast<int>(fp8x4_from_pairs(p[0], p[1]));
    b[2 * g + 1] = static_cast<int>(fp8x4_from_pairs(p[2], p[3]));
  }
  return b;
}

// Scaled-fp8 unit (W4A8): operands in registers; trellis windows of the first steps are loaded
// before the wait, the E4M3 rows and their E8M0 scales device-scope after it.
template <int BITS, int FC, class Wait>
__device__ __forceinline__ bool arm_unit_f8(const ArmArgs& a, const ArmLds& L, const UnitGeom& g, int lane_in, uint32_t mask,
                            uint32_t orv, Wait&& wait) {
  const int lane = opaque(lane_in);
  constexpr int TW = 8 * BITS;
  constexpr int D8 = 2;
  const int K = FC == 1 ? a.H : a.I, N = FC == 1 ? 2 * a.I : a.H;
  const int splits = FC == 1 ? a.s1 : a.s2;
  const long long fc_off = FC == 2 ? a.fc2_words_per_bit * BITS : 0;
  const uint32_t* mat = reinterpret_cast<const uint32_t*>(a.payload + g.woff + fc_off);
  const int NT = N >> 4;
  const int col = lane & 15, grp = lane >> 4;
  const int ksteps = (K >> 7) / splits;
  const int ks0 = g.s * ksteps, ks1 = ks0 + ksteps;
  const int nt0 = g.ng * ANS;
  const uint8_t* A = FC == 1 ? a.a1 : a.b;
  const uint8_t* AS = FC == 1 ? a.a1s : a.bs;
  const int kblocks = K >> 5;
  const bool aok = col < g.rows;
  const int slot_row = g.row0 + (aok ? col : 0);
  const size_t rr = static_cast<size_t>(FC == 1 ? L.sorted[slot_row] : slot_row);
  const uint8_t* arow = A + rr * K + 16 * grp;
  const uint8_t* srow = AS + rr * kblocks + grp;
  f4 acc[ANS];
#pragma unroll
  for (int ns = 0; ns < ANS; ++ns) acc[ns] = f4{0.f, 0.f, 0.f, 0.f};
  constexpr int NWW = dec_words<BITS>();
  const uint32_t dsh[2] = {dec_shift<BITS>(2 * col), dec_shift<BITS>(2 * col + 1)};
  uint32_t w[D8][ANS][4][NWW];
  unsigned long long alo[D8][2], ahi[D8][2];
  int asc[D8];
  auto load_w = [&](int ks, uint32_t(&ww)[ANS][4][NWW]) {
    const int kt0 = 8 * ks + grp;
    const uint32_t* r0 = mat + static_cast<size_t>(kt0 * NT + nt0) * TW;
    const uint32_t* r1 = mat + static_cast<size_t>((kt0 + 4) * NT + nt0) * TW;
#pragma unroll
    for (int ns = 0; ns < ANS; ++ns) {
      load_dec_words<BITS>(r0 + ns * TW, 2 * col, ww[ns][0]);
      load_dec_words<BITS>(r0 + ns * TW, 2 * col + 1, ww[ns][1]);
      load_dec_words<BITS>(r1 + ns * TW, 2 * col, ww[ns][2]);
      load_dec_words<BITS>(r1 + ns * TW, 2 * col + 1, ww[ns][3]);
    }
  };
  auto load_a = [&](int ks, unsigned long long (&lo)[2], unsigned long long (&hi)[2], int& sc) {
    lo[0] = ld_u64(arow + 128 * ks);
    lo[1] = ld_u64(arow + 128 * ks + 8);
    hi[0] = ld_u64(arow + 128 * ks + 64);
    hi[1] = ld_u64(arow + 128 * ks + 72);
    sc = ld_u8(srow + 4 * ks);
  };
#pragma unroll
  for (int d = 0; d < D8; ++d) load_w(min(ks0 + d, ks1 - 1), w[d]);
  if (!wait()) return false;
#pragma unroll
  for (int d = 0; d < D8; ++d) load_a(min(ks0 + d, ks1 - 1), alo[d], ahi[d], asc[d]);
  for (int base = ks0; base < ks1; base += D8) {
#pragma unroll
    for (int d = 0; d < D8; ++d) {
      if (base + d < ks1) {
        i8v b[ANS];
#pragma unroll
        for (int ns = 0; ns < ANS; ++ns) b[ns] = arm_decode_b_f8<BITS>(w[d][ns], dsh, mask, orv);
        i8v av = i8v{static_cast<int>(alo[d][0]), static_cast<int>(alo[d][0] >> 32), static_cast<int>(alo[d][1]),
                     static_cast<int>(alo[d][1] >> 32), static_cast<int>(ahi[d][0]), static_cast<int>(ahi[d][0] >> 32),
                     static_cast<int>(ahi[d][1]), static_cast<int>(ahi[d][1] >> 32)};
        int sa = asc[d];
        if (!aok) {
          av = i8v{0, 0, 0, 0, 0, 0, 0, 0};
          sa = 127;
        }
        load_w(min(base + d + D8, ks1 - 1), w[d]);
        load_a(min(base + d + D8, ks1 - 1), alo[d], ahi[d], asc[d]);
#pragma unroll
        for (int ns = 0; ns < ANS; ++ns)
          acc[ns] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, b[ns], acc[ns], 0, 0, 0, sa, 0, 127);
      }
    }
  }
  float* o = (FC == 1 ? a.z : a.v) + (static_cast<size_t>(g.s) * a.R + g.row0) * N + nt0 * 16 + col;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * grp + i;
    if (r < g.rows) {
#pragma unroll
      for (int ns = 0; ns < ANS; ++ns) st_f32(o + static_cast<size_t>(r) * N + 16 * ns, acc[ns][i]);
    }
  }
  return true;
}

// Unit of the expert's width: BITS is the plan's shared width, or 0 (mixed 2-4) / kMixedWide (2-6).
template <int BITS, bool MX, int FC, class Wait>
__device__ __forceinline__ bool arm_unit(const ArmArgs& a, const ArmLds& L, const UnitGeom& g, int lane,
                                         uint32_t* ring, uint32_t mask, uint32_t orv, Wait&& wait) {
  auto go = [&](auto bits_c) -> bool {
    constexpr int B = decltype(bits_c)::value;
    if constexpr (MX) return arm_unit_f8<B, FC>(a, L, g, lane, mask, orv, wait);
    else return arm_unit_f16<B, FC>(a, L, g, lane, ring, mask, orv, wait);
  };
  if constexpr (BITS != 0 && BITS != kMixedWide) {
    return go(std::integral_constant<int, BITS>{});
  } else {
    const int bits = width_of(a, g.e);
    if (bits == 4) return go(std::integral_constant<int, 4>{});
    if (bits == 3) return go(std::integral_constant<int, 3>{});
    if constexpr (BITS == kMixedWide) {
      if (bits == 5) return go(std::integral_constant<int, 5>{});
      if (bits == 6) return go(std::integral_constant<int, 6>{});
    }
    return go(std::integral_constant<int, 2>{});
  }
}

__device__ __forceinline__ UnitGeom unit_geom(const ArmArgs& a, const ArmLds& L, int u, int NG, int S) {
  UnitGeom g;
  g.s = u % S;
  const int rest = u / S;
  g.ng = rest % NG;
  const int tile = rest / NG;
  g.e = L.tile_e[tile];
  g.row0 = L.off[g.e] + 16 * (tile - L.toff[g.e]);
  g.rows = min(16, L.off[g.e + 1] - g.row0);
  g.woff = static_cast<long long>(L.boff[g.e]) * a.words_per_bit;
  return g;
}

// ------------------------------------------------------------------ the kernel
template <int BITS, bool MX>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MX ? 2 : 4, 8))) void k_small_arm(ArmArgs a) {
  __shared__ ArmLds L;
  __shared__ uint32_t ring_all[MX ? 1 : 4 * arm_ring_words<BITS>()];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gw = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x) * 4 + wv);
  const int W = static_cast<int>(gridDim.x) * 4;
  if (tid == 0) {
    L.ep = static_cast<int>(ld_flag(&a.slot->epoch) + 1u);
    L.stop = ld_flag(&a.slot->poisoned) != 0;
    // the call's status word starts here (a failed wait, if any, comes a second later)
    if (blockIdx.x == 0) *a.arm_status = L.stop ? 2 : 0;
  }
  arm_route_map(a, L);
  if (L.stop) return;                            // an earlier call on this slot gave up a wait
  const uint32_t ep = static_cast<uint32_t>(L.ep);
  if (blockIdx.x == 0 && tid == 0) *a.status = L.bad[0] + L.bad[1] + L.bad[2] + L.bad[3];
  const int R = a.R, T = a.T, K = a.K;
  const int ntiles = L.ntiles;
  uint32_t* ring = ring_all + (MX ? 0 : wv * arm_ring_words<BITS>());
  const uint32_t mask = vreg_const(kMcgMask), orv = kMcgOr;
  ArmSlot* slot = a.slot;

  // 1. input rotations (items < R) and the rows of tokens without a valid route (items >= R)
  for (int i = gw; i < R + T; i += W) {
    if (i < R) {
      if (L.rslot[i] < 0) continue;
      const int e = L.slot_e[L.rslot[i]];
      with_epl(a.rot_h, [&](auto epl) { arm_rotate<MX, decltype(epl)::value>(a, i, i / K, e, lane); });
      stores_done();
      if (lane == 0) st_flag(&slot->route_ready[i], ep);
    } else {
      const int t = i - R;
      bool any = false;
      for (int j = 0; j < K; ++j) any |= L.rslot[t * K + j] >= 0;
      if (any) continue;
      for (int c = lane; c < a.H; c += 64) a.y[static_cast<size_t>(t) * a.H + c] = 0.0f;
      token_finished(a, ep);
    }
  }

  // 2. FC1 units; the last unit of a tile runs the tile's activation
  const int NG1 = (2 * a.I) >> 6, NG2 = a.H >> 6;
  const int U1 = ntiles * NG1 * a.s1, U2 = ntiles * NG2 * a.s2;
  for (int u = gw; u < U1; u += W) {
    const UnitGeom g = unit_geom(a, L, u, NG1, a.s1);
    const int tile = u / (NG1 * a.s1);
    if (lane == 0) ctr_open(&slot->tile_done[tile], ep);
    const int r_l = L.sorted[g.row0 + min(lane, g.rows - 1)];
    auto wait = [&]() { return wait_flags(slot->route_ready, r_l, lane < g.rows, ep); };
    if (!arm_unit<BITS, MX, 1>(a, L, g, lane, ring, mask, orv, wait)) {
      arm_fail(a);
      return;
    }
    stores_done();
    int last = 0;
    if (lane == 0) last = ctr_arrive(&slot->tile_done[tile], ep, static_cast<uint32_t>(NG1 * a.s1));
    if (__builtin_amdgcn_readfirstlane(last)) {
      for (int p = g.row0; p < g.row0 + g.rows; ++p)
        with_epl(a.rot_i, [&](auto epl) { arm_act<MX, decltype(epl)::value>(a, p, g.e, lane); });
      stores_done();
      if (lane == 0) st_flag(&slot->tile_ready[tile], ep);
    }
  }

  // 3. FC2 units. The last unit of a tile turns the tile's rows into weighted output rows; the
  //    wavefront that completes a token's last route adds the token's rows into y.
  for (int u = gw; u < U2; u += W) {
    const UnitGeom g = unit_geom(a, L, u, NG2, a.s2);
    const int tile = u / (NG2 * a.s2);
    if (lane == 0) ctr_open(&slot->tile2_done[tile], ep);
    auto wait = [&]() { return wait_flags(slot->tile_ready, tile, lane == 0, ep); };
    if (!arm_unit<BITS, MX, 2>(a, L, g, lane, ring, mask, orv, wait)) {
      arm_fail(a);
      return;
    }
    stores_done();
    int last = 0;
    if (lane == 0) last = ctr_arrive(&slot->tile2_done[tile], ep, static_cast<uint32_t>(NG2 * a.s2));
    if (!__builtin_amdgcn_readfirstlane(last)) continue;
    for (int p = g.row0; p < g.row0 + g.rows; ++p)
      with_epl(a.rot_h, [&](auto epl) { arm_route_out<decltype(epl)::value>(a, L, p, lane); });
    const bool row_l = lane < g.rows;
    const int tok_l = row_l ? L.sorted[g.row0 + lane] / K : 0;
    if (row_l) ctr_open(&slot->token_done[tok_l], ep);
    stores_done();
    bool fin = false;
    if (row_l) {
      int valid = 0;
      for (int j = 0; j < K; ++j) valid += L.rslot[tok_l * K + j] >= 0;
      fin = ctr_arrive(&slot->token_done[tok_l], ep, static_cast<uint32_t>(valid));
    }
    unsigned long long done = __ballot(fin);
    while (done) {
      const int l = __builtin_ctzll(done);
      done &= done - 1;
      const int t = __builtin_amdgcn_readlane(tok_l, l);
      with_epl(a.rot_h, [&](auto epl) { arm_token_sum<decltype(epl)::value>(a, L, t, lane); });
      token_finished(a, ep);
    }
  }
}

// ------------------------------------------------------------------ host side
struct ArmDevice {
  ArmSlot* slots = nullptr;                            // device address of arm_slots
  std::map<uintptr_t, int> slot_of;                    // scratch arena -> slot
  std::map<const void*, int> groups;                   // kernel -> workgroups co-resident on the GPU
};

std::mutex g_arm_mu;
std::vector<ArmDevice> g_arm_dev;

template <int BITS, bool MX>
const void* arm_kernel() { return reinterpret_cast<const void*>(&k_small_arm<BITS, MX>); }

const void* pick_kernel(int bits, bool mx) {
  if (mx) {
    switch (bits) {
      case 4: return arm_kernel<4, true>();
      case 3: return arm_kernel<3, true>();
      case 2: return arm_kernel<2, true>();
      default: return arm_kernel<0, true>();
    }
  }
  switch (bits) {
    case 4: return arm_kernel<4, false>();
    case 3: return arm_kernel<3, false>();
    case 2: return arm_kernel<2, false>();
    case 5: return arm_kernel<5, false>();
    case 6: return arm_kernel<6, false>();
    case kMixedWide: return arm_kernel<kMixedWide, false>();
    default: return arm_kernel<0, false>();
  }
}

}  // namespace

// Slot of the arena and the co-resident grid of the kernel on the current device; false when the
// arm cannot run here (slots exhausted, a HIP query failed, nothing fits).
bool small_arm_prepare(const void* arena, int bits, bool mx, ArmSlot** slot, int* groups) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return false;
  const void* k = pick_kernel(bits, mx);
  std::lock_guard<std::mutex> lock(g_arm_mu);
  if (static_cast<int>(g_arm_dev.size()) <= dev) g_arm_dev.resize(dev + 1);
  ArmDevice& d = g_arm_dev[dev];
  if (!d.slots) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(arm_slots)) != hipSuccess || !p) return false;
    d.slots = static_cast<ArmSlot*>(p);
  }
  auto it = d.slot_of.find(reinterpret_cast<uintptr_t>(arena));
  int s;
  if (it != d.slot_of.end()) {
    s = it->second;
  } else {
    if (static_cast<int>(d.slot_of.size()) >= kArmSlots) return false;
    s = static_cast<int>(d.slot_of.size());
    d.slot_of.emplace(reinterpret_cast<uintptr_t>(arena), s);
  }
  auto g = d.groups.find(k);
  if (g == d.groups.end()) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, 256, 0) != hipSuccess) return false;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return false;
    g = d.groups.emplace(k, per_cu * cus).first;
  }
  if (g->second <= 0) return false;
  *slot = d.slots + s;
  *groups = g->second;
  return true;
}

void launch_small_arm(const ArmArgs& a, int bits, bool mx, int groups, hipStream_t s) {
  ArmArgs arg = a;
  void* args[] = {&arg};
  (void)hipLaunchKernel(pick_kernel(bits, mx), dim3(groups), dim3(256), args, 0, s);
}

}  // namespace tmoe
