// k_route_map.hip -- stable token-major route map: one workgroup up to 4096 routes, else a count
// launch and a placement launch over 1024-route chunks; the same launch carries the input rotation.
//
// The route map is materialised once and consumed directly by FC1 and FC2 ("serve canonical Fruit
// QSRT atoms", Hot path); per-expert counts and an exclusive prefix give expert offsets and routed
// blocks ("integrate EXL3 Trellis into the fused W4A16 API", review of route_pack.py). Stable
// token-major order within an expert
// follows the O(routes + experts * tiles) stable design asked for in the review of route_pack.py
// on "Share trellis preparation across native and EXL3 containers": the routes are walked once per
// pass in wave-sized chunks, and per-wave, per-expert running positions replace any rescan.
//
// Same-expert lanes of a 64-route chunk are found with the ballot multi-split of
// tmoe_routemap.hpp: ceil(log2(E+1)) ballots per chunk, independent of how many distinct experts
// the chunk holds.
#include "tmoe_device.hpp"
#include "tmoe_internal.hpp"
#include "tmoe_rowbody.hpp"
#include "tmoe_routemap.hpp"

namespace tmoe {

namespace {

constexpr int kWaves = 16;           // 1024 threads
constexpr int kMaxExperts = 512;

// Exclusive scans of four values per thread over the workgroup at once; totals returned in *total.
__device__ int4 block_exclusive_scan4(int4 v, int4* smem, int4* total) {
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
  if (w == 0) {
    int4 s = lane < kWaves ? smem[lane] : make_int4(0, 0, 0, 0);
#pragma unroll
    for (int d = 1; d < kWaves; d <<= 1) {
      const int y0 = __shfl_up(s.x, d, 64), y1 = __shfl_up(s.y, d, 64);
      const int y2 = __shfl_up(s.z, d, 64), y3 = __shfl_up(s.w, d, 64);
      if (lane >= d) {
        s.x += y0;
        s.y += y1;
        s.z += y2;
        s.w += y3;
      }
    }
    if (lane < kWaves) smem[lane] = s;
  }
  __syncthreads();
  const int4 prefix = w > 0 ? smem[w - 1] : make_int4(0, 0, 0, 0);
  *total = smem[kWaves - 1];
  __syncthreads();                               // smem may be reused after this
  return make_int4(prefix.x + x.x - v.x, prefix.y + x.y - v.y, prefix.z + x.z - v.z, prefix.w + x.w - v.w);
}

}  // namespace

// Per-expert prefix sums kept in LDS while the tile tables are written: slots, block_m tiles, GEMM
// tiles of the first and of the second class (see publish_tables) and payload bit offsets, each
// with its total in entry E.
struct TableSmem {
  int off[kMaxExperts + 1], toff[kMaxExperts + 1], goff[kMaxExperts + 1], loff[kMaxExperts + 1], boff[kMaxExperts + 1];
};

// The expert whose range [tab[e], tab[e + 1]) holds i, for 0 <= i < tab[E]: the last e with
// tab[e] <= i (empty experts before it share its start and come earlier).
__device__ __forceinline__ int owner_of(const int* tab, int E, int i) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tab[mid] <= i) lo = mid;
    else hi = mid;
  }
  return lo;
}

// Expert totals given, one expert per thread: offsets, tile tables, expert table, scalars. Every
// thread of the workgroup calls it (it holds workgroup barriers); returns this thread's expert
// offset (0 for threads past E). With COOP the tile tables are written by all threads, one tile each
// in turn (large batches, where one expert may hold hundreds of tiles); otherwise each expert's
// thread writes its own few tiles.
// GEMM tiles of 128 rows come in two classes: those of more than 64 rows (the GEMM computes all
// eight 16-row groups) and those of at most 64 rows (four groups, half the work). The list holds
// the first class, then the second, each in expert order: a launch deals its units in list order,
// so its last round, which runs on a partly idle chip, takes the short units.
template <bool COOP>
__device__ int publish_tables(const RouteMapArgs& a, int total_e, int bad, int4* scan_smem, TableSmem& tb) {
  const int tid = threadIdx.x, E = a.num_experts;
  const bool own = tid < E;                      // E <= 512 < 1024: one expert per thread
  const int bits_e = own ? static_cast<int>((a.packed_bits[tid >> 3] >> (4 * (tid & 7))) & 15u) : 0;
  const int tiles_e = own ? (total_e + a.block_m - 1) / a.block_m : 0;
  const int gtiles_e = own ? (total_e + a.gemm_rows - 1) / a.gemm_rows : 0;
  const int rem_e = total_e % a.gemm_rows;
  const int short_e = own && a.gemm_rows == 128 && rem_e > 0 && rem_e <= 64 ? 1 : 0;   // second-class tiles
  const int long_e = gtiles_e - short_e;                                                // first-class tiles
  // the payload bit offsets (< 2^13: widths <= 6, E <= 512) share a scan lane with the short tiles
  int4 totals;
  const int4 offs = block_exclusive_scan4(make_int4(own ? total_e : 0, tiles_e, long_e, bits_e | (short_e << 16)),
                                          scan_smem, &totals);
  const int off_e = offs.x;
  const int boff_e = offs.w & 0xffff, soff_e = offs.w >> 16;
  const int nlong = totals.z, nbits = totals.w & 0xffff, nshort = totals.w >> 16;
  if (own) {
    a.counts[tid] = total_e;
    a.offsets[tid] = off_e;
    ExpertInfo info;
    info.word_offset = static_cast<long long>(boff_e) * a.words_per_bit;
    info.bits = bits_e;
    info.pad = 0;
    a.einfo[tid] = info;
    if constexpr (COOP) {
      tb.off[tid] = off_e;
      tb.toff[tid] = offs.y;
      tb.goff[tid] = offs.z;
      tb.loff[tid] = soff_e;
      tb.boff[tid] = boff_e;
    } else {
      for (int t = 0; t < tiles_e; ++t) {
        a.tile_expert[offs.y + t] = tid;
        a.tile_row0[offs.y + t] = off_e + t * a.block_m;
        a.tile_rows[offs.y + t] = min(a.block_m, total_e - t * a.block_m);
      }
      for (int t = 0; t < gtiles_e; ++t) {
        int4 g;
        g.x = tid | (bits_e << 24);
        g.y = off_e + t * a.gemm_rows;
        g.z = min(a.gemm_rows, total_e - t * a.gemm_rows);
        g.w = static_cast<int>(info.word_offset >> 8);   // expert regions start on 256-word multiples
        a.gtiles[t < long_e ? offs.z + t : nlong + soff_e] = g;
      }
    }
  }
  if (tid == 0) {
    if constexpr (COOP) {
      tb.off[E] = totals.x;
      tb.toff[E] = totals.y;
      tb.goff[E] = nlong;
      tb.loff[E] = nshort;
      tb.boff[E] = nbits;
    }
    a.offsets[E] = totals.x;
    *a.num_tiles = totals.y;
    *a.num_gtiles = nlong + nshort;
    a.splits[0] = a.nsplit[0];
    a.splits[1] = a.nsplit[1];
    if (a.half) {
      a.half[0] = a.nhalf[0];
      a.half[1] = a.nhalf[1];
    }
    *a.status = bad;
  }
  // slots past the filled ones (dropped routes leave them empty) read as expert -1
  for (int q = totals.x + tid; q < a.routes; q += blockDim.x) a.slot_expert[q] = -1;
  if constexpr (!COOP) return off_e;
  __syncthreads();
  for (int i = tid; i < totals.y; i += blockDim.x) {
    const int e = owner_of(tb.toff, E, i);
    const int t = i - tb.toff[e];
    const int cnt_e = tb.off[e + 1] - tb.off[e];
    a.tile_expert[i] = e;
    a.tile_row0[i] = tb.off[e] + t * a.block_m;
    a.tile_rows[i] = min(a.block_m, cnt_e - t * a.block_m);
  }
  for (int i = tid; i < nlong + nshort; i += blockDim.x) {
    // first class: tile i - goff[e] of its expert; second class: the expert's last tile
    const int e = i < nlong ? owner_of(tb.goff, E, i) : owner_of(tb.loff, E, i - nlong);
    const int t = i < nlong ? i - tb.goff[e] : tb.goff[e + 1] - tb.goff[e];
    const int cnt_e = tb.off[e + 1] - tb.off[e];
    const int b = tb.boff[e + 1] - tb.boff[e];
    int4 g;
    g.x = e | (b << 24);
    g.y = tb.off[e] + t * a.gemm_rows;
    g.z = min(a.gemm_rows, cnt_e - t * a.gemm_rows);
    g.w = static_cast<int>((static_cast<long long>(tb.boff[e]) * a.words_per_bit) >> 8);   // expert regions start on 256-word multiples
    a.gtiles[i] = g;
  }
  return off_e;
}

// All routes in one workgroup (workgroup 0): each wave takes a contiguous segment of R/16 routes.
// Workgroups 1.. rotate the input rows, 16 items each (ROT = false: none).
template <bool ROT, int EPL, bool MX>
__global__ __launch_bounds__(1024) void k_route_map(RouteMapArgs a, RotateArgs ra) {
  if constexpr (ROT) {
    if (blockIdx.x > 0) {
      rotate_routes<EPL, MX>(ra, (blockIdx.x - 1) * kWaves);
      return;
    }
  }
  __shared__ int cnt[kWaves * kMaxExperts];   // per wave, per expert: count, then running slot
  __shared__ int4 scan_smem[kWaves];
  __shared__ int bad_w[kWaves];
  __shared__ TableSmem tb;
  const int tid = threadIdx.x, w = tid >> 6;
  const int E = a.num_experts, R = a.routes;
  for (int i = tid; i < kWaves * E; i += 1024) cnt[i] = 0;
  if (tid < kWaves) bad_w[tid] = 0;
  __syncthreads();

  const int nbits = 32 - __clz(E);              // keys 0..E (E marks an invalid id)
  const int seg = (R + kWaves - 1) / kWaves;
  const int beg = w * seg, end = min(R, beg + seg);
  int kept[kKeep];
  count_segment(a, beg, end, nbits, cnt + w * E, bad_w + w, kept);
  __syncthreads();

  int total_e = 0, bad = 0;
  if (tid < E)
    for (int ww = 0; ww < kWaves; ++ww) total_e += cnt[ww * E + tid];
  if (tid == 0)
    for (int ww = 0; ww < kWaves; ++ww) bad += bad_w[ww];
  const int off_e = publish_tables<false>(a, total_e, bad, scan_smem, tb);
  if (tid < E) {                                 // per-wave starting slots
    int acc = off_e;
    for (int ww = 0; ww < kWaves; ++ww) {
      const int c = cnt[ww * E + tid];
      cnt[ww * E + tid] = acc;
      acc += c;
    }
  }
  __syncthreads();
  place_segment(a, beg, end, nbits, cnt + w * E, kept);
}

// Large batches, launch 1 of 2: workgroup g counts routes [g * kRouteChunk, (g + 1) * kRouteChunk)
// per expert into wg_counts[g][0..E) and its invalid ids into wg_counts[g][E]. Workgroups past the
// counting ones rotate the input rows, 16 items each (the first third of the rotation groups; the
// placement launch takes the rest).
template <bool ROT, int EPL, bool MX>
__global__ __launch_bounds__(1024) void k_route_count(RouteMapArgs a, RotateArgs ra, int count_groups) {
  if constexpr (ROT) {
    if (static_cast<int>(blockIdx.x) >= count_groups) {
      rotate_routes<EPL, MX>(ra, (blockIdx.x - count_groups) * kWaves);
      return;
    }
  }
  __shared__ int cnt[kWaves * kMaxExperts];
  __shared__ int bad_w[kWaves];
  const int tid = threadIdx.x, w = tid >> 6;
  const int E = a.num_experts, R = a.routes;
  for (int i = tid; i < kWaves * E; i += 1024) cnt[i] = 0;
  if (tid < kWaves) bad_w[tid] = 0;
  __syncthreads();
  const int nbits = 32 - __clz(E);
  const int beg = min(R, static_cast<int>(blockIdx.x) * kRouteChunk + w * 64), end = min(R, beg + 64);
  int kept[kKeep];
  count_segment(a, beg, end, nbits, cnt + w * E, bad_w + w, kept);
  __syncthreads();
  int32_t* out = a.wg_counts + static_cast<size_t>(blockIdx.x) * (E + 1);
  if (tid < E) {
    int c = 0;
    for (int ww = 0; ww < kWaves; ++ww) c += cnt[ww * E + tid];
    out[tid] = c;
  }
  if (tid == 0) {
    int b = 0;
    for (int ww = 0; ww < kWaves; ++ww) b += bad_w[ww];
    out[E] = b;
  }
}

// Large batches, launch 2 of 2: every workgroup derives the expert offsets from all workgroups'
// counts, recounts its own chunk per wave and places it; workgroup 0 also writes the tables. The
// slot of a route is its expert's offset + the routes of that expert in earlier workgroups + in
// earlier waves of this workgroup + earlier lanes of its chunk: stable token-major order.
// Workgroups past the placing ones rotate the input rows from rotation group rot_first on (the
// rotation is split between the two launches, so each overlaps its own share).
template <bool ROT, int EPL, bool MX>
__global__ __launch_bounds__(1024) void k_route_place(RouteMapArgs a, RotateArgs ra, int place_groups, int rot_first) {
  if constexpr (ROT) {
    if (static_cast<int>(blockIdx.x) >= place_groups) {
      rotate_routes<EPL, MX>(ra, (static_cast<int>(blockIdx.x) - place_groups + rot_first) * kWaves);
      return;
    }
  }
  __shared__ int cnt[kWaves * kMaxExperts];
  __shared__ int4 scan_smem[kWaves];
  __shared__ int bad_w[kWaves];
  __shared__ TableSmem tb;
  __shared__ int bad_all;
  const int tid = threadIdx.x, w = tid >> 6;
  const int E = a.num_experts, R = a.routes;
  const int G = place_groups, g = blockIdx.x;
  for (int i = tid; i < kWaves * E; i += 1024) cnt[i] = 0;
  if (tid < kWaves) bad_w[tid] = 0;
  __syncthreads();
  const int nbits = 32 - __clz(E);
  const int beg = min(R, g * kRouteChunk + w * 64), end = min(R, beg + 64);
  int kept[kKeep];
  count_segment(a, beg, end, nbits, cnt + w * E, bad_w + w, kept);

  // column tid (an expert, or E: the invalid ids) of all workgroups' counts, eight loads in flight
  int total_e = 0, before_e = 0, bad = 0;
  if (tid <= E) {
    const int32_t* col = a.wg_counts + tid;
    const size_t pitch = static_cast<size_t>(E + 1);
    int gg = 0;
    for (; gg + 8 <= G; gg += 8) {
      int c[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) c[u] = col[(gg + u) * pitch];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        total_e += c[u];
        before_e += gg + u < g ? c[u] : 0;
      }
    }
    for (; gg < G; ++gg) {
      const int c = col[gg * pitch];
      total_e += c;
      before_e += gg < g ? c : 0;
    }
    if (tid == E) {
      bad = total_e;
      total_e = 0;
      before_e = 0;
    }
  }
  if (tid == E) bad_all = bad;
  __syncthreads();                               // cnt complete
  int off_e;
  if (g == 0) {
    off_e = publish_tables<true>(a, total_e, bad_all, scan_smem, tb);
  } else {
    int4 totals;
    off_e = block_exclusive_scan4(make_int4(tid < E ? total_e : 0, 0, 0, 0), scan_smem, &totals).x;
  }
  if (tid < E) {
    int acc = off_e + before_e;
    for (int ww = 0; ww < kWaves; ++ww) {
      const int c = cnt[ww * E + tid];
      cnt[ww * E + tid] = acc;
      acc += c;
    }
  }
  __syncthreads();
  place_segment(a, beg, end, nbits, cnt + w * E, kept);
}

void launch_route_map(const RouteMapArgs& a, const RotateArgs* ra, bool mx, hipStream_t s) {
  // rotation workgroups: one wavefront per route or per (route, row segment)
  const long long rot_items = ra ? static_cast<long long>(ra->routes) * rotate_items_per_route(*ra) : 0;
  const unsigned rot_groups = static_cast<unsigned>((rot_items + kWaves - 1) / kWaves);
  const RotateArgs none{};
  const RotateArgs& r = ra ? *ra : none;
  auto go = [&](auto rot, auto epl, auto m) {
    constexpr bool ROT = decltype(rot)::value;
    constexpr int E = decltype(epl)::value;
    constexpr bool M = decltype(m)::value;
    if (a.routes <= kRouteSingleMax) {
      hipLaunchKernelGGL((k_route_map<ROT, E, M>), dim3(1 + rot_groups), dim3(1024), 0, s, a, r);
      return;
    }
    const int groups = (a.routes + kRouteChunk - 1) / kRouteChunk;
    // a third of the rotation with the counting, two thirds with the placement (measured best of
    // 1/3, 1/2, 2/3: prefill route stage 23.0 -> 19.5 us against all of it in the first launch)
    const unsigned rot_count = rot_groups / 3, rot_place = rot_groups - rot_count;
    hipLaunchKernelGGL((k_route_count<ROT, E, M>), dim3(groups + rot_count), dim3(1024), 0, s, a, r, groups);
    hipLaunchKernelGGL((k_route_place<ROT, E, M>), dim3(groups + rot_place), dim3(1024), 0, s, a, r, groups,
                       static_cast<int>(rot_count));
  };
  if (!ra) {
    go(std::false_type{}, std::integral_constant<int, 1>{}, std::false_type{});
    return;
  }
  dispatch_epl(ra->rot, [&](auto epl) {
    if (mx) go(std::true_type{}, epl, std::true_type{});
    else go(std::true_type{}, epl, std::false_type{});
  });
}

}  // namespace tmoe
