// tmoe_routemap.hpp -- per-wave pieces of the stable token-major route map, shared by the route-map
// launches and the single-launch small-batch arm (which builds the map in each workgroup's LDS).
//
// Same-expert lanes of a 64-route chunk are found with one ballot per key bit (a "multi-split",
// after the GPU multisplit primitive of Ashkiani et al., "GPU Multisplit", PPoPP 2016): the AND of
// the ballots that agree with a lane's key bits is exactly the set of lanes holding the same key,
// so the rank of a lane among equal keys is a popcount.
#pragma once
#include "tmoe_device.hpp"
#include "tmoe_internal.hpp"

namespace tmoe {

__device__ __forceinline__ long long load_id(const void* ids, int ids64, int r) {
  return ids64 ? static_cast<const long long*>(ids)[r] : static_cast<long long>(static_cast<const int*>(ids)[r]);
}

// Lanes of the current chunk that hold the same key as this lane (among `active` lanes).
__device__ __forceinline__ unsigned long long same_key_mask(int key, int nbits, unsigned long long active) {
  unsigned long long m = active;
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (key >> b) & 1;
    const unsigned long long bal = __ballot(bit);
    m &= bit ? bal : ~bal;
  }
  return m;
}


// Counts of one wave's segment [beg, end) per expert into cnt[w * E + key] (invalid ids into
// *bad). The keys of the first kKeep 64-route chunks are returned in kept[] for the placement pass.
constexpr int kKeep = 4;

__device__ __forceinline__ void count_segment(const RouteMapArgs& a, int beg, int end, int nbits, int* cnt_w,
                                              int* bad, int (&kept)[kKeep]) {
  const int lane = threadIdx.x & 63, E = a.num_experts;
  int ci = 0;
  for (int base = beg; base < end; base += 64, ++ci) {
    const int r = base + lane;
    const bool act = r < end;
    const long long id = act ? load_id(a.ids, a.ids64, r) : -1;
    const bool valid = act && id >= 0 && id < E;
    const int key = valid ? static_cast<int>(id) : E;
#pragma unroll
    for (int k = 0; k < kKeep; ++k)
      if (ci == k) kept[k] = key;
    const unsigned long long active = __ballot(act);
    const unsigned long long m = same_key_mask(key, nbits, active);
    const bool leader = act && ((m >> lane) == 1ull);        // highest lane of its key group
    if (leader) {
      const int c = __popcll(m);
      if (valid) cnt_w[key] += c;
      else *bad += c;
    }
  }
}

// Stable placement of one wave's segment: cnt_w[e] holds the wave's next slot for expert e.
__device__ __forceinline__ void place_segment(const RouteMapArgs& a, int beg, int end, int nbits, int* cnt_w,
                                              const int (&kept)[kKeep]) {
  const int lane = threadIdx.x & 63, E = a.num_experts;
  const unsigned long long lt = (1ull << lane) - 1ull;
  int ci = 0;
  for (int base = beg; base < end; base += 64, ++ci) {
    const int r = base + lane;
    const bool act = r < end;
    int key = E;
    if (ci < kKeep) {
#pragma unroll
      for (int k = 0; k < kKeep; ++k)
        if (ci == k) key = kept[k];
    } else {
      const long long id = act ? load_id(a.ids, a.ids64, r) : -1;
      key = act && id >= 0 && id < E ? static_cast<int>(id) : E;
    }
    const bool valid = act && key < E;
    const unsigned long long active = __ballot(act);
    const unsigned long long m = same_key_mask(key, nbits, active);
    if (valid) {
      const int pos = cnt_w[key] + __popcll(m & lt);
      a.sorted_routes[pos] = r;
      a.slot_expert[pos] = key;
      a.route_slot[r] = pos;
    } else if (act) {
      a.route_slot[r] = -1;
    }
    // every lane of the wave has read its running slot above (LDS accesses of one wave complete
    // in order), so the group leader may now advance it
    if (valid && ((m >> lane) == 1ull)) cnt_w[key] += __popcll(m);
  }
}

}  // namespace tmoe
