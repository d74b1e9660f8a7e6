// tmoe_host.cpp -- the C ABI: plan validation, scratch layout and the launch sequence.
//
// Every argument is checked before the first launch, so a rejected call leaves the caller's
// output and scratch untouched (the Summary of "serve canonical Fruit QSRT atoms" rejects bad
// layouts and route maps before any work). Plans are host-only; the library allocates
// nothing: per-expert payload offsets travel as packed launch arguments and are expanded into the
// caller's scratch by the route-map kernel, so a forward call can be captured into a hipGraph.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include <hip/hip_runtime.h>

#include "tmoe.h"
#include "tmoe_device.hpp"
#include "tmoe_internal.hpp"

using namespace tmoe;

namespace {

constexpr int kMaxExperts = 512;
constexpr int kMaxTopK = 32;
constexpr int kMaxDim = 4096;
constexpr long long kMaxRoutes = 1LL << 24;
constexpr size_t kAlign = 256;
constexpr int kGemmWaveCap = 5120;     // 256 CUs x 4 SIMDs x 5 wavefronts
constexpr int kGemmGroupCap = 1 << 20; // workgroups of a 128-row tile launch (one unit each)

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
bool is_pow2(int n) { return n > 0 && (n & (n - 1)) == 0; }

RowRot make_rot(int n, int identity) {
  RowRot r;
  r.n = n;
  r.pow2 = is_pow2(n) ? 1 : 0;
  r.nblk128 = r.pow2 ? 0 : n / 128;
  r.tail64 = r.pow2 ? 0 : ((n % 128) ? 1 : 0);
  r.identity = identity;
  return r;
}

// K-split count: more splits for fewer routes so small batches still fill the chip; must divide
// the K steps so every split has the same depth.
int choose_splits(long long routes, int ksteps) {
  int target = routes <= 32 ? 8 : routes <= 128 ? 4 : routes <= 512 ? 2 : 1;
  // small batches with a deep K (long rows): also keep a unit at about ten K steps, so every SIMD
  // still gets several short units (wide geometry FC1: 61 -> 44 us at T = 16)
  if (routes <= 512)
    while (target < 8 && ksteps > 10 * target) target *= 2;
  for (int s = target; s > 1; s >>= 1)
    if (ksteps % s == 0) return s;
  return 1;
}

// Extra K splits for wavefront tiles of batches past 512 routes: doubled while the doubled units
// still fit the persistent wavefronts, each unit keeping at least 8 K steps (more splits would only
// add fp32 planes for the next launch to sum: wide T = 512 FC1 in 2 splits 70.7 us, in 4 72.5 us).
int fill_splits(long long units_per_split, int ksteps) {
  int s = 1;
  while (s < 8 && units_per_split * s * 2 <= kGemmWaveCap && ksteps % (2 * s) == 0 && ksteps / (2 * s) >= 8) s *= 2;
  return s;
}

// GEMM tile shape code: 1, 2, 4 = 16-row groups per wavefront tile (64 columns); 8, 16 = workgroup
// tiles of 128 rows by 128 or 256 columns for large batches (fp16 path; `big_cols` is the widest
// workgroup tile both output widths are multiples of, or 0). Batches of at most 64 rows per expert
// on average take 64-row wavefront tiles: a 128-row workgroup tile would compute half its rows only,
// and the wavefront kernel's K splits keep the chip filled (wide geometry at T = 512: FC1 93 -> 73 us).
int choose_mg(long long routes, int experts, int big_cols) {
  if (routes <= 2LL * experts) return 1;
  if (routes <= 8LL * experts) return 2;
  if (routes <= 64LL * experts) return 4;
  if (big_cols == 256) return 16;
  if (big_cols == 128) return 8;
  return 4;
}

int tile_rows(int mg) { return mg >= 8 ? 128 : 16 * mg; }

// Row pitch (elements) of the fp16 GEMM inputs A1 and b. A row of a power-of-two multiple of 512 bytes
// would place the 16 rows one MFMA operand load touches on a couple of memory channels only; one
// extra 256-byte block spreads them.
int fp16_pitch(int k) { return (2 * k) % 512 == 0 ? k + 128 : k; }

struct Layout {
  size_t einfo, counts, offsets, sorted, slot_e, slot, tile_e, tile_r0, tile_rows, scalars, gtiles, wgc;
  size_t a1, z, b, v, total;
};

}  // namespace

struct tmoe_plan_s {
  int H, I, E, K, max_tokens, rotation, ids64, block_m, smallm_max_tokens, fc2_reduce;
  std::vector<uint8_t> bits;
  std::vector<long long> offsets;   // word offset per expert, [E+1]
  uint32_t packed_bits[64];      // 4 bits per expert: its width
  long long routes_max;
  long long zrows, vrows;           // rows of the FC1 / FC2 output area (split planes included)
  int max_tiles, max_gtiles;
  bool fp8_ok;
  int uniform_bits;                 // the width shared by all experts; 0 (mixed 2-4) or kMixedWide
  int max_bits;
  Layout lay;
};

namespace {

long long max_split_rows(long long rmax, int ksteps_a, int ksteps_b) {
  long long best = rmax;
  const long long pts[4] = {std::min(rmax, 32LL), std::min(rmax, 128LL), std::min(rmax, 512LL), rmax};
  for (long long r : pts)
    for (int ks : {ksteps_a, ksteps_b}) best = std::max(best, r * choose_splits(r, ks));
  return best;
}

void build_layout(tmoe_plan_s* p) {
  const long long R = p->routes_max;
  Layout& L = p->lay;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes); return o; };
  L.einfo = take(sizeof(ExpertInfo) * p->E);
  L.counts = take(4ull * p->E);
  L.offsets = take(4ull * (p->E + 1));
  L.sorted = take(4ull * R);
  L.slot_e = take(4ull * R);
  L.slot = take(4ull * R);
  L.tile_e = take(4ull * p->max_tiles);
  L.tile_r0 = take(4ull * p->max_tiles);
  L.tile_rows = take(4ull * p->max_tiles);
  L.scalars = take(32);                               // num_tiles, status, num_gtiles, splits[2], arm status, half[2]
  L.gtiles = take(16ull * p->max_gtiles);
  L.wgc = take(4ull * ((R + kRouteChunk - 1) / kRouteChunk) * (p->E + 1));   // per-workgroup route counts
  L.a1 = take(2ull * R * fp16_pitch(p->H));           // fp16 (padded rows), or E4M3 + E8M0 planes
  // the extra splits of 64-row wavefront tiles, sized at the largest batch (smaller batches take no
  // more splits than fit: the GEMM shape clamps them)
  const long long gt64 = std::min<long long>(R, p->E + R / 64 + 1);
  const long long zrows = std::max(max_split_rows(R, p->H / 32, p->H / 128 > 0 ? p->H / 128 : 1),
                                   R * fill_splits(gt64 * (2 * p->I / 64), p->H / 32));
  L.z = take(4ull * zrows * 2 * p->I);
  L.b = take(2ull * R * fp16_pitch(p->I));
  const long long vrows = std::max(max_split_rows(R, p->I / 32, p->I / 128 > 0 ? p->I / 128 : 1),
                                   R * fill_splits(gt64 * (p->H / 64), p->I / 32));
  L.v = take(4ull * vrows * p->H);
  p->zrows = zrows;
  p->vrows = vrows;
  L.total = off;
}

template <class T>
T* at(void* base, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(base) + off); }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

tmoe_status check_scratch(const tmoe_plan_s* p, void* scratch, size_t bytes) {
  if (!scratch) return TMOE_ERR_SCRATCH;
  if (!aligned(scratch, 16)) return TMOE_ERR_SCRATCH;
  if (bytes < p->lay.total) return TMOE_ERR_SCRATCH;
  return TMOE_OK;
}

tmoe_route_map make_view(const tmoe_plan_s* p, void* scratch) {
  tmoe_route_map v;
  v.counts = at<int32_t>(scratch, p->lay.counts);
  v.offsets = at<int32_t>(scratch, p->lay.offsets);
  v.sorted_routes = at<int32_t>(scratch, p->lay.sorted);
  v.route_slot = at<int32_t>(scratch, p->lay.slot);
  v.tile_expert = at<int32_t>(scratch, p->lay.tile_e);
  v.tile_row0 = at<int32_t>(scratch, p->lay.tile_r0);
  v.tile_rows = at<int32_t>(scratch, p->lay.tile_rows);
  v.num_tiles = at<int32_t>(scratch, p->lay.scalars);
  v.status = at<int32_t>(scratch, p->lay.scalars) + 1;
  v.max_tiles = p->max_tiles;
  v.block_m = p->block_m;
  return v;
}

struct GemmShape {          // launch shape of one grouped GEMM
  int ng, ksteps, most, waves;
};

// Column groups, K steps, split bound and launch size of FC1 (fc = 1) or FC2 (fc = 2). For 16- to
// 64-row tiles a unit is one wavefront's 64 columns and `waves` counts persistent wavefronts; for
// 128-row tiles a unit is one workgroup's 128 or 256 columns and `waves` counts workgroups.
int fc2_mg(const tmoe_plan_s* p, int mg);

GemmShape gemm_shape(const tmoe_plan_s* p, long long R, int mg_in, bool fp8, int fc) {
  GemmShape g;
  const int mg = fc == 2 ? fc2_mg(p, mg_in) : mg_in;
  const int K = fc == 1 ? p->H : p->I;
  const int N = fc == 1 ? 2 * p->I : p->H;
  const bool big = mg >= 8;
  const int gemm_rows = tile_rows(mg);
  g.ng = N / (mg == 16 ? 256 : big ? 128 : 64);
  g.ksteps = K / (fp8 ? 128 : 32);
  g.most = choose_splits(R, g.ksteps);
  const long long gt_ub = std::min<long long>(R, p->E + R / gemm_rows + 1);
  if (!big && R > 512) {
    g.most = std::max(g.most, fill_splits(gt_ub * g.ng, g.ksteps));
    const long long cap = fc == 1 ? p->zrows : p->vrows;
    while (g.most > 1 && R * g.most > cap) g.most /= 2;
  }
  g.waves = static_cast<int>(std::min<long long>(big ? kGemmGroupCap : kGemmWaveCap, gt_ub * g.ng * g.most));
  if (big) {                                    // a whole number of 8-tile rounds of units
    const int per = 8 * g.ng * g.most;
    g.waves = (g.waves + per - 1) / per * per;
  }
  return g;
}

// fp16 GEMMs with one K split finish their sums in one launch: they apply the channel scale in the
// epilogue and leave one fp16 plane, half the bytes of fp32 for the next launch to read. The opt-in
// atomic FC2 adds into y instead of leaving v.
void half_planes(bool fp8, const GemmShape (&sh)[2], bool atomic_fc2, bool (&half)[2]) {
  half[0] = !fp8 && sh[0].most == 1;
  half[1] = !fp8 && sh[1].most == 1 && !atomic_fc2;
}

// FC1's workgroup tile width for 128-row tiles (both GEMMs' widths must be multiples of 128, as
// they share the tile list), or 0.
int big_cols(const tmoe_plan_s* p, bool fp8) {
  if (fp8) return 0;                          // 128-row tiles: the fp16 GEMMs only
  if (p->H % 128 != 0 || (2 * p->I) % 128 != 0) return 0;
  return (2 * p->I) % 256 == 0 ? 256 : 128;
}

// FC2's tile shape code: its own workgroup tile width (H = 2560 with 2I = 640 takes 256 columns
// for FC2 and 128 for FC1).
int fc2_mg(const tmoe_plan_s* p, int mg) { return mg >= 8 ? (p->H % 256 == 0 ? 16 : 8) : mg; }

// With `rot` set, the same launch also writes the rotated input operand of every route. half[i]:
// GEMM i + 1 leaves one fp16 plane (published with the split counts).
void enqueue_route_map(const tmoe_plan_s* p, const void* ids, int T, int gemm_rows, const GemmShape (&sh)[2],
                       const bool (&half)[2], void* scratch, const RotateArgs* rot, bool fp8, hipStream_t st) {
  RouteMapArgs a;
  std::memset(&a, 0, sizeof(a));
  a.ids = ids;
  a.ids64 = p->ids64;
  a.routes = T * p->K;
  a.num_experts = p->E;
  a.block_m = p->block_m;
  a.gemm_rows = gemm_rows;
  a.words_per_bit = 3LL * p->H * p->I / 16;
  a.counts = at<int32_t>(scratch, p->lay.counts);
  a.offsets = at<int32_t>(scratch, p->lay.offsets);
  a.sorted_routes = at<int32_t>(scratch, p->lay.sorted);
  a.route_slot = at<int32_t>(scratch, p->lay.slot);
  a.tile_expert = at<int32_t>(scratch, p->lay.tile_e);
  a.tile_row0 = at<int32_t>(scratch, p->lay.tile_r0);
  a.tile_rows = at<int32_t>(scratch, p->lay.tile_rows);
  a.num_tiles = at<int32_t>(scratch, p->lay.scalars);
  a.status = at<int32_t>(scratch, p->lay.scalars) + 1;
  a.num_gtiles = at<int32_t>(scratch, p->lay.scalars) + 2;
  a.splits = at<int32_t>(scratch, p->lay.scalars) + 3;
  a.nsplit[0] = sh[0].most;
  a.nsplit[1] = sh[1].most;
  a.half = at<int32_t>(scratch, p->lay.scalars) + 6;
  a.nhalf[0] = half[0] ? 1 : 0;
  a.nhalf[1] = half[1] ? 1 : 0;
  a.slot_expert = at<int32_t>(scratch, p->lay.slot_e);
  a.wg_counts = at<int32_t>(scratch, p->lay.wgc);
  a.gtiles = at<int4>(scratch, p->lay.gtiles);
  a.einfo = at<ExpertInfo>(scratch, p->lay.einfo);
  std::memcpy(a.packed_bits, p->packed_bits, sizeof(a.packed_bits));
  launch_route_map(a, rot, fp8, st);
}

tmoe_status check_common(const tmoe_plan_s* p, const void* ids, int T, void* scratch, size_t bytes) {
  if (!p) return TMOE_ERR_INVALID_ARG;
  if (T < 0) return TMOE_ERR_INVALID_ARG;
  if (T > p->max_tokens) return TMOE_ERR_CAPACITY;
  if (T == 0) return TMOE_OK;
  if (!ids) return TMOE_ERR_INVALID_ARG;
  if (!aligned(ids, p->ids64 ? 8 : 4)) return TMOE_ERR_ALIGNMENT;
  return check_scratch(p, scratch, bytes);
}

// The FP32-atomic FC2 reduction: W4A16, widths 2-4, output rows of 512 or 1024 values (one
// workgroup of H/128 wavefronts owns whole rows); other plans keep the deterministic epilogue.
bool fc2_atomic_fits(const tmoe_plan_s* p, bool fp8) {
  return !fp8 && p->max_bits <= 4 && (p->H == 512 || p->H == 1024);
}

// The small-batch arm runs rows of 128 to 1024 values (2 to 16 per lane) or rows rotated in
// 128-blocks, and at most kArmMaxRoutes routes.
bool arm_rot_ok(int n) { return !is_pow2(n) || (n >= 128 && n <= 1024); }
bool arm_fits(const tmoe_plan_s* p, long long R) {
  return R <= kArmMaxRoutes && arm_rot_ok(p->H) && arm_rot_ok(p->I);
}

// The whole layer as one persistent launch (k_small_arm.hip); UNSUPPORTED if it cannot run here,
// and the caller then takes the five-launch path.
tmoe_status forward_arm(const tmoe_plan_s* p, const void* x, const void* ids, const float* w, int32_t T,
                        const tmoe_weights* wt, float* y, void* scratch, hipStream_t s, bool fp8) {
  ArmSlot* slot = nullptr;
  int groups = 0;
  if (!small_arm_prepare(scratch, p->uniform_bits, fp8, &slot, &groups)) return TMOE_ERR_UNSUPPORTED;
  const long long R = static_cast<long long>(T) * p->K;
  ArmArgs a;
  std::memset(&a, 0, sizeof(a));
  a.x = static_cast<const uint16_t*>(x);
  a.ids = ids;
  a.ids64 = p->ids64;
  a.w = w;
  a.payload = wt->payload;
  a.scale1 = wt->scale1;
  a.scale2 = wt->scale2;
  a.su1 = wt->su1;
  a.sv1 = wt->sv1;
  a.su2 = wt->su2;
  a.sv2 = wt->sv2;
  a.y = y;
  a.T = T;
  a.H = p->H;
  a.I = p->I;
  a.E = p->E;
  a.K = p->K;
  a.R = static_cast<int>(R);
  a.rot_h = make_rot(p->H, p->rotation == TMOE_ROT_IDENTITY);
  a.rot_i = make_rot(p->I, p->rotation == TMOE_ROT_IDENTITY);
  a.words_per_bit = 3LL * p->H * p->I / 16;
  a.fc2_words_per_bit = 2LL * p->H * p->I / 16;
  const int kstep = fp8 ? 128 : 32;
  a.s1 = choose_splits(R, p->H / kstep);
  a.s2 = choose_splits(R, p->I / kstep);
  a.a1 = at<uint8_t>(scratch, p->lay.a1);
  a.a1s = a.a1 + static_cast<size_t>(R) * p->H;
  a.lda = fp16_pitch(p->H);
  a.z = at<float>(scratch, p->lay.z);
  a.b = at<uint8_t>(scratch, p->lay.b);
  a.bs = a.b + static_cast<size_t>(R) * p->I;
  a.ldb = fp16_pitch(p->I);
  a.v = at<float>(scratch, p->lay.v);
  a.status = at<int32_t>(scratch, p->lay.scalars) + 1;
  a.arm_status = at<int32_t>(scratch, p->lay.scalars) + 5;
  a.slot = slot;
  std::memcpy(a.packed_bits, p->packed_bits, sizeof(a.packed_bits));
  // enough wavefronts for the widest step, and no more than are resident at once
  const long long tiles = std::min<long long>(R, p->E + R / 16 + 1);
  const long long units = std::max(tiles * (2 * p->I / 64) * a.s1, tiles * (p->H / 64) * a.s2);
  const long long items = std::max(units, R + T);
  const int need = static_cast<int>(std::min<long long>((items + 3) / 4, 1 << 20));
  (void)hipGetLastError();
  launch_small_arm(a, p->uniform_bits, fp8, std::max(1, std::min(groups, need)), s);
  return hipGetLastError() == hipSuccess ? TMOE_OK : TMOE_ERR_HIP;
}

// Stages: 0 route map with the input rotation, 1 FC1, 2 activation, 3 FC2, 4 combine.
tmoe_status forward(tmoe_plan_t p, const void* x, const void* ids, const float* w, int32_t T,
                    const tmoe_weights* wt, float* y, void* scratch, size_t bytes, void* stream, bool fp8,
                    int first = 0, int last = 4, bool staged = false) {
  tmoe_status st = check_common(p, ids, T, scratch, bytes);
  if (st != TMOE_OK) return st;
  if (fp8 && !p->fp8_ok) return TMOE_ERR_UNSUPPORTED;
  if (T == 0) return TMOE_OK;
  if (!x || !w || !wt || !y) return TMOE_ERR_INVALID_ARG;
  if (!wt->payload || !wt->scale1 || !wt->scale2 || !wt->su1 || !wt->sv1 || !wt->su2 || !wt->sv2)
    return TMOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(w, 4) || !aligned(wt->payload, 16) ||
      !aligned(wt->scale1, 2) || !aligned(wt->scale2, 2) || !aligned(wt->su1, 2) || !aligned(wt->sv1, 2) ||
      !aligned(wt->su2, 2) || !aligned(wt->sv2, 2))
    return TMOE_ERR_ALIGNMENT;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const long long R = static_cast<long long>(T) * p->K;
  if (!staged && T <= p->smallm_max_tokens && arm_fits(p, R)) {
    const tmoe_status st_arm = forward_arm(p, x, ids, w, T, wt, y, scratch, s, fp8);
    if (st_arm != TMOE_ERR_UNSUPPORTED) return st_arm;
  }
  const int mg = choose_mg(R, p->E, big_cols(p, fp8));
  const int gemm_rows = tile_rows(mg);
  const GemmShape sh[2] = {gemm_shape(p, R, mg, fp8, 1), gemm_shape(p, R, mg, fp8, 2)};
  // the FP32-atomic FC2 reduction adds into y, which the activation launch zeroes beforehand
  const bool atomic_fc2 = p->fc2_reduce == TMOE_FC2_ATOMIC && fc2_atomic_fits(p, fp8);
  bool half[2];
  half_planes(fp8, sh, atomic_fc2, half);

  const int32_t* sorted = at<int32_t>(scratch, p->lay.sorted);
  const int32_t* slot_expert = at<int32_t>(scratch, p->lay.slot_e);
  uint8_t* a1 = at<uint8_t>(scratch, p->lay.a1);
  uint8_t* a1s = a1 + static_cast<size_t>(R) * p->H;
  uint8_t* bq = at<uint8_t>(scratch, p->lay.b);
  uint8_t* bs = bq + static_cast<size_t>(R) * p->I;
  float* z = at<float>(scratch, p->lay.z);
  float* v = at<float>(scratch, p->lay.v);

  RotateArgs ra;
  ra.x = static_cast<const uint16_t*>(x);
  ra.ids = ids;
  ra.ids64 = p->ids64;
  ra.top_k = p->K;
  ra.num_experts = p->E;
  ra.su1 = wt->su1;
  ra.rot = make_rot(p->H, p->rotation == TMOE_ROT_IDENTITY);
  ra.a1 = a1;
  ra.a1_scale = a1s;
  ra.lda = fp16_pitch(p->H);
  ra.routes = static_cast<int>(R);
  // rows of a non-power-of-two length split into their 128-blocks while the routes alone would not
  // fill the chip; with many routes one wavefront per route keeps its loads better in flight
  ra.split_segments = R < 2048 ? 1 : 0;

  (void)hipGetLastError();   // clear a stale error so the check below reports this call only
  auto on = [&](int stage) { return first <= stage && stage <= last; };
  if (on(0)) enqueue_route_map(p, ids, T, gemm_rows, sh, half, scratch, &ra, fp8, s);

  GemmArgs g1;
  g1.payload = wt->payload;
  g1.einfo = at<ExpertInfo>(scratch, p->lay.einfo);
  g1.fc2_words_per_bit = 0;
  g1.a = a1;
  g1.a_scale = a1s;
  g1.out = z;
  g1.gtiles = at<int4>(scratch, p->lay.gtiles);
  g1.num_gtiles = at<int32_t>(scratch, p->lay.scalars) + 2;
  g1.max_gtiles = p->max_gtiles;
  g1.K = p->H;
  g1.N = 2 * p->I;
  g1.lda = fp16_pitch(p->H);
  g1.nsplit = sh[0].most;
  g1.routes = static_cast<int>(R);
  g1.arow = sorted;
  g1.out16 = half[0] ? reinterpret_cast<uint16_t*>(z) : nullptr;
  g1.oscale = wt->scale1;
  const int waves1 = sh[0].waves;
  if (on(1)) {
    if (fp8) launch_gemm_f8(g1, 1, p->uniform_bits, mg, waves1, s);
    else launch_gemm_f16(g1, 1, p->uniform_bits, mg, waves1, s);
  }

  ActArgs aa;
  aa.z = z;
  aa.z16 = g1.out16;
  aa.nsplit = sh[0].most;
  aa.slot_expert = slot_expert;
  aa.scale1 = wt->scale1;
  aa.sv1 = wt->sv1;
  aa.su2 = wt->su2;
  aa.rot = make_rot(p->I, p->rotation == TMOE_ROT_IDENTITY);
  aa.b = bq;
  aa.b_scale = bs;
  aa.ldb = fp16_pitch(p->I);
  aa.routes = static_cast<int>(R);
  aa.y_zero = atomic_fc2 ? y : nullptr;
  aa.y_count = atomic_fc2 ? static_cast<long long>(T) * p->H : 0;
  aa.act_blocks = 0;
  if (on(2)) launch_act(aa, fp8, s);

  GemmArgs g2 = g1;
  g2.fc2_words_per_bit = 2LL * p->H * p->I / 16;
  g2.a = bq;
  g2.a_scale = bs;
  g2.out = v;
  g2.K = p->I;
  g2.N = p->H;
  g2.lda = fp16_pitch(p->I);
  g2.nsplit = sh[1].most;
  g2.arow = nullptr;
  g2.out16 = half[1] ? reinterpret_cast<uint16_t*>(v) : nullptr;
  g2.oscale = wt->scale2;
  const int waves2 = sh[1].waves;
  if (on(3) && atomic_fc2) {
    Fc2AtomicArgs fa;
    fa.g = g2;
    fa.sorted_routes = sorted;
    fa.ids = ids;
    fa.ids64 = p->ids64;
    fa.w = w;
    fa.scale2 = wt->scale2;
    fa.sv2 = wt->sv2;
    fa.identity = p->rotation == TMOE_ROT_IDENTITY;
    fa.top_k = p->K;
    fa.tile_rows = gemm_rows;
    const int mg2 = std::min(mg, 4);
    fa.sub_rows = 16 * mg2;
    fa.y = y;
    const long long gt_ub = std::min<long long>(R, p->E + R / gemm_rows + 1);
    const long long units = gt_ub * (gemm_rows / fa.sub_rows) * sh[1].most;
    launch_fc2_atomic(fa, p->uniform_bits, mg2, static_cast<int>(std::min<long long>(units, 2048)), s);
  } else if (on(3)) {
    if (fp8) launch_gemm_f8(g2, 2, p->uniform_bits, mg, waves2, s);
    else launch_gemm_f16(g2, 2, p->uniform_bits, fc2_mg(p, mg), waves2, s);
  }

  CombineArgs ca;
  ca.v = v;
  ca.v16 = g2.out16;
  ca.nsplit = sh[1].most;
  ca.ids = ids;
  ca.ids64 = p->ids64;
  ca.w = w;
  ca.route_slot = at<int32_t>(scratch, p->lay.slot);
  ca.top_k = p->K;
  ca.tokens = T;
  ca.routes = static_cast<int>(R);
  ca.scale2 = wt->scale2;
  ca.sv2 = wt->sv2;
  ca.rot = make_rot(p->H, p->rotation == TMOE_ROT_IDENTITY);
  ca.y = y;
  // non-power-of-two rows: few tokens (token x block items up to 2048) get a workgroup per (token,
  // block) with one wavefront per route; more tokens a wavefront per (token, block) for all routes
  ca.split_segments = static_cast<long long>(T) * make_rot(p->H, 0).nblk128 <= 2048 ? 1 : 0;
  if (on(4) && !atomic_fc2) launch_combine(ca, s);

  return hipGetLastError() == hipSuccess ? TMOE_OK : TMOE_ERR_HIP;
}

bool dim_ok(int n) { return n >= 64 && n <= kMaxDim && n % 64 == 0; }

}  // namespace

// ---------------------------------------------------------------- library-owned scratch
// One arena per GPU for callers that cannot allocate. In host code `scratch` names a host-side
// stand-in, not device memory: its device address is looked up once per device with the device
// current and only that address is ever passed on.
static __device__ __align__(256) uint8_t scratch[TMOE_STATIC_SCRATCH_BYTES];

namespace {

std::mutex g_static_mu;
std::vector<void*> g_static_ptr;       // device address of `scratch`, per device id (null: not yet)

tmoe_status static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return TMOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_static_mu);
  if (static_cast<int>(g_static_ptr.size()) <= dev) g_static_ptr.resize(dev + 1, nullptr);
  if (!g_static_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return TMOE_ERR_HIP;
    g_static_ptr[dev] = ptr;
  }
  *out = g_static_ptr[dev];
  return TMOE_OK;
}

}  // namespace

// ---------------------------------------------------------------- dense trellis linear
// y_t = sv * R_N(scale * (C^T R_K(su * x_t))): the layer's input rotation, one trellis matrix (as
// the grouped GEMM of a single expert whose tiles hold every token) and the layer's output
// rotation with one route of weight 1 per token (the combine with k = 1).
struct tmoe_linear_plan_s {
  int K, N, bits, max_tokens, rotation;
  int max_gtiles;
  size_t gtiles, scalars, slot, ids, w, a1, z, total;    // arena offsets
};

namespace {

// Tile rows of the dense GEMM: every weight is decoded once per tile, so the tile holds all tokens
// up to 64 (16, 32 or 64 rows), and 128-row workgroup tiles beyond (when N allows them).
int linear_mg(int T, int N) {
  if (T <= 16) return 1;
  if (T <= 32) return 2;
  if (T <= 64) return 4;
  if (N % 256 == 0) return 16;
  if (N % 128 == 0) return 8;
  return 4;
}

tmoe_status linear_forward(const tmoe_linear_plan_s* p, const void* x, int32_t T, const tmoe_linear_weights* wt,
                           float* y, void* scratch, size_t bytes, hipStream_t s) {
  if (T < 0) return TMOE_ERR_INVALID_ARG;
  if (T > p->max_tokens) return TMOE_ERR_CAPACITY;
  if (!scratch || !aligned(scratch, 16) || bytes < p->total) return TMOE_ERR_SCRATCH;
  if (T == 0) return TMOE_OK;
  if (!x || !wt || !y || !wt->payload || !wt->scale || !wt->su || !wt->sv) return TMOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(wt->payload, 16) || !aligned(wt->scale, 2) ||
      !aligned(wt->su, 2) || !aligned(wt->sv, 2))
    return TMOE_ERR_ALIGNMENT;

  const int mg = linear_mg(T, p->N);
  const int rows = tile_rows(mg);
  const bool big = mg >= 8;
  const int ntiles = (T + rows - 1) / rows;
  const int ng = p->N / (mg == 16 ? 256 : big ? 128 : 64);
  const int splits = choose_splits(T, p->K / 32);
  long long waves = std::min<long long>(big ? kGemmGroupCap : kGemmWaveCap, 1LL * ntiles * ng * splits);
  if (big) {                                    // a whole number of 8-tile rounds of units
    const long long per = 8LL * ng * splits;
    waves = (waves + per - 1) / per * per;
  }

  LinearPrepArgs lp;
  lp.rot.x = static_cast<const uint16_t*>(x);
  lp.rot.ids = nullptr;
  lp.rot.ids64 = 0;
  lp.rot.top_k = 1;
  lp.rot.num_experts = 1;
  lp.rot.su1 = wt->su;
  lp.rot.rot = make_rot(p->K, p->rotation == TMOE_ROT_IDENTITY);
  lp.rot.a1 = at<uint8_t>(scratch, p->a1);
  lp.rot.a1_scale = nullptr;
  lp.rot.lda = fp16_pitch(p->K);
  lp.rot.routes = T;
  lp.rot.split_segments = T < 2048 ? 1 : 0;
  lp.gtiles = at<int4>(scratch, p->gtiles);
  lp.num_gtiles = at<int32_t>(scratch, p->scalars);
  lp.slot = at<int32_t>(scratch, p->slot);
  lp.ids = at<int32_t>(scratch, p->ids);
  lp.w = at<float>(scratch, p->w);
  lp.tokens = T;
  lp.tile_rows = rows;
  lp.bits = p->bits;
  const RowRot& rk = lp.rot.rot;
  const long long items = 1LL * T * (rk.pow2 || !lp.rot.split_segments ? 1 : rk.nblk128 + rk.tail64);
  lp.rot_blocks = static_cast<int>((items + 3) / 4);

  GemmArgs g;
  g.payload = wt->payload;
  g.einfo = nullptr;
  g.fc2_words_per_bit = 0;
  g.a = lp.rot.a1;
  g.arow = nullptr;
  g.a_scale = nullptr;
  g.out = at<float>(scratch, p->z);
  g.gtiles = lp.gtiles;
  g.num_gtiles = lp.num_gtiles;
  g.max_gtiles = p->max_gtiles;
  g.nsplit = splits;
  g.K = p->K;
  g.N = p->N;
  g.lda = lp.rot.lda;
  g.routes = T;

  CombineArgs ca;
  ca.v = g.out;
  ca.nsplit = splits;
  ca.ids = lp.ids;
  ca.ids64 = 0;
  ca.w = lp.w;
  ca.route_slot = lp.slot;
  ca.top_k = 1;
  ca.tokens = T;
  ca.routes = T;
  ca.scale2 = wt->scale;
  ca.sv2 = wt->sv;
  ca.rot = make_rot(p->N, p->rotation == TMOE_ROT_IDENTITY);
  ca.y = y;
  ca.split_segments = static_cast<long long>(T) * make_rot(p->N, 0).nblk128 <= 2048 ? 1 : 0;

  (void)hipGetLastError();
  launch_linear_prep(lp, s);
  launch_gemm_f16(g, 1, p->bits, mg, static_cast<int>(waves), s);
  launch_combine(ca, s);
  return hipGetLastError() == hipSuccess ? TMOE_OK : TMOE_ERR_HIP;
}

}  // namespace

extern "C" {

tmoe_status tmoe_plan(const tmoe_config* cfg, tmoe_plan_t* out, size_t* scratch_bytes, size_t* payload_words) {
  if (!cfg || !out) return TMOE_ERR_INVALID_ARG;
  *out = nullptr;
  if (cfg->hidden <= 0 || cfg->inter <= 0 || cfg->num_experts <= 0 || cfg->top_k <= 0 || cfg->max_tokens <= 0)
    return TMOE_ERR_INVALID_ARG;
  if (!cfg->expert_bits) return TMOE_ERR_INVALID_ARG;
  if (cfg->rotation != TMOE_ROT_HADAMARD && cfg->rotation != TMOE_ROT_IDENTITY) return TMOE_ERR_INVALID_ARG;
  if (cfg->ids_dtype != TMOE_IDS_I32 && cfg->ids_dtype != TMOE_IDS_I64) return TMOE_ERR_INVALID_ARG;
  const int bm = cfg->block_m;
  if (bm != 0 && bm != 8 && bm != 16 && bm != 32 && bm != 48 && bm != 64) return TMOE_ERR_INVALID_ARG;
  if (!dim_ok(cfg->hidden) || !dim_ok(cfg->inter)) return TMOE_ERR_UNSUPPORTED;
  if (cfg->num_experts > kMaxExperts || cfg->top_k > kMaxTopK) return TMOE_ERR_UNSUPPORTED;
  const long long rmax = static_cast<long long>(cfg->max_tokens) * cfg->top_k;
  if (rmax > kMaxRoutes) return TMOE_ERR_UNSUPPORTED;
  for (int e = 0; e < cfg->num_experts; ++e) {
    const int b = cfg->expert_bits[e];
    if (b < 1 || b > 16) return TMOE_ERR_INVALID_ARG;
    if (b < 2 || b > 6) return TMOE_ERR_UNSUPPORTED;
  }
  tmoe_plan_s* p = new (std::nothrow) tmoe_plan_s();
  if (!p) return TMOE_ERR_INVALID_ARG;
  p->H = cfg->hidden;
  p->I = cfg->inter;
  p->E = cfg->num_experts;
  p->K = cfg->top_k;
  p->max_tokens = cfg->max_tokens;
  p->rotation = cfg->rotation;
  p->ids64 = cfg->ids_dtype == TMOE_IDS_I64;
  p->block_m = bm ? bm : 16;
  if (cfg->smallm_max_tokens < 0) { delete p; return TMOE_ERR_INVALID_ARG; }
  if (cfg->fc2_reduce != TMOE_FC2_DETERMINISTIC && cfg->fc2_reduce != TMOE_FC2_ATOMIC) { delete p; return TMOE_ERR_INVALID_ARG; }
  p->smallm_max_tokens = cfg->smallm_max_tokens;
  p->fc2_reduce = cfg->fc2_reduce;
  p->bits.assign(cfg->expert_bits, cfg->expert_bits + p->E);
  p->offsets.assign(p->E + 1, 0);
  std::memset(p->packed_bits, 0, sizeof(p->packed_bits));
  for (int e = 0; e < p->E; ++e) {
    p->offsets[e + 1] = p->offsets[e] + 3LL * p->H * p->I * p->bits[e] / 16;
    p->packed_bits[e >> 3] |= static_cast<uint32_t>(p->bits[e]) << (4 * (e & 7));
  }
  p->routes_max = rmax;
  p->max_tiles = static_cast<int>(rmax / p->block_m + p->E + 1);
  p->max_gtiles = static_cast<int>(rmax / 16 + p->E + 1);
  // W4A8 decodes widths 2-4 only (its LDS ring holds one step of 4-bit tiles)
  p->max_bits = *std::max_element(p->bits.begin(), p->bits.end());
  p->fp8_ok = (p->H % 128 == 0) && (p->I % 128 == 0) && p->max_bits <= 4;
  p->uniform_bits = p->bits[0];
  for (int e = 1; e < p->E; ++e)
    if (p->bits[e] != p->bits[0]) p->uniform_bits = p->max_bits <= 4 ? 0 : kMixedWide;
  build_layout(p);
  *out = p;
  if (scratch_bytes) *scratch_bytes = p->lay.total;
  if (payload_words) *payload_words = static_cast<size_t>(p->offsets[p->E]);
  return TMOE_OK;
}

tmoe_status tmoe_plan_destroy(tmoe_plan_t plan) {
  if (!plan) return TMOE_ERR_INVALID_ARG;
  delete plan;
  return TMOE_OK;
}

tmoe_status tmoe_plan_get_info(tmoe_plan_t p, tmoe_plan_info* info) {
  if (!p || !info) return TMOE_ERR_INVALID_ARG;
  info->scratch_bytes = p->lay.total;
  info->payload_words = static_cast<size_t>(p->offsets[p->E]);
  info->block_m = p->block_m;
  info->max_tiles = p->max_tiles;
  return TMOE_OK;
}

tmoe_status tmoe_plan_expert_offset(tmoe_plan_t p, int32_t expert, size_t* word_offset) {
  if (!p || !word_offset || expert < 0 || expert >= p->E) return TMOE_ERR_INVALID_ARG;
  *word_offset = static_cast<size_t>(p->offsets[expert]);
  return TMOE_OK;
}

tmoe_status tmoe_build_route_map(tmoe_plan_t p, const void* ids, int32_t T, void* scratch, size_t bytes,
                                 tmoe_route_map* view, void* stream) {
  tmoe_status st = check_common(p, ids, T, scratch, bytes);
  if (st != TMOE_OK) return st;
  if (!view) return TMOE_ERR_INVALID_ARG;
  if (T == 0) return TMOE_OK;
  const long long R = static_cast<long long>(T) * p->K;
  const int mg = choose_mg(R, p->E, big_cols(p, false));
  const int gemm_rows = tile_rows(mg);
  const GemmShape sh[2] = {gemm_shape(p, R, mg, false, 1), gemm_shape(p, R, mg, false, 2)};
  bool half[2];
  half_planes(false, sh, p->fc2_reduce == TMOE_FC2_ATOMIC && fc2_atomic_fits(p, false), half);
  (void)hipGetLastError();
  enqueue_route_map(p, ids, T, gemm_rows, sh, half, scratch, nullptr, false, static_cast<hipStream_t>(stream));
  *view = make_view(p, scratch);
  return hipGetLastError() == hipSuccess ? TMOE_OK : TMOE_ERR_HIP;
}

tmoe_status tmoe_forward_w4a16(tmoe_plan_t p, const void* x, const void* ids, const float* w, int32_t T,
                               const tmoe_weights* wt, float* y, void* scratch, size_t bytes, void* stream) {
  return forward(p, x, ids, w, T, wt, y, scratch, bytes, stream, false);
}

tmoe_status tmoe_forward_w4a8(tmoe_plan_t p, const void* x, const void* ids, const float* w, int32_t T,
                              const tmoe_weights* wt, float* y, void* scratch, size_t bytes, void* stream) {
  return forward(p, x, ids, w, T, wt, y, scratch, bytes, stream, true);
}

tmoe_status tmoe_forward_w4a16_static(tmoe_plan_t p, const void* x, const void* ids, const float* w, int32_t T,
                                      const tmoe_weights* wt, float* y, void* stream) {
  if (!p) return TMOE_ERR_INVALID_ARG;
  if (p->lay.total > TMOE_STATIC_SCRATCH_BYTES) return TMOE_ERR_STATIC_SCRATCH;
  if (T == 0) return forward(p, x, ids, w, T, wt, y, nullptr, 0, stream, false);
  void* arena = nullptr;
  const tmoe_status st = static_scratch(&arena);
  if (st != TMOE_OK) return st;
  return forward(p, x, ids, w, T, wt, y, arena, TMOE_STATIC_SCRATCH_BYTES, stream, false);
}

tmoe_status tmoe_forward_stages(tmoe_plan_t p, int32_t w4a8, int32_t first, int32_t last, const void* x,
                                const void* ids, const float* w, int32_t T, const tmoe_weights* wt, float* y,
                                void* scratch, size_t bytes, void* stream) {
  if ((w4a8 != 0 && w4a8 != 1) || first < 0 || last > 4 || first > last) return TMOE_ERR_INVALID_ARG;
  return forward(p, x, ids, w, T, wt, y, scratch, bytes, stream, w4a8 != 0, first, last, true);
}

const char* tmoe_status_str(tmoe_status s) {
  switch (s) {
    case TMOE_OK: return "ok";
    case TMOE_ERR_INVALID_ARG: return "invalid argument";
    case TMOE_ERR_UNSUPPORTED: return "unsupported shape or bit width";
    case TMOE_ERR_SCRATCH: return "scratch arena too short or not 16-byte aligned";
    case TMOE_ERR_CAPACITY: return "token count above the planned capacity";
    case TMOE_ERR_ALIGNMENT: return "device pointer misaligned";
    case TMOE_ERR_HIP: return "HIP launch error";
    case TMOE_ERR_STATIC_SCRATCH: return "plan needs more scratch than the library's static arena holds";
  }
  return "unknown status";
}

tmoe_status tmoe_debug_decode(tmoe_plan_t p, const tmoe_weights* wt, int32_t expert, int32_t matrix,
                              int32_t as_e4m3, void* out, void* stream) {
  if (!p || !wt || !wt->payload || !out) return TMOE_ERR_INVALID_ARG;
  if (expert < 0 || expert >= p->E || (matrix != 0 && matrix != 1) || (as_e4m3 != 0 && as_e4m3 != 1))
    return TMOE_ERR_INVALID_ARG;
  if (!aligned(out, 16) || !aligned(wt->payload, 16)) return TMOE_ERR_ALIGNMENT;
  const int bits = p->bits[expert];
  const int K = matrix ? p->I : p->H;
  const int N = matrix ? p->H : 2 * p->I;
  const uint16_t* words = wt->payload + p->offsets[expert] + (matrix ? 2LL * p->H * p->I * bits / 16 : 0);
  (void)hipGetLastError();
  launch_debug_decode(words, bits, K, N, as_e4m3, out, static_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? TMOE_OK : TMOE_ERR_HIP;
}

tmoe_status tmoe_debug_mxfp8(const float* in, int64_t rows, int32_t cols, uint8_t* q, uint8_t* e8m0, void* stream) {
  if (!in || !q || !e8m0 || rows < 0 || cols <= 0 || cols % 32) return TMOE_ERR_INVALID_ARG;
  if (!aligned(in, 4)) return TMOE_ERR_ALIGNMENT;
  if (rows == 0) return TMOE_OK;
  (void)hipGetLastError();
  launch_debug_mxfp8(in, rows, cols, q, e8m0, static_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? TMOE_OK : TMOE_ERR_HIP;
}

tmoe_status tmoe_debug_rotate(float* data, int64_t rows, int32_t n, void* stream) {
  if (!data || rows < 0) return TMOE_ERR_INVALID_ARG;
  if (!dim_ok(n)) return TMOE_ERR_UNSUPPORTED;
  if (!aligned(data, 4)) return TMOE_ERR_ALIGNMENT;
  if (rows == 0) return TMOE_OK;
  (void)hipGetLastError();
  launch_debug_rotate(data, rows, make_rot(n, 0), static_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? TMOE_OK : TMOE_ERR_HIP;
}

tmoe_status tmoe_debug_get_views(tmoe_plan_t p, int32_t T, int32_t w4a8, void* scratch, size_t bytes,
                                 tmoe_debug_views* out) {
  if (!p || !out || T < 0 || (w4a8 != 0 && w4a8 != 1)) return TMOE_ERR_INVALID_ARG;
  if (T > p->max_tokens) return TMOE_ERR_CAPACITY;
  tmoe_status st = check_scratch(p, scratch, bytes);
  if (st != TMOE_OK) return st;
  const long long R = static_cast<long long>(T) * p->K;
  out->a1 = at<void>(scratch, p->lay.a1);
  out->a1_scale = at<uint8_t>(scratch, p->lay.a1) + static_cast<size_t>(R) * p->H;
  out->z = at<float>(scratch, p->lay.z);
  out->b = at<void>(scratch, p->lay.b);
  out->b_scale = at<uint8_t>(scratch, p->lay.b) + static_cast<size_t>(R) * p->I;
  out->v = at<float>(scratch, p->lay.v);
  out->splits = at<int32_t>(scratch, p->lay.scalars) + 3;
  out->arm_status = at<int32_t>(scratch, p->lay.scalars) + 5;
  out->half_planes = at<int32_t>(scratch, p->lay.scalars) + 6;
  out->a1_pitch = w4a8 ? p->H : fp16_pitch(p->H);
  out->b_pitch = w4a8 ? p->I : fp16_pitch(p->I);
  return TMOE_OK;
}

tmoe_status tmoe_linear_plan(const tmoe_linear_config* cfg, tmoe_linear_plan_t* out, size_t* scratch_bytes,
                             size_t* payload_words) {
  if (!cfg || !out) return TMOE_ERR_INVALID_ARG;
  *out = nullptr;
  if (cfg->in_features <= 0 || cfg->out_features <= 0 || cfg->max_tokens <= 0 || cfg->bits <= 0 || cfg->bits > 16)
    return TMOE_ERR_INVALID_ARG;
  if (cfg->rotation != TMOE_ROT_HADAMARD && cfg->rotation != TMOE_ROT_IDENTITY) return TMOE_ERR_INVALID_ARG;
  if (!dim_ok(cfg->in_features) || !dim_ok(cfg->out_features)) return TMOE_ERR_UNSUPPORTED;
  if (cfg->bits < 2 || cfg->bits > 6) return TMOE_ERR_UNSUPPORTED;
  if (cfg->max_tokens > kMaxRoutes) return TMOE_ERR_UNSUPPORTED;
  tmoe_linear_plan_s* p = new (std::nothrow) tmoe_linear_plan_s();
  if (!p) return TMOE_ERR_INVALID_ARG;
  p->K = cfg->in_features;
  p->N = cfg->out_features;
  p->bits = cfg->bits;
  p->max_tokens = cfg->max_tokens;
  p->rotation = cfg->rotation;
  const long long T = cfg->max_tokens;
  p->max_gtiles = static_cast<int>(T / 16 + 1);
  size_t off = 0;
  auto take = [&](size_t b) { size_t o = off; off = align_up(off + b); return o; };
  p->gtiles = take(16ull * p->max_gtiles);
  p->scalars = take(32);
  p->slot = take(4ull * T);
  p->ids = take(4ull * T);
  p->w = take(4ull * T);
  p->a1 = take(2ull * T * fp16_pitch(p->K));
  const int ks = p->K / 32;
  p->z = take(4ull * max_split_rows(T, ks, ks) * p->N);
  p->total = off;
  *out = p;
  if (scratch_bytes) *scratch_bytes = p->total;
  if (payload_words) *payload_words = static_cast<size_t>(p->K / 16) * (p->N / 16) * 16 * p->bits;
  return TMOE_OK;
}

tmoe_status tmoe_linear_plan_destroy(tmoe_linear_plan_t plan) {
  delete plan;
  return TMOE_OK;
}

tmoe_status tmoe_linear_w4a16(tmoe_linear_plan_t p, const void* x, int32_t T, const tmoe_linear_weights* w,
                              float* y, void* scratch, size_t bytes, void* stream) {
  if (!p) return TMOE_ERR_INVALID_ARG;
  return linear_forward(p, x, T, w, y, scratch, bytes, static_cast<hipStream_t>(stream));
}

}  // extern "C"
