// k_trellis_gemm.hip -- grouped GEMMs over the route map with trellis weights decoded in registers.
//
// Weights are never expanded in HBM: each wavefront streams the packed trellis words of its
// tiles, decodes them straight into MFMA operands (the hot path of "serve canonical Fruit QSRT
// atoms" turns the packed payload into E4M3 matrix operands directly in its W4A8 path) and
// multiplies them with the route rows of one expert. Output is route-major in slot order, one
// plane per K split, summed in a fixed order by the consumer kernel (deterministic; no atomics).
//
// Work unit of one wavefront: (GEMM tile = expert + up to 16*MG slots, 64 output columns, one K
// split); the large-batch kernel's unit is a workgroup's (128-slot tile, 256 columns, K split).
// Units are dealt to a persistent grid whose size is fixed on the host, so the launch is
// graph-capturable although the tile count is only known on the device. Within a unit the payload
// words and activation fragments of the next steps are kept in flight in an LDS ring filled by
// direct global->LDS loads (the fp16 kernels) or in registers (the fp8 kernel), so the decode of
// one step overlaps the memory latency of the next ones.
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
constexpr int DF = 2;   // fp16 path: K steps in flight
constexpr int D8 = 2;   // fp8 path: K steps in flight (each step is 4x deeper)

// A wave-uniform global pointer held in scalar registers (loads through it use the global path with
// a scalar base and a per-lane 32-bit offset).
template <class T>
using gptr = const T __attribute__((address_space(1)))*;

template <class T>
__device__ __forceinline__ gptr<T> uniform_ptr(const T* p) {
  const unsigned long long v = reinterpret_cast<unsigned long long>(p);
  const unsigned lo = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(v));
  const unsigned hi = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(v >> 32));
  return reinterpret_cast<gptr<T>>((static_cast<unsigned long long>(hi) << 32) | lo);
}

// One wavefront unit of the fp16 GEMM. Every K step's operands arrive with direct global->LDS
// loads (16 bytes per lane) into the wavefront's own slot of an LDS ring DF steps deep: the step's
// trellis words (two 16-deep tile rows x NS strips = 2*NS*TW 32-bit words, 1 KB at 4 bits; lane L
// copies chunk L, and at widths 5 and 6 lanes L < 16 or 32 also chunk 64 + L) and its A fragments (MG x 1 KB; each lane copies exactly the 16 bytes it later
// feeds to the MFMA). The memory pipeline thus holds DF steps per wavefront without registers, and
// the only waits are on the ring. Rows of the A fragment beyond the tile are not loaded (first row
// group) or repeat the tile's last row (later groups); their output rows are never stored (an MFMA
// output row depends on its own A row only), so no masking sits in the MFMA chain.
// Ring words of one wavefront for a kernel instantiated at width code BITS: its slots hold 2*NS
// tiles of up to 4 bits (widths 2-4, and BITS = 0 for mixed 2-4) or of the width itself (5, 6; 6
// for kMixedWide), then the A fragments.
template <int BITS>
constexpr int ring_tile_bits() { return BITS == kMixedWide ? 6 : (BITS > 4 ? BITS : 4); }
template <int BITS, int MG>
constexpr int ring_words() { return DF * (2 * NS * 8 * ring_tile_bits<BITS>() + MG * 256); }

// Operand row of slot p: the FC1 input is stored per route (arow maps slot -> route), the FC2 input
// per slot.
__device__ __forceinline__ long long operand_row(const GemmArgs& a, int p) {
  return a.arow ? static_cast<long long>(a.arow[p]) : static_cast<long long>(p);
}

template <int BITS, int MG>
__device__ __forceinline__ void unit_f16(const GemmArgs& a, const int4 t, int ng, int s, int splits, int lane,
                                         uint32_t* ring, uint32_t mask, uint32_t orv) {
  constexpr int TW = 8 * BITS;                         // 32-bit words per 16x16 tile
  constexpr int BW = 2 * NS * TW;                      // trellis words per K step
  constexpr int AOFF = 2 * NS * 8 * ring_tile_bits<BITS>();   // A fragments follow the trellis words
  constexpr int STAGE = AOFF + MG * 256;               // words per ring slot
  constexpr int CPT = TW / 4;                          // 16-byte chunks per tile
  constexpr int NL = BW / 4 > 64 ? 2 : 1;              // staging loads per step (5 and 6 bits: 80, 96 chunks)
  static_assert(BW / 4 <= 128, "two staging loads per step at most");
  const long long woff = (static_cast<long long>(static_cast<unsigned>(t.w)) << 8);
  const int row0 = t.y, rows = t.z;
  const int NT = a.N >> 4;
  const int col = lane & 15, grp = lane >> 4;
  const int q = 2 * col + (grp & 1);                   // 8-element group inside the tile
  const int ksteps = (a.K >> 5) / splits;
  const int ks0 = s * ksteps, ks1 = ks0 + ksteps;
  const int nt0 = ng * NS;
  const gptr<uint32_t> mat = uniform_ptr(reinterpret_cast<const uint32_t*>(a.payload + woff + a.fc2_words_per_bit * BITS) +
                                         static_cast<size_t>(nt0) * TW);
  const gptr<_Float16> A = uniform_ptr(static_cast<const _Float16*>(a.a));
  // staging of trellis words: lane L < BW/4 copies 16-byte chunk L, [tile row][strip][chunk] order
  const bool stager = lane < BW / 4;
  const int st_tile = lane / (NS * CPT), st_strip = (lane / CPT) % NS, st_chunk = lane % CPT;
  const int st_off = (st_tile * NT + st_strip) * TW + 4 * st_chunk;          // words, relative to the step
  // widths 5 and 6: lane L < BW/4 - 64 also copies chunk 64 + L, to ring word 256 + 4L
  const int c2 = 64 + lane;
  const bool stager2 = NL == 2 && c2 < BW / 4;
  const int st2_off = ((c2 / (NS * CPT)) * NT + (c2 / CPT) % NS) * TW + 4 * (c2 % CPT);
  const int kstride = 2 * NT * TW;                                            // words between K steps
  // reading: the words of group q in tile row (grp>>1) of strip ns (tmoe_device.hpp, state windows)
  constexpr int NWW = dec_words<BITS>();
  const uint32_t dsh = dec_shift<BITS>(q);
  int rd[NWW];
#pragma unroll
  for (int i = 0; i < NWW; ++i) rd[i] = (grp >> 1) * NS * TW + (dec_first_word<BITS>(q) + i + TW) % TW;
  long long aoff[MG];
#pragma unroll
  for (int mg = 0; mg < MG; ++mg) aoff[mg] = operand_row(a, row0 + min(16 * mg + col, rows - 1)) * a.lda + 8 * grp;
  // Lanes of the first row group whose row lies beyond the tile load nothing (lane 0's row always
  // exists, so every step still issues the same number of load instructions and the ring's wait
  // counts hold); their LDS bytes are stale and only feed output rows that are never stored. The
  // other row groups load a repeat of the last row instead, as a whole group may lie beyond the tile.
  const bool a_live = col < rows;

  f4 acc[MG][NS];
#pragma unroll
  for (int mg = 0; mg < MG; ++mg)
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) acc[mg][ns] = f4{0.f, 0.f, 0.f, 0.f};
  // one K split: the epilogue's channel scales, read before the staging loads (older than all of
  // them, so the constant wait counts still hold)
  uint16_t sc16[NS];
  if (a.out16) {
    const uint16_t* cs = a.oscale + static_cast<size_t>(t.x & 0xffffff) * a.N + nt0 * 16 + col;
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) sc16[ns] = cs[16 * ns];
  }

  auto issue = [&](int ks, int d) {
    uint32_t* slot = ring + d * STAGE;
    if (stager)
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(mat + static_cast<size_t>(ks) * kstride + st_off),
                                       (void __attribute__((address_space(3)))*)(slot), 16, 0, 0);
    if constexpr (NL == 2) {
      if (stager2)
        __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(mat + static_cast<size_t>(ks) * kstride + st2_off),
                                         (void __attribute__((address_space(3)))*)(slot + 256), 16, 0, 0);
    }
    const gptr<_Float16> ab = A + 32 * ks;
#pragma unroll
    for (int mg = 0; mg < MG; ++mg)
      if (mg > 0 || a_live)
        __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(ab + aoff[mg]),
                                         (void __attribute__((address_space(3)))*)(slot + AOFF + mg * 256), 16, 0, 0);
  };
  auto step = [&](int d, int next) {
    // the direct loads of the DF-1 younger steps may still be in flight
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((DF - 1) * (NL + MG)) : "memory");
    const uint32_t* slot = ring + d * STAGE;
    uint32_t w[NS][NWW];
#pragma unroll
    for (int ns = 0; ns < NS; ++ns)
#pragma unroll
      for (int i = 0; i < NWW; ++i) w[ns][i] = slot[rd[i] + ns * TW];
    half8 aa[MG];
#pragma unroll
    for (int mg = 0; mg < MG; ++mg) aa[mg] = *reinterpret_cast<const half8*>(slot + AOFF + mg * 256 + 4 * lane);
    half8 b[NS];
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) b[ns] = decode8<BITS>(w[ns], dsh, mask, orv);
    // every LDS read of this slot has returned before the slot is refilled
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    issue(next, d);
#pragma unroll
    for (int mg = 0; mg < MG; ++mg)
#pragma unroll
      for (int ns = 0; ns < NS; ++ns)
        acc[mg][ns] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aa[mg], b[ns], acc[mg][ns], 0, 0, 0);
  };
#pragma unroll
  for (int d = 0; d < DF; ++d) issue(min(ks0 + d, ks1 - 1), d);
  int base = ks0;
  for (; base + DF <= ks1; base += DF) {
#pragma unroll
    for (int d = 0; d < DF; ++d) step(d, min(base + d + DF, ks1 - 1));
  }
#pragma unroll
  for (int d = 0; d < DF; ++d)
    if (base + d < ks1) step(d, ks1 - 1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");      // no load may still target the ring

  if (a.out16) {
    // one K split: the finished sums times the expert's channel scale, rounded once to fp16
    float sc[NS];
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) sc[ns] = h2f(sc16[ns]);
    _Float16* o16 = reinterpret_cast<_Float16*>(a.out16) + static_cast<size_t>(row0) * a.N + nt0 * 16 + col;
#pragma unroll
    for (int mg = 0; mg < MG; ++mg)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * mg + 4 * grp + i;
        if (r < rows) {
#pragma unroll
          for (int ns = 0; ns < NS; ++ns)
            o16[static_cast<size_t>(r) * a.N + 16 * ns] = static_cast<_Float16>(acc[mg][ns][i] * sc[ns]);
        }
      }
    return;
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

// BITS = 0: experts of mixed widths 2-4, chosen per unit; BITS = kMixedWide: mixed widths 2-6. FC (1 or 2) only names the instantiation,
// so profiles tell the two GEMMs apart.
template <int BITS, int MG, int FC>
__device__ __forceinline__ void gemm_f16_body(const GemmArgs& a, uint32_t* ring_all) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform, kept in an SGPR
  const int gw = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + wv);
  const int W = gridDim.x * 4;
  const int NG = a.N / (16 * NS);
  const int ntiles = *a.num_gtiles;
  const int splits = a.nsplit;
  const int units = ntiles * NG * splits;
  uint32_t* ring = ring_all + wv * ring_words<BITS, MG>();
  const uint32_t mask = vreg_const(kMcgMask), orv = kMcgOr;
  for (int u = gw; u < units; u += W) {
    const int s = u % splits;
    const int rest = u / splits;
    const int ng = rest % NG;
    const int4 t = a.gtiles[rest / NG];
    if constexpr (BITS != 0 && BITS != kMixedWide) {
      unit_f16<BITS, MG>(a, t, ng, s, splits, lane, ring, mask, orv);
    } else {
      const int bits = (t.x >> 24) & 0xff;
      if (bits == 4) unit_f16<4, MG>(a, t, ng, s, splits, lane, ring, mask, orv);
      else if (bits == 3) unit_f16<3, MG>(a, t, ng, s, splits, lane, ring, mask, orv);
      else if (BITS == 0 || bits == 2) unit_f16<2, MG>(a, t, ng, s, splits, lane, ring, mask, orv);
      else if constexpr (BITS == kMixedWide) {
        if (bits == 5) unit_f16<5, MG>(a, t, ng, s, splits, lane, ring, mask, orv);
        else unit_f16<6, MG>(a, t, ng, s, splits, lane, ring, mask, orv);
      }
    }
  }
}

// Decode-size tiles (16 rows): sized to keep five wavefronts per SIMD resident, so a round of
// units covers the chip evenly.
template <int BITS, int MG, int FC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(BITS == 0 || BITS >= 5 ? 3 : 5, 8))) void k_gemm_f16_small(GemmArgs a) {
  __shared__ uint32_t ring_all[4 * ring_words<BITS, MG>()];
  gemm_f16_body<BITS, MG, FC>(a, ring_all);
}

template <int BITS, int MG, int FC>
__global__ __launch_bounds__(256) void k_gemm_f16(GemmArgs a) {
  __shared__ uint32_t ring_all[4 * ring_words<BITS, MG>()];
  gemm_f16_body<BITS, MG, FC>(a, ring_all);
}

// Prefill-size tiles: one workgroup of four wavefronts computes a tile of 128 slots (one expert) x
// 64*SPW output columns over its K range; each wavefront owns SPW adjacent 16-column strips. Each
// 32-deep K step's operands arrive with direct global->LDS loads into a ring BIG_D steps deep: the
// A rows of the step (shared: each wavefront copies two of the eight 16-row groups, already in the
// MFMA A-operand order) and the trellis words of each wavefront's own strips. A wavefront decodes
// only its own strips, so no decoded weight crosses LDS and every weight of the tile is decoded once
// per 128 rows; each A fragment read from LDS feeds SPW MFMAs. One barrier per step publishes the A
// rows and frees the ring slot of the step before. Every load is issued for every step (indices
// clamped at the end of the range), so the wait counts are constants.
constexpr int BIG_D = 4;                       // ring depth in K steps (3 in flight)
constexpr int BIG_A_U4 = 8 * 64;               // 16-byte chunks of A per step (8 KB)

// Words of one step of a wavefront: two tile rows of SPW tiles of up to RB bits, staged in NLB
// loads of 64 16-byte pieces (1 KB each): one load up to 4 bits, two at 5 and 6 bits with 4 strips.
template <int SPW, int RB>
constexpr int big_loads() { return (2 * SPW * 8 * RB / 4 + 63) / 64; }
template <int SPW, int RB>
constexpr int big_w_u4() { return 4 * 64 * big_loads<SPW, RB>(); }   // 16-byte chunks per step
template <int SPW, int RB>
constexpr int big_slot_u4() { return BIG_A_U4 + big_w_u4<SPW, RB>(); }
// Ring width of a kernel instantiated at width code BITS (mixed 2-4 and 2-6 sized for 4 and 6).
template <int BITS>
constexpr int big_ring_bits() { return BITS == kMixedWide ? 6 : (BITS > 4 ? BITS : 4); }

// NGR: 16-row groups computed, 8 for a full 128-row tile or 4 for a tile of at most 64 rows, whose
// upper four groups would only repeat its last row: those take neither MFMAs nor A loads.
template <int BITS, int SPW, int NGR, int RB>
__device__ __forceinline__ void unit_f16_big(const GemmArgs& a, const int4 t, int nb, int s, int splits, int lane,
                                             int wv, uint4* ring, uint32_t mask, uint32_t orv) {
  constexpr int TW = 8 * BITS;                   // 32-bit words per tile
  constexpr int SLOT = big_slot_u4<SPW, RB>();
  constexpr int NLB = big_loads<SPW, RB>();      // staging loads per step and wavefront
  constexpr int WREG = 64 * NLB;                 // 16-byte chunks of a wavefront's staging area
  constexpr int RUN = SPW * TW;                  // words of one tile row of this wavefront's strips
  const long long woff = (static_cast<long long>(static_cast<unsigned>(t.w)) << 8);
  const int row0 = t.y, rows = t.z;
  const int NT = a.N >> 4;
  const int col = lane & 15, grp = lane >> 4;
  const int q = 2 * col + (grp & 1);
  const int ksteps = (a.K >> 5) / splits;
  const int ks0 = s * ksteps, last = ks0 + ksteps - 1;
  const int nt0 = (nb * 4 + wv) * SPW;                    // this wavefront's first strip
  const gptr<uint32_t> mat = uniform_ptr(reinterpret_cast<const uint32_t*>(a.payload + woff + a.fc2_words_per_bit * BITS) +
                                         static_cast<size_t>(nt0) * TW);
  const gptr<_Float16> A = uniform_ptr(static_cast<const _Float16*>(a.a));
  // A rows copied by this wavefront: row groups GPW * wv .. GPW * wv + GPW - 1, in MFMA operand order
  static_assert(NGR == 8 || NGR == 4, "row groups: 8 or 4");
  constexpr int GPW = NGR / 4;                   // row groups copied per wavefront
  constexpr int LPS = GPW + NLB;                 // loads per step and wavefront (A groups + words)
  static_assert(2 * SPW * TW / 4 <= WREG, "a step's words fit the staging area");
  long long aoff[GPW];
#pragma unroll
  for (int i = 0; i < GPW; ++i) aoff[i] = operand_row(a, row0 + min(16 * (GPW * wv + i) + col, rows - 1)) * a.lda + 8 * grp;
  // trellis words: per step two tile rows x SPW adjacent tiles = two runs of RUN words in RUN / 2
  // 16-byte pieces; load i of lane L copies piece (64 i + L) mod (RUN / 2) -- piece p % (RUN / 4)
  // of run p / (RUN / 4) -- to byte 16 (64 i + L) of the wavefront's staging area. Every lane loads,
  // so the staging loads have no branch around them (a branch lets the compiler merge loads of
  // different paths, whose LDS addresses then no longer match); pieces past RUN / 2 are copies
  // written beyond the words read back.
  int st_src[NLB];
#pragma unroll
  for (int i = 0; i < NLB; ++i) {
    const int st_p = (64 * i + lane) % (RUN / 2);
    st_src[i] = (st_p / (RUN / 4)) * NT * TW + 4 * (st_p % (RUN / 4));   // words, relative to the step
  }
  // words of group q in tile row (grp >> 1) of strip j: [run][strip][TW] in the slot
  constexpr int NWW = dec_words<BITS>();
  const uint32_t dsh = dec_shift<BITS>(q);
  int rd[NWW];
#pragma unroll
  for (int i = 0; i < NWW; ++i) rd[i] = (grp >> 1) * RUN + (dec_first_word<BITS>(q) + i + TW) % TW;

  auto issue = [&](int ks, int slot) {
    uint4* sl = ring + slot * SLOT;
#pragma unroll
    for (int i = 0; i < GPW; ++i)
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(A + 32 * ks + aoff[i]),
                                       (void __attribute__((address_space(3)))*)(sl + (GPW * wv + i) * 64), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < NLB; ++i)
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(mat + static_cast<size_t>(2 * ks) * NT * TW + st_src[i]),
                                       (void __attribute__((address_space(3)))*)(sl + BIG_A_U4 + wv * WREG + 64 * i), 16, 0, 0);
  };

  f4 acc[NGR][SPW];
#pragma unroll
  for (int g = 0; g < NGR; ++g)
#pragma unroll
    for (int j = 0; j < SPW; ++j) acc[g][j] = f4{0.f, 0.f, 0.f, 0.f};
  // one K split: the channel scales of the epilogue are read now, so their latency passes during
  // the K loop (they are older than every staging load, so the constant wait counts still hold)
  uint16_t sc16[SPW];
  if (a.out16) {
    const uint16_t* cs = a.oscale + static_cast<size_t>(t.x & 0xffffff) * a.N + nt0 * 16 + col;
#pragma unroll
    for (int j = 0; j < SPW; ++j) sc16[j] = cs[16 * j];
  }

#pragma unroll
  for (int d = 0; d < BIG_D - 1; ++d) issue(min(ks0 + d, last), d);
  // The weights of step ks are decoded during step ks - 1, interleaved with its MFMAs (scheduling
  // groups below), so the VALU work of one step overlaps the matrix work of the step before.
  auto decode_slot = [&](int slot, half8 (&bb)[SPW]) {
    const uint32_t* ws = reinterpret_cast<const uint32_t*>(ring + slot * SLOT + BIG_A_U4 + wv * WREG);
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      uint32_t w[NWW];
#pragma unroll
      for (int i = 0; i < NWW; ++i) w[i] = ws[rd[i] + j * TW];
      bb[j] = decode8<BITS>(w, dsh, mask, orv);
    }
  };
  half8 b0[SPW], b1[SPW];
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LPS * (BIG_D - 2)) : "memory");   // step ks0 is in
  decode_slot(0, b0);
  int slot = 0;
  // One K step: MFMAs on b (decoded during the step before) while decoding the next step into nb.
  auto step = [&](int ks, half8 (&b)[SPW], half8 (&nb)[SPW]) {
    // Step ks + 1 has landed (only step ks + 2's LPS loads may be in flight) and this wavefront's
    // LDS reads are done; a plain barrier (no fence: a fence would also wait for the younger loads)
    // then publishes steps ks and ks + 1 and frees the slot of step ks - 1.
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(LPS * (BIG_D - 3)) : "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");                          // no LDS access moves above the barrier
    const int refill = slot == 0 ? BIG_D - 1 : slot - 1;
    issue(min(ks + BIG_D - 1, last), refill);
    const uint4* sl = ring + slot * SLOT;
    slot = slot + 1 == BIG_D ? 0 : slot + 1;
    // next step's words (the slot of step ks + 1; after the last step a stale slot, decoded unused)
    const uint32_t* wsn = reinterpret_cast<const uint32_t*>(ring + slot * SLOT + BIG_A_U4 + wv * WREG);
    uint32_t wn[SPW][NWW];
#pragma unroll
    for (int j = 0; j < SPW; ++j)
#pragma unroll
      for (int i = 0; i < NWW; ++i) wn[j][i] = wsn[rd[i] + j * TW];
    half8 av = *reinterpret_cast<const half8*>(sl + lane);
    __builtin_amdgcn_sched_barrier(0);
    // NGR pieces, kept in this order: the next A fragment's LDS read, this row group's SPW MFMAs
    // and, spread over the pieces, the next step's decode one strip (or, with four pieces and four
    // strips, one strip per piece) at a time.
#pragma unroll
    for (int g = 0; g < NGR; ++g) {
      const half8 an = g + 1 < NGR ? *reinterpret_cast<const half8*>(sl + (g + 1) * 64 + lane) : av;
#pragma unroll
      for (int j = 0; j < SPW; ++j) acc[g][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, b[j], acc[g][j], 0, 0, 0);
      constexpr int every = NGR / SPW > 0 ? NGR / SPW : 1;
      if (g % every == every - 1) nb[g / every] = decode8<BITS>(wn[g / every], dsh, mask, orv);
      av = an;
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  int ks = ks0;
  for (; ks + 1 <= last; ks += 2) {
    step(ks, b0, b1);
    step(ks + 1, b1, b0);
  }
  if (ks <= last) step(ks, b0, b1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();                                          // the next unit refills the ring

  // the lane's row offset passes through an empty asm so the store offsets are not hoisted out of
  // the unit loop into VGPRs
  int lane_off = 4 * grp * a.N;
  asm volatile("" : "+v"(lane_off));
  if (a.out16) {
    // one K split: the finished sums times the expert's channel scale, rounded once to fp16
    float sc[SPW];
#pragma unroll
    for (int j = 0; j < SPW; ++j) sc[j] = h2f(sc16[j]);
    _Float16* o = reinterpret_cast<_Float16*>(a.out16) + static_cast<size_t>(row0) * a.N + nt0 * 16 + col;
#pragma unroll
    for (int g = 0; g < NGR; ++g)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (16 * g + 4 * grp + i < rows) {
#pragma unroll
          for (int j = 0; j < SPW; ++j)
            o[lane_off + (16 * g + i) * a.N + 16 * j] = static_cast<_Float16>(acc[g][j][i] * sc[j]);
        }
      }
    return;
  }
  float* o = a.out + (static_cast<size_t>(s) * a.routes + row0) * a.N + nt0 * 16 + col;
#pragma unroll
  for (int g = 0; g < NGR; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (16 * g + 4 * grp + i < rows) {
#pragma unroll
        for (int j = 0; j < SPW; ++j) o[lane_off + (16 * g + i) * a.N + 16 * j] = acc[g][j][i];   // < 2^31
      }
    }
}

// A unit body as a separate function: the mixed-width kernel holds six bodies (three widths, two
// row-group counts), and inlining them all lets values hoisted above the width switch stay live
// through every body and spill inside the K loops.
// The launch arguments reach it through memory: they are copied into registers first and those
// loads are complete before the unit's first staging load, so the unit's constant wait counts still
// count its own staging loads only.
template <int BITS, int SPW, int NGR, int RB>
__device__ __attribute__((noinline)) void unit_f16_big_call(const GemmArgs& a, const int4 t, int nb, int s, int splits,
                                                            int lane, int wv, uint4* ring, uint32_t mask, uint32_t orv) {
  const GemmArgs la = a;
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  unit_f16_big<BITS, SPW, NGR, RB>(la, t, nb, s, splits, lane, wv, ring, mask, orv);
}

// One unit at the tile's width (BITS = 0 or kMixedWide: experts of mixed widths 2-4 or 2-6, read
// from the tile).
template <int BITS, int SPW, int NGR>
__device__ __forceinline__ void big_unit_width(const GemmArgs& a, const int4 t, int nb, int s, int splits, int lane,
                                               int wv, uint4* ring, uint32_t mask, uint32_t orv) {
  constexpr int RB = big_ring_bits<BITS>();
  if constexpr (BITS != 0 && BITS != kMixedWide) {
    unit_f16_big<BITS, SPW, NGR, RB>(a, t, nb, s, splits, lane, wv, ring, mask, orv);
  } else {
    const int bits = __builtin_amdgcn_readfirstlane((t.x >> 24) & 0xff);
    if (bits == 4) unit_f16_big_call<4, SPW, NGR, RB>(a, t, nb, s, splits, lane, wv, ring, mask, orv);
    else if (bits == 3) unit_f16_big_call<3, SPW, NGR, RB>(a, t, nb, s, splits, lane, wv, ring, mask, orv);
    else if (BITS == 0 || bits == 2) unit_f16_big_call<2, SPW, NGR, RB>(a, t, nb, s, splits, lane, wv, ring, mask, orv);
    else if constexpr (BITS == kMixedWide) {
      if (bits == 5) unit_f16_big_call<5, SPW, NGR, RB>(a, t, nb, s, splits, lane, wv, ring, mask, orv);
      else unit_f16_big_call<6, SPW, NGR, RB>(a, t, nb, s, splits, lane, wv, ring, mask, orv);
    }
  }
}

// Units (tile, 64*SPW-column block, K split) are dealt to workgroups. Workgroups are dealt to the
// eight XCDs round-robin (workgroup b runs on XCD b mod 8), so workgroup b serves the units of tile
// (b mod 8) + 8 * (g / upt), unit g mod upt of it, with g = b div 8 and upt the units of one tile:
// the units of one tile run on one XCD and share its L2 copy of the tile's A rows, and consecutive
// tiles go to different XCDs. The grid is a multiple of 8 * upt (sized on the host from an upper
// bound on the tile count), so this is a permutation of the grid; surplus workgroups leave at once.
template <int BITS, int SPW, int FC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(SPW >= 4 ? 2 : 3, 8))) void k_gemm_f16_big(GemmArgs a) {
  __shared__ uint4 ring[BIG_D * big_slot_u4<SPW, big_ring_bits<BITS>()>()];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform, kept in an SGPR
  const int NB = a.N / (64 * SPW);
  const int splits = a.nsplit;
  const int G = gridDim.x;
  const int upt = NB * splits;                              // units of one tile
  const int gi = blockIdx.x >> 3;
  const int first = ((blockIdx.x & 7) + 8 * (gi / upt)) * upt + gi % upt;
  // The first unit's tile entry is read beside the tile count; every later unit's entry is a scalar
  // load issued when the unit before it starts, so it has landed when that unit ends (the tile list
  // is written by an earlier launch and only read here; an entry past the count is read but never
  // used).
  typedef int tile_v __attribute__((ext_vector_type(4)));
  typedef const __attribute__((address_space(4))) tile_v* tiles_ptr;
  const tiles_ptr gt = reinterpret_cast<tiles_ptr>(reinterpret_cast<uintptr_t>(a.gtiles));
  auto tile_at = [&](int u) {
    const tile_v v = gt[min(u / upt, a.max_gtiles - 1)];
    return make_int4(v.x, v.y, v.z, v.w);
  };
  int4 t = tile_at(first);
  int ntiles = *a.num_gtiles;
  t = make_int4(__builtin_amdgcn_readfirstlane(t.x), __builtin_amdgcn_readfirstlane(t.y),
                __builtin_amdgcn_readfirstlane(t.z), __builtin_amdgcn_readfirstlane(t.w));
  ntiles = __builtin_amdgcn_readfirstlane(ntiles);
  asm volatile("" : "+s"(t.x), "+s"(t.y), "+s"(t.z), "+s"(t.w), "+s"(ntiles));   // both loads in flight together
  const int units = ntiles * NB * splits;
  const uint32_t mask = vreg_const(kMcgMask), orv = kMcgOr;
  for (int u = first; u < units; u += G) {
    const int4 tn = tile_at(u + G);
    const int s = u % splits;
    const int rest = u / splits;
    const int nb = rest % NB;
    if (__builtin_amdgcn_readfirstlane(t.z) > 64) big_unit_width<BITS, SPW, 8>(a, t, nb, s, splits, lane, wv, ring, mask, orv);
    else big_unit_width<BITS, SPW, 4>(a, t, nb, s, splits, lane, wv, ring, mask, orv);
    t = tn;
  }
}

// 32 E4M3 weights of one lane for one 128-deep K step: tiles kt0 (bytes 0-15) and kt0+4
// (bytes 16-31) of one column, 16 consecutive elements of each (groups 2*col and 2*col+1).
// w[g] holds the words of group 2*col + (g & 1) of tile kt0 (g < 2) or kt0+4 (g >= 2); sh[g & 1] is
// that group's window shift.
template <int BITS>
__device__ __forceinline__ i8v decode_b_f8(const uint32_t (&w)[4][dec_words<BITS>()], const uint32_t (&sh)[2],
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

// Ring words of one wavefront of the scaled-fp8 GEMM: D8 steps of 8 tile rows x NS strips, sized for
// 4 bits (4 KB per step).
constexpr int kF8StepWords = 8 * NS * 8 * 4;

template <int BITS, int MG>
__device__ __forceinline__ void unit_f8(const GemmArgs& a, const int4 t, int ng, int s, int splits, int lane,
                                        uint32_t* ring, uint32_t mask, uint32_t orv) {
  constexpr int TW = 8 * BITS;
  const long long woff = (static_cast<long long>(static_cast<unsigned>(t.w)) << 8);
  const int row0 = t.y, rows = t.z;
  const int NT = a.N >> 4;
  const int col = lane & 15, grp = lane >> 4;
  const int ksteps = (a.K >> 7) / splits;
  const int ks0 = s * ksteps, ks1 = ks0 + ksteps;
  const int nt0 = ng * NS;
  const gptr<uint32_t> mat = uniform_ptr(reinterpret_cast<const uint32_t*>(a.payload + woff + a.fc2_words_per_bit * BITS) +
                                         static_cast<size_t>(nt0) * TW);
  const uint8_t* A = static_cast<const uint8_t*>(a.a);
  const int kblocks = a.K >> 5;

  const uint8_t* arow[MG];
  const uint8_t* srow[MG];
#pragma unroll
  for (int mg = 0; mg < MG; ++mg) {
    const int r = 16 * mg + col;
    const size_t rr = static_cast<size_t>(operand_row(a, row0 + (r < rows ? r : 0)));
    arow[mg] = A + rr * a.K + 16 * grp;
    srow[mg] = a.a_scale + rr * kblocks + grp;
  }
  f4 acc[MG][NS];
#pragma unroll
  for (int mg = 0; mg < MG; ++mg)
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) acc[mg][ns] = f4{0.f, 0.f, 0.f, 0.f};

  // A step's trellis words (8 tile rows of NS adjacent tiles, NS*TW words each) arrive with BITS
  // direct global->LDS loads per lane, 16 bytes each: piece c = 64 i + lane is 16-byte chunk c % (NS*TW/4)
  // of tile row c / (NS*TW/4), written to ring word 4c ([tile row][strip][TW] order). A lane then reads
  // the words of its four groups -- 2*col and 2*col+1 of tile rows grp and grp + 4 -- from the slot.
  constexpr int CPR = NS * TW / 4;                     // 16-byte chunks per tile row
  int st_src[BITS];
#pragma unroll
  for (int i = 0; i < BITS; ++i) {
    const int c = 64 * i + lane;
    st_src[i] = (c / CPR) * NT * TW + 4 * (c % CPR);
  }
  constexpr int NWW = dec_words<BITS>();
  const uint32_t dsh[2] = {dec_shift<BITS>(2 * col), dec_shift<BITS>(2 * col + 1)};
  int rd[4][NWW];
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int i = 0; i < NWW; ++i)
      rd[g][i] = (grp + 4 * (g >> 1)) * NS * TW + (dec_first_word<BITS>(2 * col + (g & 1)) + i + TW) % TW;
  // A operands in the MFMA's register shape: bytes 0-15 from k = 16*grp + [0, 16) of the step, bytes
  // 16-31 from k = 64 + 16*grp + [0, 16). Rows beyond the tile load row 0 of the tile instead; their
  // output rows are never stored (an MFMA output row depends on its own A row and scale only).
  i8v areg[D8][MG];
  int asc[D8][MG];
  auto issue = [&](int ks, int d) {
    uint32_t* slot = ring + d * kF8StepWords;
    const gptr<uint32_t> src = mat + static_cast<size_t>(8 * ks) * NT * TW;
#pragma unroll
    for (int i = 0; i < BITS; ++i)
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(src + st_src[i]),
                                       (void __attribute__((address_space(3)))*)(slot + 256 * i), 16, 0, 0);
#pragma unroll
    for (int mg = 0; mg < MG; ++mg) {
      typedef int i4v __attribute__((ext_vector_type(4)));
      const i4v lo = *reinterpret_cast<const i4v*>(arow[mg] + 128 * ks);
      const i4v hi = *reinterpret_cast<const i4v*>(arow[mg] + 128 * ks + 64);
      areg[d][mg] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      asc[d][mg] = srow[mg][4 * ks];
    }
  };
  auto step = [&](int d, int next) {
    // the loads of the D8-1 younger steps may still be in flight
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((D8 - 1) * (BITS + 3 * MG)) : "memory");
    const uint32_t* slot = ring + d * kF8StepWords;
    i8v b[NS];
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
      uint32_t w[4][NWW];
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int i = 0; i < NWW; ++i) w[g][i] = slot[rd[g][i] + ns * TW];
      b[ns] = decode_b_f8<BITS>(w, dsh, mask, orv);
    }
    i8v av[MG];
    int sa[MG];
#pragma unroll
    for (int mg = 0; mg < MG; ++mg) {
      av[mg] = areg[d][mg];
      sa[mg] = asc[d][mg];
    }
    // every LDS read of this slot has returned before the slot is refilled
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    issue(next, d);
#pragma unroll
    for (int mg = 0; mg < MG; ++mg)
#pragma unroll
      for (int ns = 0; ns < NS; ++ns)
        acc[mg][ns] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av[mg], b[ns], acc[mg][ns], 0, 0, 0,
                                                                      sa[mg], 0, 127);
  };
#pragma unroll
  for (int d = 0; d < D8; ++d) issue(min(ks0 + d, ks1 - 1), d);
  int base = ks0;
  for (; base + D8 <= ks1; base += D8) {
#pragma unroll
    for (int d = 0; d < D8; ++d) step(d, min(base + d + D8, ks1 - 1));
  }
#pragma unroll
  for (int d = 0; d < D8; ++d)
    if (base + d < ks1) step(d, ks1 - 1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");      // no load may still target the ring

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

template <int BITS, int MG, int FC>
__global__ __launch_bounds__(256) void k_gemm_f8(GemmArgs a) {
  __shared__ uint32_t ring_all[4 * D8 * kF8StepWords];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint32_t* ring = ring_all + wv * D8 * kF8StepWords;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int W = gridDim.x * 4;
  const int NG = a.N / (16 * NS);
  const int splits = a.nsplit;
  int4 t = a.gtiles[min(gw / (NG * splits), a.max_gtiles - 1)];   // read beside the tile count
  int ntiles = *a.num_gtiles;
  t = make_int4(__builtin_amdgcn_readfirstlane(t.x), __builtin_amdgcn_readfirstlane(t.y),
                __builtin_amdgcn_readfirstlane(t.z), __builtin_amdgcn_readfirstlane(t.w));
  ntiles = __builtin_amdgcn_readfirstlane(ntiles);
  asm volatile("" : "+s"(t.x), "+s"(t.y), "+s"(t.z), "+s"(t.w), "+s"(ntiles));   // both loads in flight together
  const int units = ntiles * NG * splits;
  const uint32_t mask = vreg_const(kMcgMask), orv = kMcgOr;
  for (int u = gw; u < units; u += W, t = a.gtiles[min(u / (NG * splits), a.max_gtiles - 1)]) {
    const int s = u % splits;
    const int rest = u / splits;
    const int ng = rest % NG;
    if constexpr (BITS != 0) {
      unit_f8<BITS, MG>(a, t, ng, s, splits, lane, ring, mask, orv);
    } else {
      const int bits = (t.x >> 24) & 0xff;
      if (bits == 4) unit_f8<4, MG>(a, t, ng, s, splits, lane, ring, mask, orv);
      else if (bits == 3) unit_f8<3, MG>(a, t, ng, s, splits, lane, ring, mask, orv);
      else unit_f8<2, MG>(a, t, ng, s, splits, lane, ring, mask, orv);
    }
  }
}

// FC2 with the opt-in FP32-atomic reduction ("Share trellis preparation across native and EXL3
// containers", b12x PR #433: the optional FP32 atomic prefill reduction, which gives up a bitwise
// summation order). A workgroup of NW = H/128 wavefronts owns whole output rows: its unit is (GEMM
// tile, block of 16*MG rows of it, K split), and wavefront wv computes columns [128 wv, 128 wv +
// 128) of the block (8 strips, decoded by that wavefront alone, once per block). The epilogue goes
// one 16-row group at a time through LDS as fp32 rows; a wavefront then takes whole rows and applies
// the combine's per-route work -- scale2, the H-point rotation, sv2, the route's top-k weight -- and
// adds the row into y[t] with fp32 atomics. The split-plane v and the combine launch disappear; the
// sum over a token's routes and over the K splits (each split's partial is rotated and added on
// its own: every step after the contraction is linear) follows the order in which the atomics land.
constexpr int FNS = 8;   // 16-column strips per wavefront (128 columns)

template <int BITS, int MG>
constexpr int fa_ring_words() { return DF * (2 * FNS * 8 * 4 + MG * 256); }

template <int BITS, int MG, int NW>
__device__ __forceinline__ void fc2_atomic_unit(const Fc2AtomicArgs& fa, const int4 t, int row0, int rows, int s,
                                                int splits, int lane, int wv, uint32_t* lds_all, uint32_t mask,
                                                uint32_t orv) {
  const GemmArgs& a = fa.g;
  constexpr int TW = 8 * BITS;
  constexpr int BW = 2 * FNS * TW;                     // trellis words per K step
  constexpr int AOFF = 2 * FNS * 8 * 4;                // A fragments after the trellis words (sized for 4 bits)
  constexpr int STAGE = AOFF + MG * 256;
  constexpr int CPT = TW / 4;
  constexpr int NL = BW / 4 > 64 ? 2 : 1;
  static_assert(BW / 4 <= 128, "two staging loads per step at most");
  constexpr int H = 128 * NW;
  uint32_t* ring = lds_all + wv * fa_ring_words<BITS, MG>();
  const long long woff = (static_cast<long long>(static_cast<unsigned>(t.w)) << 8);
  const int NT = H >> 4;
  const int col = lane & 15, grp = lane >> 4;
  const int q = 2 * col + (grp & 1);
  const int ksteps = (a.K >> 5) / splits;
  const int ks0 = s * ksteps, ks1 = ks0 + ksteps;
  const int nt0 = wv * FNS;
  const gptr<uint32_t> mat = uniform_ptr(reinterpret_cast<const uint32_t*>(a.payload + woff + a.fc2_words_per_bit * BITS) +
                                         static_cast<size_t>(nt0) * TW);
  const gptr<_Float16> A = uniform_ptr(static_cast<const _Float16*>(a.a));
  const bool stager = lane < BW / 4;
  const int st_off = ((lane / (FNS * CPT)) * NT + (lane / CPT) % FNS) * TW + 4 * (lane % CPT);
  const int c2 = 64 + lane;
  const bool stager2 = NL == 2 && c2 < BW / 4;
  const int st2_off = ((c2 / (FNS * CPT)) * NT + (c2 / CPT) % FNS) * TW + 4 * (c2 % CPT);
  const int kstride = 2 * NT * TW;
  constexpr int NWW = dec_words<BITS>();
  const uint32_t dsh = dec_shift<BITS>(q);
  int rd[NWW];
#pragma unroll
  for (int i = 0; i < NWW; ++i) rd[i] = (grp >> 1) * FNS * TW + (dec_first_word<BITS>(q) + i + TW) % TW;
  long long aoff[MG];
#pragma unroll
  for (int mg = 0; mg < MG; ++mg) aoff[mg] = static_cast<long long>(row0 + min(16 * mg + col, rows - 1)) * a.lda + 8 * grp;
  const bool a_live = col < rows;

  f4 acc[MG][FNS];
#pragma unroll
  for (int mg = 0; mg < MG; ++mg)
#pragma unroll
    for (int ns = 0; ns < FNS; ++ns) acc[mg][ns] = f4{0.f, 0.f, 0.f, 0.f};

  auto issue = [&](int ks, int d) {
    uint32_t* slot = ring + d * STAGE;
    if (stager)
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(mat + static_cast<size_t>(ks) * kstride + st_off),
                                       (void __attribute__((address_space(3)))*)(slot), 16, 0, 0);
    if constexpr (NL == 2) {
      if (stager2)
        __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(mat + static_cast<size_t>(ks) * kstride + st2_off),
                                         (void __attribute__((address_space(3)))*)(slot + 256), 16, 0, 0);
    }
    const gptr<_Float16> ab = A + 32 * ks;
#pragma unroll
    for (int mg = 0; mg < MG; ++mg)
      if (mg > 0 || a_live)
        __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(ab + aoff[mg]),
                                         (void __attribute__((address_space(3)))*)(slot + AOFF + mg * 256), 16, 0, 0);
  };
  auto step = [&](int d, int next) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((DF - 1) * (NL + MG)) : "memory");
    const uint32_t* slot = ring + d * STAGE;
    uint32_t w[FNS][NWW];
#pragma unroll
    for (int ns = 0; ns < FNS; ++ns)
#pragma unroll
      for (int i = 0; i < NWW; ++i) w[ns][i] = slot[rd[i] + ns * TW];
    half8 aa[MG];
#pragma unroll
    for (int mg = 0; mg < MG; ++mg) aa[mg] = *reinterpret_cast<const half8*>(slot + AOFF + mg * 256 + 4 * lane);
    half8 b[FNS];
#pragma unroll
    for (int ns = 0; ns < FNS; ++ns) b[ns] = decode8<BITS>(w[ns], dsh, mask, orv);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    issue(next, d);
#pragma unroll
    for (int mg = 0; mg < MG; ++mg)
#pragma unroll
      for (int ns = 0; ns < FNS; ++ns)
        acc[mg][ns] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aa[mg], b[ns], acc[mg][ns], 0, 0, 0);
  };
#pragma unroll
  for (int d = 0; d < DF; ++d) issue(min(ks0 + d, ks1 - 1), d);
  int base = ks0;
  for (; base + DF <= ks1; base += DF) {
#pragma unroll
    for (int d = 0; d < DF; ++d) step(d, min(base + d + DF, ks1 - 1));
  }
#pragma unroll
  for (int d = 0; d < DF; ++d)
    if (base + d < ks1) step(d, ks1 - 1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();                                   // every ring is idle: LDS becomes the row buffer

  float* rowbuf = reinterpret_cast<float*>(lds_all);  // [16][H]
  const int e = t.x & 0xffffff;
  const uint16_t* c2v = fa.scale2 + static_cast<size_t>(e) * H + lane;
  const uint16_t* sgv = fa.sv2 + static_cast<size_t>(e) * H + lane;
  constexpr int S = H / 64;
#pragma unroll
  for (int g = 0; g < MG; ++g) {
    if (16 * g >= rows) break;                        // uniform over the workgroup
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int ns = 0; ns < FNS; ++ns) rowbuf[(4 * grp + i) * H + 128 * wv + 16 * ns + col] = acc[g][ns][i];
    __syncthreads();
    const int nrows = min(16, rows - 16 * g);
    for (int rr = wv; rr < nrows; rr += NW) {
      const int p = row0 + 16 * g + rr;
      const int route = fa.sorted_routes[p];
      const float wt = fa.w[route];
      float v[S];
#pragma unroll
      for (int i = 0; i < S; ++i) v[i] = rowbuf[rr * H + 64 * i + lane] * h2f(c2v[64 * i]);
      if (!fa.identity) fwht_segment<S>(v, lane);
      float* yr = fa.y + static_cast<size_t>(route / fa.top_k) * H + lane;
#pragma unroll
      for (int i = 0; i < S; ++i)
        __hip_atomic_fetch_add(yr + 64 * i, wt * (v[i] * h2f(sgv[64 * i])), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();                                  // the row buffer is rewritten next
  }
}

template <int BITS, int MG, int NW>
__global__ __launch_bounds__(64 * NW) void k_fc2_atomic(Fc2AtomicArgs fa) {
  constexpr int RING = NW * fa_ring_words<BITS, MG>();
  constexpr int ROWS = 16 * 128 * NW;                // one 16-row group of fp32 rows
  __shared__ uint32_t lds_all[RING > ROWS ? RING : ROWS];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int splits = fa.g.nsplit;
  const int subs = fa.tile_rows / fa.sub_rows;
  const int units = *fa.g.num_gtiles * subs * splits;
  const uint32_t mask = vreg_const(kMcgMask), orv = kMcgOr;
  for (int u = blockIdx.x; u < units; u += gridDim.x) {
    const int s = u % splits;
    const int rest = u / splits;
    const int sub = rest % subs;
    const int4 t = fa.g.gtiles[rest / subs];
    const int rows = min(fa.sub_rows, t.z - sub * fa.sub_rows);
    if (rows <= 0) continue;                          // uniform: a part of a tile past its last row
    const int row0 = t.y + sub * fa.sub_rows;
    if constexpr (BITS != 0) {
      fc2_atomic_unit<BITS, MG, NW>(fa, t, row0, rows, s, splits, lane, wv, lds_all, mask, orv);
    } else {
      const int bits = (t.x >> 24) & 0xff;
      if (bits == 4) fc2_atomic_unit<4, MG, NW>(fa, t, row0, rows, s, splits, lane, wv, lds_all, mask, orv);
      else if (bits == 3) fc2_atomic_unit<3, MG, NW>(fa, t, row0, rows, s, splits, lane, wv, lds_all, mask, orv);
      else fc2_atomic_unit<2, MG, NW>(fa, t, row0, rows, s, splits, lane, wv, lds_all, mask, orv);
    }
  }
}

// Dense decode of one K x N matrix with the GEMM's own lane mapping and decode (test hook).
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
  const uint32_t mask = vreg_const(kMcgMask);
  uint32_t p[4];
  uint32_t w[dec_words<BITS>()];
  load_dec_words<BITS>(tile, q, w);
  decode8_pairs<BITS>(w, dec_shift<BITS>(q), mask, kMcgOr, p);
  const int k0 = 16 * kt + 8 * (grp & 1);
  const int n = 16 * nt + col;
  if (!as_e4m3) {
    uint16_t* o = static_cast<uint16_t*>(out);
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
      o[static_cast<size_t>(k0 + jj) * N + n] = static_cast<uint16_t>(p[jj >> 1] >> (16 * (jj & 1)));
  } else {
    const uint32_t w0 = fp8x4_from_pairs(p[0], p[1]), w1 = fp8x4_from_pairs(p[2], p[3]);
    uint8_t* o = static_cast<uint8_t*>(out);
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const uint32_t w = jj < 4 ? w0 : w1;
      o[static_cast<size_t>(k0 + jj) * N + n] = static_cast<uint8_t>((w >> (8 * (jj & 3))) & 0xffu);
    }
  }
}

template <int BITS, int FC>
void launch_f16(const GemmArgs& a, int mg, dim3 grid, hipStream_t s) {
  if (mg >= 16) hipLaunchKernelGGL((k_gemm_f16_big<BITS, 4, FC>), grid, dim3(256), 0, s, a);
  else if (mg >= 8) hipLaunchKernelGGL((k_gemm_f16_big<BITS, 2, FC>), grid, dim3(256), 0, s, a);
  else if (mg >= 4) hipLaunchKernelGGL((k_gemm_f16<BITS, 4, FC>), grid, dim3(256), 0, s, a);
  else if (mg == 2) hipLaunchKernelGGL((k_gemm_f16<BITS, 2, FC>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((k_gemm_f16_small<BITS, 1, FC>), grid, dim3(256), 0, s, a);
}

template <int BITS, int FC>
void launch_f8(const GemmArgs& a, int mg, dim3 grid, hipStream_t s) {
  if (mg >= 4) hipLaunchKernelGGL((k_gemm_f8<BITS, 4, FC>), grid, dim3(256), 0, s, a);
  else if (mg == 2) hipLaunchKernelGGL((k_gemm_f8<BITS, 2, FC>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((k_gemm_f8<BITS, 1, FC>), grid, dim3(256), 0, s, a);
}

template <int FC>
void launch_f16_bits(const GemmArgs& a, int bits, int mg, dim3 grid, hipStream_t s) {
  switch (bits) {
    case 4: launch_f16<4, FC>(a, mg, grid, s); break;
    case 3: launch_f16<3, FC>(a, mg, grid, s); break;
    case 2: launch_f16<2, FC>(a, mg, grid, s); break;
    case 5: launch_f16<5, FC>(a, mg, grid, s); break;
    case 6: launch_f16<6, FC>(a, mg, grid, s); break;
    case kMixedWide: launch_f16<kMixedWide, FC>(a, mg, grid, s); break;
    default: launch_f16<0, FC>(a, mg, grid, s); break;
  }
}

template <int FC>
void launch_f8_bits(const GemmArgs& a, int bits, int mg, dim3 grid, hipStream_t s) {
  switch (bits) {
    case 4: launch_f8<4, FC>(a, mg, grid, s); break;
    case 3: launch_f8<3, FC>(a, mg, grid, s); break;
    case 2: launch_f8<2, FC>(a, mg, grid, s); break;
    default: launch_f8<0, FC>(a, mg, grid, s); break;
  }
}

}  // namespace

void launch_gemm_f16(const GemmArgs& a, int fc, int bits, int mg, int waves, hipStream_t s) {
  const dim3 grid(mg >= 8 ? waves : (waves + 3) / 4);   // mg >= 8: workgroups (a multiple of 8 tiles' units)
  if (fc == 1) launch_f16_bits<1>(a, bits, mg, grid, s);
  else launch_f16_bits<2>(a, bits, mg, grid, s);
}

void launch_gemm_f8(const GemmArgs& a, int fc, int bits, int mg, int waves, hipStream_t s) {
  const dim3 grid((waves + 3) / 4);
  if (fc == 1) launch_f8_bits<1>(a, bits, mg, grid, s);
  else launch_f8_bits<2>(a, bits, mg, grid, s);
}

void launch_fc2_atomic(const Fc2AtomicArgs& a, int bits, int mg2, int groups, hipStream_t s) {
  auto go = [&](auto b_c, auto m_c, auto w_c) {
    constexpr int B = decltype(b_c)::value, M = decltype(m_c)::value, NW = decltype(w_c)::value;
    hipLaunchKernelGGL((k_fc2_atomic<B, M, NW>), dim3(groups), dim3(64 * NW), 0, s, a);
  };
  auto with_mg = [&](auto b_c, auto w_c) {
    if (mg2 >= 4) go(b_c, std::integral_constant<int, 4>{}, w_c);
    else if (mg2 == 2) go(b_c, std::integral_constant<int, 2>{}, w_c);
    else go(b_c, std::integral_constant<int, 1>{}, w_c);
  };
  auto with_bits = [&](auto w_c) {
    switch (bits) {
      case 4: with_mg(std::integral_constant<int, 4>{}, w_c); break;
      case 3: with_mg(std::integral_constant<int, 3>{}, w_c); break;
      case 2: with_mg(std::integral_constant<int, 2>{}, w_c); break;
      default: with_mg(std::integral_constant<int, 0>{}, w_c); break;
    }
  };
  if (a.g.N == 1024) with_bits(std::integral_constant<int, 8>{});
  else with_bits(std::integral_constant<int, 4>{});
}

void launch_debug_decode(const uint16_t* matrix_words, int bits, int K, int N, int as_e4m3, void* out,
                         hipStream_t s) {
  const int units = (K / 32) * (N / 16);
  const dim3 grid((units + 3) / 4), block(256);
  if (bits == 4) hipLaunchKernelGGL(k_debug_decode<4>, grid, block, 0, s, matrix_words, K, N, as_e4m3, out);
  else if (bits == 3) hipLaunchKernelGGL(k_debug_decode<3>, grid, block, 0, s, matrix_words, K, N, as_e4m3, out);
  else if (bits == 5) hipLaunchKernelGGL(k_debug_decode<5>, grid, block, 0, s, matrix_words, K, N, as_e4m3, out);
  else if (bits == 6) hipLaunchKernelGGL(k_debug_decode<6>, grid, block, 0, s, matrix_words, K, N, as_e4m3, out);
  else hipLaunchKernelGGL(k_debug_decode<2>, grid, block, 0, s, matrix_words, K, N, as_e4m3, out);
}

}  // namespace tmoe
