// tmoe_internal.hpp -- launch-argument structs and launchers shared by the host code and kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tmoe {

struct ExpertInfo;

struct RouteMapArgs {
  const void* ids;
  int ids64;
  int routes;               // T * k
  int num_experts;
  int block_m;              // exported tile table
  int gemm_rows;            // internal GEMM tile table
  long long words_per_bit;  // 3*H*I/16: payload words of one expert per bit of width
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted_routes;
  int32_t* route_slot;
  int32_t* tile_expert;
  int32_t* tile_row0;
  int32_t* tile_rows;
  int32_t* num_tiles;
  int32_t* status;
  int4* gtiles;             // (expert | bits << 24, first slot, rows, payload word offset >> 8)
  int32_t* num_gtiles;
  int32_t* splits;          // [2] K splits of FC1 and FC2, published for the consumers and tests
  int nsplit[2];            // the host's split counts
  int32_t* half;            // [2] 1 where that GEMM leaves one fp16 plane with its channel scale applied
  int nhalf[2];             //   (published like splits; null: not published)
  int32_t* slot_expert;     // [R]: expert of each slot, -1 past the filled slots
  int32_t* wg_counts;       // [workgroups][E + 1]: per-workgroup counts (large batches; E = invalid)
  ExpertInfo* einfo;
  uint32_t packed_bits[64]; // 4 bits per expert: its width
};

// Rotation of a row of n values: one power-of-two block (pow2 = true, EPL = n / 64 values per
// lane) or n / 128 blocks of 128 plus an optional 64-block.
struct RowRot {
  int n;
  int pow2;
  int nblk128;
  int tail64;
  int identity;
};

struct RotateArgs {          // a = R_H(su1_e * x_t) per route, fp16 or MXFP8, row = route index
  const uint16_t* x;         // bf16 [T][H]
  const void* ids;           // [T][k] expert ids (routes with an invalid id are skipped)
  int ids64;
  int top_k;
  int num_experts;
  const uint16_t* su1;       // [E][H]
  RowRot rot;
  void* a1;                  // fp16 [R][lda] or e4m3 [R][H]
  uint8_t* a1_scale;         // [R][H/32]
  int lda;                   // fp16 row pitch in elements (>= H)
  int routes;
  int split_segments;        // non-power-of-two H: one wavefront per (route, 128-block) instead of per route
};

struct ActArgs {             // b = R_I(su2 * silu(sv1g * R_I(z_g)) * (sv1u * R_I(z_u)))
  const float* z;            // [nsplit][R][2I] unscaled partial sums
  const uint16_t* z16 = nullptr;  // or (one K split): fp16 [R][2I], scale1 already applied
  int nsplit;                // FC1 K splits: 1, 2, 4 or 8
  const int32_t* slot_expert;  // [R]: expert of each slot, -1 past the filled slots
  const uint16_t* scale1;    // [E][2I]
  const uint16_t* sv1;       // [E][2I]
  const uint16_t* su2;       // [E][I]
  RowRot rot;                // n = I
  void* b;                   // fp16 [R][ldb] or e4m3 [R][I]
  uint8_t* b_scale;          // [R][I/32]
  int ldb;                   // fp16 row pitch in elements (>= I)
  int routes;
  float* y_zero;             // non-null: workgroups past the activation's also zero y (the atomic
  long long y_count;         //   FC2 reduction adds into it); y_count floats
  int act_blocks;            // workgroups of the activation itself
};

struct CombineArgs {         // y_t = sum_j w[t,j] * sv2_e * R_H(scale2_e * v_slot), j ascending
  const float* v;            // [nsplit][R][H] FC2 partial sums (read only)
  const uint16_t* v16 = nullptr;  // or (one K split): fp16 [R][H], scale2 already applied
  int nsplit;                // FC2 K splits: 1, 2, 4 or 8
  const void* ids;
  int ids64;
  const float* w;            // [T][k]
  const int32_t* route_slot; // [T][k]: slot of route (t, j), -1 if dropped
  int top_k;
  int tokens;
  int routes;                // R: row stride between split planes
  const uint16_t* scale2;    // [E][H]
  const uint16_t* sv2;       // [E][H]
  RowRot rot;                // n = H
  float* y;                  // [T][H]
  int split_segments;        // non-power-of-two H: a workgroup (1) or a wavefront (0) per (token, block)
};

struct GemmArgs {            // out[s][slot][n] = sum over k in split s of A[slot][k] * C_e[k][n]
  const uint16_t* payload;
  const ExpertInfo* einfo;
  long long fc2_words_per_bit;  // FC2 region starts after H*2I*bits/16 words: pass H*2I/16 or 0
  const void* a;             // fp16 [rows][lda] or e4m3 [rows][K]
  const int32_t* arow;       // operand row of each slot (FC1: the slot's route), or null: row = slot
  const uint8_t* a_scale;    // [R][K/32] (fp8 only)
  float* out;                // [splits][R][N]
  uint16_t* out16 = nullptr; // fp16 GEMMs with one K split may instead leave fp16 [R][N] of
  const uint16_t* oscale = nullptr;  //   out * oscale[e][n] (the channel scale, [E][N]), rounded once
  const int4* gtiles;
  const int32_t* num_gtiles;
  int max_gtiles = 1;        // entries the tile list has room for
  int nsplit;                // K splits of this GEMM (the host's choice, also published in splits[])
  int K, N;
  int lda;                   // fp16 A row pitch in elements (the fp8 kernels use K)
  int routes;                // R: row stride between split planes
};

struct Fc2AtomicArgs {        // y_t += w[t,j] * sv2_e * R_H(scale2_e * (C2_e^T b_slot)), added atomically
  GemmArgs g;                // FC2 operands: b rows by slot, the GEMM tile list, K = I, N = H (out unused)
  const int32_t* sorted_routes;   // slot -> route
  const void* ids;
  int ids64;
  const float* w;            // [T][k]
  const uint16_t* scale2;    // [E][H]
  const uint16_t* sv2;       // [E][H]
  int identity;              // rotation off (test mode)
  int top_k;
  int tile_rows;             // rows of a GEMM tile (16 * mg)
  int sub_rows;              // rows of one unit: 16 * MG (MG = 1, 2 or 4 row groups)
  float* y;                  // [T][H], zeroed earlier in the forward
};

struct LinearPrepArgs {      // dense trellis linear: a = R_K(su * x_t) per token, plus the tables the
                             // grouped GEMM and the combine read (one expert, one route per token)
  RotateArgs rot;            // x, su1 = su, rot (n = K), a1, lda, routes = T; ids unused
  int4* gtiles;              // ceil(T / tile_rows) tiles of expert 0
  int32_t* num_gtiles;
  int32_t* slot;             // [T] t
  int32_t* ids;              // [T] 0
  float* w;                  // [T] 1
  int tokens, tile_rows, bits;
  int rot_blocks;            // workgroups of rotation items; the rest write the tables
};

// GEMM width code for experts of mixed widths that include 5 or 6 (0: mixed widths 2-4)
constexpr int kMixedWide = 7;

// The small-batch arm (one persistent launch for the whole layer): at most kArmMaxRoutes routes
// per call; flags and counters in kArmSlots library-owned slots per GPU, one per scratch arena.
constexpr int kArmMaxRoutes = 512;
constexpr int kArmSlots = 64;
struct ArmSlot;

struct ArmArgs {
  const uint16_t* x;         // bf16 [T][H]
  const void* ids;           // [T][K]
  int ids64;
  const float* w;            // [T][K]
  const uint16_t* payload;
  const uint16_t *scale1, *scale2, *su1, *sv1, *su2, *sv2;
  float* y;                  // [T][H]
  int T, H, I, E, K, R;      // R = T * K
  RowRot rot_h, rot_i;
  long long words_per_bit;   // 3*H*I/16: payload words of one expert per bit of width
  long long fc2_words_per_bit;   // 2*H*I/16: FC1 words per bit (FC2 starts after them)
  int s1, s2;                // K splits of FC1 and FC2
  uint8_t* a1;               // fp16 [R][lda] or E4M3 [R][H] (route order)
  uint8_t* a1s;              // E8M0 [R][H/32]
  int lda;
  float* z;                  // [s1][R][2I] (slot order)
  uint8_t* b;                // fp16 [R][ldb] or E4M3 [R][I] (slot order)
  uint8_t* bs;               // E8M0 [R][I/32]
  int ldb;
  float* v;                  // [s2][R][H] (slot order)
  int32_t* status;           // dropped routes
  int32_t* arm_status;       // 0, or 1: a wait gave up in this call, 2: the slot failed earlier
  ArmSlot* slot;
  uint32_t packed_bits[64];  // 4 bits per expert: its width
};

// Slot of the arena and the largest co-resident grid of the arm's kernel on the current device;
// false if the arm cannot run (no free slot, a HIP query failed).
bool small_arm_prepare(const void* arena, int bits, bool mx, ArmSlot** slot, int* groups);
void launch_small_arm(const ArmArgs& a, int bits, bool mx, int groups, hipStream_t s);

// one workgroup for up to kRouteSingleMax routes, else a counting and a placement launch over
// workgroups of kRouteChunk routes each
constexpr int kRouteChunk = 1024;
constexpr int kRouteSingleMax = 4096;
// the route map and, in the same launch (extra workgroups, independent work), the input rotation
void launch_route_map(const RouteMapArgs& a, const RotateArgs* rot, bool mx, hipStream_t s);
void launch_act(const ActArgs& a, bool mx, hipStream_t s);
void launch_linear_prep(const LinearPrepArgs& a, hipStream_t s);
void launch_combine(const CombineArgs& a, hipStream_t s);
// fc: 1 or 2 (names the kernel); bits: the width shared by every expert (2, 3, 4) or 0 if mixed;
// mg: 16-row groups per GEMM tile (1, 2 or 4); waves: persistent wave count
void launch_gemm_f16(const GemmArgs& a, int fc, int bits, int mg, int waves, hipStream_t s);
void launch_gemm_f8(const GemmArgs& a, int fc, int bits, int mg, int waves, hipStream_t s);
// FC2 with the FP32-atomic reduction into y (H = 512 or 1024): workgroups of H/128 wavefronts,
// `groups` of them persistent over the (tile, row block, K split) units; mg2 = 16-row groups per unit.
void launch_fc2_atomic(const Fc2AtomicArgs& a, int bits, int mg2, int groups, hipStream_t s);

void launch_debug_decode(const uint16_t* matrix_words, int bits, int K, int N, int as_e4m3, void* out,
                         hipStream_t s);
void launch_debug_mxfp8(const float* in, long long rows, int cols, uint8_t* q, uint8_t* e8m0, hipStream_t s);
void launch_debug_rotate(float* data, long long rows, const RowRot& rot, hipStream_t s);

}  // namespace tmoe
