/* tmoe.h -- C ABI of the trellis-quantized routed mixture-of-experts layer for MI355X (gfx950).
 *
 * The layer (per route r = t*top_k + j, expert e = ids[t][j]):
 *   a = R_H(su1_e * x_t)                               input sign + rotation
 *   z = scale1_e * (C1_e^T a)        C1_e: H x 2I      FC1, gate columns first
 *   g = sv1_e[0:I] * R_I(z[0:I]);  u = sv1_e[I:2I] * R_I(z[I:2I])
 *   b = R_I(su2_e * (silu(g) * u))                     activation + intermediate rotation
 *   v = scale2_e * (C2_e^T b)        C2_e: I x H       FC2
 *   y_t = sum over j ascending of w[t][j] * (sv2_e * R_H(v))
 * Sources: "serve canonical Fruit QSRT atoms" (b12x PR #129), Hot path: one fused rotation +
 * quantization launch, a route map built once and consumed by FC1 and FC2, route-major FC1 and
 * FC2 with exact top-k weighting, W4A8 decode straight into E4M3 matrix operands;
 * "integrate EXL3 Trellis into the fused W4A16 API" (sparkinfer PR #90), reviews of kernel.py
 * (activation epilogue H128 -> svh -> silu -> suh_down -> H128, FP32 routed output) and of
 * prepare.py (trellis3_t256 tiles).
 *
 * R_n is the orthonormal Walsh-Hadamard transform in natural order: one block when n is a power
 * of two, otherwise 128-point blocks plus one 64-point block.
 *
 * Weight format. Each expert stores C1 (H x 2I) then C2 (I x H) as 16x16 tiles; tile (kt, nt)
 * of a K x N matrix is tile number kt*(N/16)+nt and holds 16*bits 16-bit words. Element i of a
 * tile is (k = i mod 16, n = i div 16). Stream bit j is bit 15-(j mod 16) of word j div 16; the
 * state of element i is the 16 bits ending at stream bit (i+1)*bits (MSB first, modulo
 * 256*bits). A state s decodes to the fp16 value h(lo16(m)) + h(hi16(m)), rounded to nearest
 * even, where m = ((s*0xCBAC1FED mod 2^32) & 0x8fff8fff) | 0x3b603b60 (codebook constants from
 * the sparkinfer PR #90 review of intrinsics.py). Experts are concatenated in index order.
 *
 * Conventions for every entry point:
 *  - Every function returns tmoe_status. Arguments are validated on the host before anything is
 *    enqueued, so on error nothing has been launched and no output or scratch byte is touched
 *    ("fail closed", b12x PR #129 Summary).
 *  - Device pointers are caller-owned; the library never allocates device or pinned memory and
 *    never synchronizes. Work is enqueued on `stream` (a hipStream_t; NULL = the null stream).
 *    The forward calls are safe to capture into a hipGraph.
 *  - fp16 arrays are IEEE binary16 bit patterns (uint16_t); x is bfloat16 bit patterns.
 *  - Scratch: one caller-owned device arena of at least the planned byte count, 16-byte
 *    aligned (the arena rule of "TrellisMX (procedural NPK) ... P8 runtime", flashinfer PR #69,
 *    description: a short or misaligned arena is rejected). Its contents need not be
 *    initialised; every byte a call reads is written earlier in that call. Two calls that
 *    share one scratch arena must not overlap in time.
 *  - ids outside [0, num_experts) do not fault: the route is dropped, contributes zero to y, and
 *    is counted in the route map's status word (readable after the stream completes).
 */
#ifndef TMOE_H
#define TMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TMOE_OK = 0,
  TMOE_ERR_INVALID_ARG = 1,   /* null pointer, bad dimension or enum, T < 0 */
  TMOE_ERR_UNSUPPORTED = 2,   /* a shape or bit width this library does not implement */
  TMOE_ERR_SCRATCH = 3,       /* scratch shorter than planned, or not 16-byte aligned */
  TMOE_ERR_CAPACITY = 4,      /* T > max_tokens of the plan */
  TMOE_ERR_ALIGNMENT = 5,     /* a device pointer not aligned as documented */
  TMOE_ERR_HIP = 6,           /* a HIP launch reported an error */
  TMOE_ERR_STATIC_SCRATCH = 7 /* plan needs more than TMOE_STATIC_SCRATCH_BYTES (static entry point) */
} tmoe_status;

/* Size of the library-owned scratch arena of tmoe_forward_w4a16_static, per GPU (32 MiB). */
#define TMOE_STATIC_SCRATCH_BYTES (32u << 20)

enum { TMOE_ROT_HADAMARD = 0, TMOE_ROT_IDENTITY = 1 };   /* identity: every R_n = I (test mode) */
enum { TMOE_IDS_I32 = 0, TMOE_IDS_I64 = 1 };             /* 32- or 64-bit ids (flashinfer PR #69)  */

typedef struct {
  int32_t hidden;              /* H: multiple of 64, 64..4096; power of two or 128*q (+64)  */
  int32_t inter;               /* I: same rules as H                                          */
  int32_t num_experts;         /* E: 1..512                                                   */
  int32_t top_k;               /* k: 1..32                                                    */
  int32_t max_tokens;          /* capacity T_max >= 1; T*k <= 2^24                            */
  const uint8_t *expert_bits;  /* host array [E], each 2..6 (W4A8: 2..4); copied by tmoe_plan  */
  int32_t rotation;            /* TMOE_ROT_HADAMARD or TMOE_ROT_IDENTITY                       */
  int32_t ids_dtype;           /* TMOE_IDS_I32 or TMOE_IDS_I64                                 */
  int32_t block_m;             /* route-map tile rows: 8, 16, 32, 48 or 64; 0 = 16             */
  int32_t smallm_max_tokens;   /* forwards with T <= this run as one persistent launch (the
                                  small-M arm of flashinfer PR #69, whose default is 16); 0 = never.
                                  Needs T*top_k <= 512 and H, I in {128, 256, 512, 1024} or not a
                                  power of two; other calls take the five-launch path.          */
  int32_t fc2_reduce;          /* TMOE_FC2_DETERMINISTIC (0) or TMOE_FC2_ATOMIC (1)             */
} tmoe_config;

/* FC2 reduction of the forwards: the deterministic route-major epilogue (bitwise reproducible), or
 * the opt-in FP32-atomic sum into y ("Share trellis preparation across native and EXL3
 * containers", b12x PR #433: optional FP32 atomic prefill reduction, which gives up bitwise
 * summation order). */
enum { TMOE_FC2_DETERMINISTIC = 0, TMOE_FC2_ATOMIC = 1 };

typedef struct tmoe_plan_s *tmoe_plan_t;   /* opaque, host-only, immutable, shareable across threads */

typedef struct {                 /* device pointers, read only */
  const uint16_t *payload;       /* all experts' trellis words; 16-byte aligned                 */
  const uint16_t *scale1;        /* fp16 [E][2I] FC1 output-channel scales                      */
  const uint16_t *scale2;        /* fp16 [E][H]  FC2 output-channel scales                      */
  const uint16_t *su1;           /* fp16 [E][H]  FC1 input signs                                */
  const uint16_t *sv1;           /* fp16 [E][2I] FC1 output signs (gate | up)                   */
  const uint16_t *su2;           /* fp16 [E][I]  FC2 input signs                                */
  const uint16_t *sv2;           /* fp16 [E][H]  FC2 output signs                               */
} tmoe_weights;

typedef struct {                 /* device pointers into the caller's scratch (set by the library) */
  int32_t *counts;               /* [E] valid routes per expert                                  */
  int32_t *offsets;              /* [E+1] exclusive prefix of counts                             */
  int32_t *sorted_routes;        /* [T*k]: slot p -> route r, stable token-major within an expert */
  int32_t *route_slot;           /* [T*k]: route r -> slot p, -1 for a dropped (invalid) route    */
  int32_t *tile_expert;          /* [max_tiles] expert of each block_m tile, expert-major         */
  int32_t *tile_row0;            /* [max_tiles] first slot of each tile                          */
  int32_t *tile_rows;            /* [max_tiles] rows of each tile, 1..block_m                    */
  int32_t *num_tiles;            /* [1]                                                          */
  int32_t *status;               /* [1] number of dropped routes (ids outside [0, E))            */
  int32_t max_tiles;             /* capacity of the tile arrays                                  */
  int32_t block_m;
} tmoe_route_map;

typedef struct {                 /* sizes derived from a plan */
  size_t scratch_bytes;          /* arena size needed by any call with T <= max_tokens           */
  size_t payload_words;          /* 16-bit words of all experts' payload                         */
  int32_t block_m;
  int32_t max_tiles;
} tmoe_plan_info;

/* Validate a configuration and build a plan (host only: no HIP call, no device allocation).
 * The plan fixes the geometry, the per-expert widths and the token capacity once and declares the
 * size of the caller's scratch arena, so every later call is checked on the host and enqueues
 * kernels only ("TrellisMX (procedural NPK) ... P8 runtime", flashinfer PR #69, description: the
 * plan/arena split with a declared arena size, int32 or int64 ids, smallm_max_tokens; b12x PR
 * #129 Summary: caller-owned storage, fail closed). The tile rule of 16*bits words per 16x16 tile
 * and the widths follow the sparkinfer PR #90 reviews of prepare.py and kernel.py. Configuration
 * errors: INVALID_ARG (null or out-of-range field), UNSUPPORTED (a shape or width this library
 * does not implement). The plan is owned by the caller until tmoe_plan_destroy.
 * scratch_bytes / payload_words may be NULL. */
tmoe_status tmoe_plan(const tmoe_config *cfg, tmoe_plan_t *out, size_t *scratch_bytes,
                      size_t *payload_words);
tmoe_status tmoe_plan_destroy(tmoe_plan_t plan);
tmoe_status tmoe_plan_get_info(tmoe_plan_t plan, tmoe_plan_info *info);
/* Word offset of expert e's region inside the payload. */
tmoe_status tmoe_plan_expert_offset(tmoe_plan_t plan, int32_t expert, size_t *word_offset);

/* Build the route map of T tokens (route map paragraph of b12x PR #129 Hot path; per-expert
 * counts and prefix offsets of the sparkinfer PR #90 route_pack.py review): a stable counting
 * sort of the T*k routes by expert, its inverse, and the block_m tile table. topk_ids is a
 * device array [T][k] of int32 or int64 (per the plan). view_out (host struct) receives device
 * pointers into scratch. One kernel launch; T = 0 launches nothing and leaves scratch alone. */
tmoe_status tmoe_build_route_map(tmoe_plan_t plan, const void *topk_ids, int32_t T, void *scratch,
                                 size_t scratch_bytes, tmoe_route_map *view_out, void *stream);

/* The layer with fp16 activations and trellis weights decoded to fp16 MFMA operands: the W4A16
 * routed MoE of "integrate EXL3 Trellis into the fused W4A16 API" (sparkinfer PR #90: Summary and
 * the kernel.py review for the epilogue order) with the launch structure of b12x PR #129 (Hot
 * path: one rotation + quantization launch, the route map reused by FC1 and FC2, route-major FC1
 * and FC2, exact top-k weighting into an FP32 output). Five launches on `stream`: route map with
 * the input rotation, FC1, activation with the intermediate rotation, FC2, output rotation with
 * the combine (one launch when the plan's smallm_max_tokens admits T).
 * x: bf16 [T][H] (16-byte aligned); topk_ids [T][k]; topk_w: fp32 [T][k]; y: fp32 [T][H]
 * (16-byte aligned), fully overwritten. Errors (nothing enqueued): INVALID_ARG (null pointer,
 * T < 0), CAPACITY (T > max_tokens), SCRATCH (arena short or misaligned), ALIGNMENT, HIP (a launch
 * failed). Deterministic with the default fc2_reduce: repeated calls give identical bits. */
tmoe_status tmoe_forward_w4a16(tmoe_plan_t plan, const void *x_bf16, const void *topk_ids,
                               const float *topk_w, int32_t T, const tmoe_weights *weights,
                               float *y, void *scratch, size_t scratch_bytes, void *stream);

/* Same layer with both rotated activations quantized to MXFP8 (E4M3 values, one E8M0 scale per
 * 32 along the contraction axis; exponent from the fp32 bits of amax/448, flashinfer PR #69
 * Precision notes) and trellis weights decoded straight to E4M3 operands of scaled-fp8 MFMA. */
tmoe_status tmoe_forward_w4a8(tmoe_plan_t plan, const void *x_bf16, const void *topk_ids,
                              const float *topk_w, int32_t T, const tmoe_weights *weights,
                              float *y, void *scratch, size_t scratch_bytes, void *stream);

/* tmoe_forward_w4a16 for callers that cannot allocate device memory (code under hipGraph capture,
 * tight serving loops, harnesses that forbid allocation): no scratch argument; the arena is a
 * device array of TMOE_STATIC_SCRATCH_BYTES that the library holds on each GPU it runs on, from
 * the first call on that GPU until the process ends. The call itself allocates nothing (the
 * array's device address is looked up once per GPU, on the first call there). Plans whose
 * scratch_bytes exceed TMOE_STATIC_SCRATCH_BYTES are rejected with TMOE_ERR_STATIC_SCRATCH before
 * anything is enqueued (a decode plan of H = 1024, I = 512, E = 96, top-8 needs 4.4 MiB at
 * max_tokens = 16 and 13.8 MiB at 64). Same kernels, same results, same checks as
 * tmoe_forward_w4a16. Every call on one GPU shares that GPU's array, whose contents are left by
 * the last call (no call reads a byte it has not written earlier in that call), so two calls that
 * overlap in time on one GPU -- on different streams, or from different threads -- race and must
 * not be issued. */
tmoe_status tmoe_forward_w4a16_static(tmoe_plan_t plan, const void *x_bf16, const void *topk_ids,
                                      const float *topk_w, int32_t T, const tmoe_weights *weights,
                                      float *y, void *stream);

/* Run only stages first..last (0 route map with the input rotation + quantize, 1 FC1,
 * 2 activation, 3 FC2, 4 output rotation + combine) of tmoe_forward_w4a16 (w4a8 = 0) or
 * tmoe_forward_w4a8 (w4a8 = 1), with that call's arguments and checks. A stage reads what the
 * earlier stages of a call with the same T, ids and precision left in scratch, so stages 0..4
 * issued in order, in one call or several, equal one forward call. Lets a caller put timing events between the launches. */
tmoe_status tmoe_forward_stages(tmoe_plan_t plan, int32_t w4a8, int32_t first, int32_t last,
                                const void *x_bf16, const void *topk_ids, const float *topk_w,
                                int32_t T, const tmoe_weights *weights, float *y, void *scratch,
                                size_t scratch_bytes, void *stream);

const char *tmoe_status_str(tmoe_status s);

/* ---- dense trellis linear: one trellis matrix, no routing ----
 * y_t = sv * R_N(scale * (C^T R_K(su * x_t))),  C: K x N in the layer's tile format and codebook.
 * Source: "integrate EXL3 Trellis into the fused W4A16 API" (sparkinfer PR #90) names a dense
 * trellis GEMM and a trellis_linear API beside the fused MoE, with the same tiles, codebook and
 * rotations; it prints no formula, so this is the layer's input rotation, one trellis contraction
 * with per-output-channel scales, and the layer's output rotation, with no routing and weight 1.
 * Runs the layer's kernels: one launch rotates x and writes the tables, then the grouped GEMM of a
 * single expert, then the output rotation (the combine with k = 1). */
typedef struct {
  int32_t in_features;         /* K: multiple of 64, 64..4096 (same rules as H)                 */
  int32_t out_features;        /* N: same rules                                                 */
  int32_t bits;                /* 2..6                                                          */
  int32_t max_tokens;          /* capacity T_max >= 1                                           */
  int32_t rotation;            /* TMOE_ROT_HADAMARD or TMOE_ROT_IDENTITY                         */
} tmoe_linear_config;

typedef struct tmoe_linear_plan_s *tmoe_linear_plan_t;   /* opaque, host-only, immutable */

typedef struct {                 /* device pointers, read only */
  const uint16_t *payload;       /* C: (K/16)*(N/16) tiles of 16*bits words; 16-byte aligned   */
  const uint16_t *scale;         /* fp16 [N] output-channel scales                             */
  const uint16_t *su;            /* fp16 [K] input signs                                       */
  const uint16_t *sv;            /* fp16 [N] output signs                                      */
} tmoe_linear_weights;

/* Validate and plan (host only). scratch_bytes / payload_words may be NULL. Errors: INVALID_ARG,
 * UNSUPPORTED. */
tmoe_status tmoe_linear_plan(const tmoe_linear_config *cfg, tmoe_linear_plan_t *out,
                             size_t *scratch_bytes, size_t *payload_words);
tmoe_status tmoe_linear_plan_destroy(tmoe_linear_plan_t plan);

/* x: bf16 [T][K] (16-byte aligned); y: fp32 [T][N] (16-byte aligned), fully overwritten. Scratch
 * rules as for the layer. T = 0 launches nothing. Deterministic; safe to capture in a hipGraph. */
tmoe_status tmoe_linear_w4a16(tmoe_linear_plan_t plan, const void *x_bf16, int32_t T,
                              const tmoe_linear_weights *weights, float *y, void *scratch,
                              size_t scratch_bytes, void *stream);

/* ---- test hooks: expose single steps so their bit-exactness can be graded ---- */

/* Decode expert `expert`'s FC1 (matrix 0, H x 2I) or FC2 (matrix 1, I x H) with the same device
 * decode the GEMMs use, into a dense row-major [K][N] array: fp16 codebook values (as_e4m3 = 0,
 * 2 bytes each) or their E4M3 roundings (as_e4m3 = 1, 1 byte each). out: device, 16-byte aligned. */
tmoe_status tmoe_debug_decode(tmoe_plan_t plan, const tmoe_weights *weights, int32_t expert,
                              int32_t matrix, int32_t as_e4m3, void *out, void *stream);

/* MXFP8-quantize rows x cols fp32 values (cols a multiple of 32) with the forward's quantizer:
 * q [rows][cols] E4M3 bytes, e8m0 [rows][cols/32]. All device pointers. */
tmoe_status tmoe_debug_mxfp8(const float *in, int64_t rows, int32_t cols, uint8_t *q,
                             uint8_t *e8m0, void *stream);

/* Apply the rotation R_n of the forward's kernels to rows x n fp32 values in place (device). */
tmoe_status tmoe_debug_rotate(float *rows_data, int64_t rows, int32_t n, void *stream);

typedef struct {                 /* where a forward call leaves its intermediates, for tests */
  void *a1;                      /* [T*k][a1_pitch] fp16 (W4A16) or E4M3 bytes (W4A8), route order
                                    (row t*k + j); the first H entries of each row are the rotated
                                    input                                                          */
  uint8_t *a1_scale;             /* [T*k][H/32] E8M0 (W4A8), route order                         */
  float *z;                      /* [splits[0]][T*k][2I] fp32 FC1 partial sums, unscaled, slot order;
                                    where half_planes[0] is 1 instead one fp16 plane [T*k][2I] of
                                    the finished sums times scale1                                  */
  void *b;                       /* [T*k][b_pitch] fp16 or E4M3, slot order (first I entries used) */
  uint8_t *b_scale;              /* [T*k][I/32] E8M0 (W4A8)                                      */
  float *v;                      /* [splits[1]][T*k][H] fp32 FC2 partial sums, unscaled, slot order;
                                    where half_planes[1] is 1 instead one fp16 plane [T*k][H] of
                                    the finished sums times scale2                                  */
  int32_t *splits;               /* device [2]: K splits of FC1 and FC2 that the call used (the plan's
                                    choice for T; readable after the stream completes)             */
  int32_t a1_pitch, b_pitch;     /* row pitch of a1 and b in elements: H and I for W4A8; for W4A16
                                    padded so that rows do not all start on the same memory channel */
  int32_t *arm_status;           /* device [1]: 0 after a forward that ran as one persistent launch;
                                    1 if a wait of that launch gave up (its y is invalid), 2 if an
                                    earlier call on this arena failed so the launch did not run     */
  int32_t *half_planes;          /* device [2]: 1 where FC1 (FC2) left the fp16 plane described at z
                                    (v): calls with one K split on 128-row tiles                   */
} tmoe_debug_views;

/* Views of the intermediates a forward call with T tokens leaves in scratch; w4a8 names the
 * precision of that call (0 = tmoe_forward_w4a16, 1 = tmoe_forward_w4a8). */
tmoe_status tmoe_debug_get_views(tmoe_plan_t plan, int32_t T, int32_t w4a8, void *scratch,
                                 size_t scratch_bytes, tmoe_debug_views *out);

#ifdef __cplusplus
}
#endif
#endif /* TMOE_H */
