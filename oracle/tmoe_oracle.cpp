// tmoe_oracle.cpp -- plain float64 CPU reference of the trellis-quantized routed MoE layer.
//
// TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU-baseline leg
// load this library. The product path never calls it, and it shares no code, header, table
// or constant generator with the HIP library: every step here is written out from its
// definition, slowly and in float64.
//
// Sources (page title, section):
//  * "serve canonical Fruit QSRT atoms" (b12x PR #129), "Hot path": the input rotation,
//    the route map consumed by FC1 and FC2, route-major FC1/FC2, exact top-k weighting,
//    trellis payload decoded without dense reconstruction.
//  * "integrate EXL3 Trellis into the fused W4A16 API" (sparkinfer PR #90), review of
//    prepare.py: a trellis3_t256 tile of 256 weights is 16*bits 16-bit words; review of
//    intrinsics.py: the procedural codebook constants 0xCBAC1FED, 0x8fff8fff, 0x3b603b60;
//    review of kernel.py: the 128-point butterfly with scale 1/sqrt(128) and the activation
//    epilogue order "H128 -> svh -> silu -> suh_down -> H128"; review of route_pack.py:
//    per-expert counts, prefix offsets and routed blocks.
//  * "TrellisMX (procedural NPK) ... P8 runtime" (flashinfer PR #69), "Precision notes":
//    the UE8M0 exponent is taken from the exact fp32 bits of amax/448; one scale byte per 32.
//
// Readings where the pages are silent (each is also listed in the design notes):
//  R1 tile element i <-> (k = i mod 16, n = i div 16) inside a 16x16 tile (column-major);
//     tile (kt, nt) of a K x N matrix is tile number kt*(N/16)+nt; an expert's region is
//     FC1 (H x 2I, gate columns first) then FC2 (I x H); experts are concatenated.
//  R2 stream bit j is bit 15-(j mod 16) of word j div 16 (MSB first); the state of element
//     i is the 16 stream bits ending at bit (i+1)*bits, read MSB first, indices taken
//     modulo 256*bits (tail-biting).
//  R3 codebook: x = state*0xCBAC1FED mod 2^32, m = (x & 0x8fff8fff) | 0x3b603b60, value =
//     fp16 round-to-nearest-even of half(low 16 bits of m) + half(high 16 bits of m).
//  R4 R_n is the orthonormal Walsh-Hadamard transform in natural (Sylvester) order: one
//     block when n is a power of two, otherwise floor(n/128) blocks of 128 and one block of
//     n mod 128 (which must be a power of two).
//  R5 gate and up share one input sign vector su1; the intermediate sign row is
//     [sv1_gate | sv1_up | su2]; top-k weights are applied as given (no renormalisation).
//  R6 MXFP8: blocks of 32 along the contraction axis; e = ceil(log2(fp32(amax32/448)))
//     computed from the float's bits, clamped to [-127,127], -127 for zero/subnormal q;
//     element = e4m3 round-to-nearest-even (saturating at 448) of v / 2^e.
//  R7 the W4A8 layer is the W4A16 layer with both rotated activations (FC1 and FC2 inputs)
//     replaced by their MXFP8 quantize-dequantize, and each codebook value replaced by its
//     E4M3 rounding (weight scale byte 127, i.e. 1.0); channel scales apply after the sum.
//  R8 the dense trellis linear (sparkinfer PR #90 names a dense trellis GEMM and a trellis_linear
//     API next to the fused MoE, with the same tiles, codebook and rotations, but prints no
//     formula) is one trellis matrix C (K x N, R1-R3) between the layer's input rotation and its
//     output rotation, with no routing and weight 1: y_t = sv * R_N(scale * (C^T R_K(su * x_t))),
//     i.e. the FC1 input step, the FC2 contraction and scaling, and the combine's output step.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

// ---------------------------------------------------------------- number formats
double half_to_double(uint16_t h) {
  const int sign = h >> 15;
  const int ex = (h >> 10) & 0x1f;
  const int man = h & 0x3ff;
  double v;
  if (ex == 0) {
    v = std::ldexp(static_cast<double>(man), -24);
  } else if (ex == 31) {
    v = man ? NAN : INFINITY;
  } else {
    v = std::ldexp(static_cast<double>(man + 1024), ex - 25);
  }
  return sign ? -v : v;
}

// Round-to-nearest-even of an integer-valued scaled double (x = v / quantum).
double round_half_even(double x) {
  double f = std::floor(x);
  double d = x - f;
  if (d > 0.5) return f + 1.0;
  if (d < 0.5) return f;
  return (std::fmod(f, 2.0) == 0.0) ? f : f + 1.0;
}

// float64 -> IEEE binary16, round to nearest even, overflow to infinity.
uint16_t double_to_half(double v) {
  if (std::isnan(v)) return 0x7e00;
  const uint16_t sign = std::signbit(v) ? 0x8000 : 0;
  double a = std::fabs(v);
  if (a == 0.0) return sign;
  int e;
  std::frexp(a, &e);                     // a = f * 2^e, f in [0.5, 1)
  int qexp = std::max(e - 11, -24);      // 11 significant bits; subnormal quantum 2^-24
  double n = round_half_even(std::ldexp(a, -qexp));
  double r = std::ldexp(n, qexp);
  if (r >= 65520.0) return sign | 0x7c00;
  if (r < std::ldexp(1.0, -14)) {
    return sign | static_cast<uint16_t>(std::ldexp(r, 24));
  }
  int re;
  double rf = std::frexp(r, &re);        // r = rf * 2^re
  uint16_t field = static_cast<uint16_t>(re + 14);
  uint16_t man = static_cast<uint16_t>(std::ldexp(rf * 2.0 - 1.0, 10));
  return sign | static_cast<uint16_t>(field << 10) | man;
}

// float64 -> E4M3 (fn variant: bias 7, max normal 448, no infinities), round to nearest
// even, saturating to +-448.
uint8_t double_to_e4m3(double v) {
  const uint8_t sign = std::signbit(v) ? 0x80 : 0;
  double a = std::fabs(v);
  if (a == 0.0) return sign;
  int e;
  std::frexp(a, &e);
  int qexp = std::max(e - 4, -9);        // 4 significant bits; subnormal quantum 2^-9
  double n = round_half_even(std::ldexp(a, -qexp));
  double r = std::ldexp(n, qexp);
  if (r > 448.0) r = 448.0;
  if (r == 0.0) return sign;
  if (r < std::ldexp(1.0, -6)) {
    return sign | static_cast<uint8_t>(std::ldexp(r, 9));
  }
  int re;
  double rf = std::frexp(r, &re);
  uint8_t field = static_cast<uint8_t>(re + 6);
  uint8_t man = static_cast<uint8_t>(std::ldexp(rf * 2.0 - 1.0, 3));
  return sign | static_cast<uint8_t>(field << 3) | man;
}

double e4m3_to_double(uint8_t b) {
  const int sign = b >> 7;
  const int ex = (b >> 3) & 0xf;
  const int man = b & 7;
  double v;
  if (ex == 0) {
    v = std::ldexp(static_cast<double>(man), -9);
  } else if (ex == 15 && man == 7) {
    v = NAN;
  } else {
    v = std::ldexp(static_cast<double>(man + 8), ex - 10);
  }
  return sign ? -v : v;
}

double bf16_to_double(uint16_t b) {
  uint32_t u = static_cast<uint32_t>(b) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return static_cast<double>(f);
}

// ---------------------------------------------------------------- trellis codebook
uint16_t codebook(uint16_t state) {
  uint32_t x = static_cast<uint32_t>(state) * 0xCBAC1FEDu;  // mod 2^32 by unsigned wrap
  uint32_t m = (x & 0x8fff8fffu) | 0x3b603b60u;
  double lo = half_to_double(static_cast<uint16_t>(m & 0xffffu));
  double hi = half_to_double(static_cast<uint16_t>(m >> 16));
  return double_to_half(lo + hi);        // exact sum in float64, one rounding to fp16
}

// Stream bit j of a tile (R2): bit 15 - (j mod 16) of word j / 16, j taken modulo 256*bits.
int stream_bit(const uint16_t* words, int bits, long j) {
  const long len = 256L * bits;
  j %= len;
  if (j < 0) j += len;
  return (words[j / 16] >> (15 - (j % 16))) & 1;
}

// Decoder 1: read each element's 16-bit window bit by bit.
void decode_tile_bitwise(const uint16_t* words, int bits, uint16_t* states) {
  for (int i = 0; i < 256; ++i) {
    long end = static_cast<long>(i + 1) * bits;
    uint16_t s = 0;
    for (long j = end - 16; j < end; ++j) s = static_cast<uint16_t>((s << 1) | stream_bit(words, bits, j));
    states[i] = s;
  }
}

// Decoder 2: a 16-bit shift register seeded with the last 16 bits of the stream, shifted
// by `bits` new bits per element.
void decode_tile_shiftreg(const uint16_t* words, int bits, uint16_t* states) {
  const long len = 256L * bits;
  uint32_t reg = 0;
  for (long j = len - 16; j < len; ++j) reg = ((reg << 1) | stream_bit(words, bits, j)) & 0xffffu;
  for (int i = 0; i < 256; ++i) {
    for (int b = 0; b < bits; ++b) {
      reg = ((reg << 1) | stream_bit(words, bits, static_cast<long>(i) * bits + b)) & 0xffffu;
    }
    states[i] = static_cast<uint16_t>(reg);
  }
}

// Decode one K x N trellis matrix (R1) into fp16 codebook values, row-major [K][N].
void decode_matrix(const uint16_t* mat_words, int bits, int K, int N, uint16_t* codes) {
  uint16_t states[256];
  const int ntn = N / 16;
  for (int kt = 0; kt < K / 16; ++kt) {
    for (int nt = 0; nt < ntn; ++nt) {
      const uint16_t* tile = mat_words + static_cast<size_t>(kt * ntn + nt) * 16 * bits;
      decode_tile_shiftreg(tile, bits, states);
      for (int i = 0; i < 256; ++i) {
        int k = kt * 16 + (i % 16);
        int n = nt * 16 + (i / 16);
        codes[static_cast<size_t>(k) * N + n] = codebook(states[i]);
      }
    }
  }
}

// ---------------------------------------------------------------- rotation R_n (R4)
bool is_pow2(int n) { return n > 0 && (n & (n - 1)) == 0; }

// Block decomposition of n: fills (offset, size) pairs; returns false if unsupported.
bool hadamard_blocks(int n, std::vector<std::pair<int, int>>* blocks) {
  blocks->clear();
  if (n <= 0) return false;
  if (is_pow2(n)) {
    blocks->push_back({0, n});
    return true;
  }
  int q = n / 128, r = n % 128;
  for (int b = 0; b < q; ++b) blocks->push_back({128 * b, 128});
  if (r) {
    if (!is_pow2(r)) return false;
    blocks->push_back({128 * q, r});
  }
  return true;
}

// In-place butterfly transform of each block, then scaling by 1/sqrt(block size).
void rotate(double* v, int n, bool identity) {
  if (identity) return;
  std::vector<std::pair<int, int>> blocks;
  hadamard_blocks(n, &blocks);
  for (auto [off, b] : blocks) {
    double* p = v + off;
    for (int h = 1; h < b; h *= 2) {
      for (int i = 0; i < b; i += 2 * h) {
        for (int j = i; j < i + h; ++j) {
          double x = p[j], y = p[j + h];
          p[j] = x + y;
          p[j + h] = x - y;
        }
      }
    }
    double s = 1.0 / std::sqrt(static_cast<double>(b));
    for (int j = 0; j < b; ++j) p[j] *= s;
  }
}

// ---------------------------------------------------------------- MXFP8 (R6)
int mx_exponent(float amax) {
  float q = amax / 448.0f;               // one fp32 division, round to nearest even
  uint32_t u;
  std::memcpy(&u, &q, 4);
  int field = static_cast<int>((u >> 23) & 0xff);
  uint32_t man = u & 0x7fffffu;
  if (field == 0) return -127;           // zero or subnormal quotient
  int e = field - 127 + (man != 0 ? 1 : 0);
  return std::min(127, std::max(-127, e));
}

// Quantize one block of n values in place to its dequantized MXFP8 values.
void mx_qdq_block(double* v, int n, uint8_t* q_out, uint8_t* e_out) {
  double amax = 0.0;
  for (int i = 0; i < n; ++i) amax = std::max(amax, std::fabs(v[i]));
  int e = mx_exponent(static_cast<float>(amax));
  if (e_out) *e_out = static_cast<uint8_t>(e + 127);
  for (int i = 0; i < n; ++i) {
    uint8_t c = double_to_e4m3(std::ldexp(v[i], -e));
    if (q_out) q_out[i] = c;
    v[i] = std::ldexp(e4m3_to_double(c), e);
  }
}

void mx_qdq_row(double* v, int n) {
  for (int b = 0; b < n; b += 32) mx_qdq_block(v + b, 32, nullptr, nullptr);
}

double silu(double v) { return v / (1.0 + std::exp(-v)); }

// ---------------------------------------------------------------- layer
struct Layer {
  int T, H, I, E, K;
  const uint8_t* bits;
  const uint16_t* payload;
  const uint16_t *scale1, *scale2, *su1, *sv1, *su2, *sv2;
  const uint16_t* x;
  const int64_t* ids;
  const float* w;
  int w4a8;
  int identity;
  std::vector<int64_t> offsets;          // word offset of each expert
};

struct ExpertDense {
  std::vector<double> c1;                // [H][2I] codebook values (E4M3-rounded in W4A8)
  std::vector<double> c2;                // [I][H]
};

void decode_expert(const Layer& L, int e, ExpertDense* d) {
  const int H = L.H, I = L.I, bits = L.bits[e];
  std::vector<uint16_t> codes1(static_cast<size_t>(H) * 2 * I), codes2(static_cast<size_t>(I) * H);
  const uint16_t* base = L.payload + L.offsets[e];
  decode_matrix(base, bits, H, 2 * I, codes1.data());
  decode_matrix(base + static_cast<size_t>(H) * 2 * I * bits / 16, bits, I, H, codes2.data());
  d->c1.resize(codes1.size());
  d->c2.resize(codes2.size());
  for (size_t i = 0; i < codes1.size(); ++i) {
    double c = half_to_double(codes1[i]);
    d->c1[i] = L.w4a8 ? e4m3_to_double(double_to_e4m3(c)) : c;
  }
  for (size_t i = 0; i < codes2.size(); ++i) {
    double c = half_to_double(codes2[i]);
    d->c2[i] = L.w4a8 ? e4m3_to_double(double_to_e4m3(c)) : c;
  }
}

struct RouteTrace {                      // every intermediate of one route, for tests
  std::vector<double> a, z, g, u, h, b, v, o;
};

// One route: token t, expert e. Steps in the pages' order (see the file header).
void route_forward(const Layer& L, const ExpertDense& d, int t, int e, RouteTrace* tr) {
  const int H = L.H, I = L.I;
  tr->a.assign(H, 0.0);
  for (int k = 0; k < H; ++k) {
    tr->a[k] = half_to_double(L.su1[static_cast<size_t>(e) * H + k]) *
               bf16_to_double(L.x[static_cast<size_t>(t) * H + k]);
  }
  rotate(tr->a.data(), H, L.identity);
  if (L.w4a8) mx_qdq_row(tr->a.data(), H);

  tr->z.assign(2 * I, 0.0);
  for (int k = 0; k < H; ++k) {
    const double ak = tr->a[k];
    const double* row = d.c1.data() + static_cast<size_t>(k) * 2 * I;
    for (int n = 0; n < 2 * I; ++n) tr->z[n] += ak * row[n];
  }
  for (int n = 0; n < 2 * I; ++n) tr->z[n] *= half_to_double(L.scale1[static_cast<size_t>(e) * 2 * I + n]);

  tr->g.assign(tr->z.begin(), tr->z.begin() + I);
  tr->u.assign(tr->z.begin() + I, tr->z.end());
  rotate(tr->g.data(), I, L.identity);
  rotate(tr->u.data(), I, L.identity);
  tr->h.assign(I, 0.0);
  tr->b.assign(I, 0.0);
  for (int n = 0; n < I; ++n) {
    tr->g[n] *= half_to_double(L.sv1[static_cast<size_t>(e) * 2 * I + n]);
    tr->u[n] *= half_to_double(L.sv1[static_cast<size_t>(e) * 2 * I + I + n]);
    tr->h[n] = silu(tr->g[n]) * tr->u[n];
    tr->b[n] = half_to_double(L.su2[static_cast<size_t>(e) * I + n]) * tr->h[n];
  }
  rotate(tr->b.data(), I, L.identity);
  if (L.w4a8) mx_qdq_row(tr->b.data(), I);

  tr->v.assign(H, 0.0);
  for (int n = 0; n < I; ++n) {
    const double bn = tr->b[n];
    const double* row = d.c2.data() + static_cast<size_t>(n) * H;
    for (int m = 0; m < H; ++m) tr->v[m] += bn * row[m];
  }
  for (int m = 0; m < H; ++m) tr->v[m] *= half_to_double(L.scale2[static_cast<size_t>(e) * H + m]);

  tr->o = tr->v;
  rotate(tr->o.data(), H, L.identity);
  for (int m = 0; m < H; ++m) tr->o[m] *= half_to_double(L.sv2[static_cast<size_t>(e) * H + m]);
}

int setup_layer(Layer* L) {
  if (L->T < 0 || L->H <= 0 || L->I <= 0 || L->E <= 0 || L->K <= 0) return -1;
  if (L->H % 32 || L->I % 32) return -1;
  std::vector<std::pair<int, int>> blocks;
  if (!hadamard_blocks(L->H, &blocks) || !hadamard_blocks(L->I, &blocks)) return -2;
  L->offsets.assign(L->E + 1, 0);
  for (int e = 0; e < L->E; ++e) {
    int b = L->bits[e];
    if (b < 1 || b > 16) return -3;
    L->offsets[e + 1] = L->offsets[e] + static_cast<int64_t>(3) * L->H * L->I * b / 16;
  }
  return 0;
}

int worker_count(int requested) {
  int hc = static_cast<int>(std::thread::hardware_concurrency());
  if (hc <= 0) hc = 1;
  return requested > 0 ? requested : hc;
}

}  // namespace

extern "C" {

uint16_t orc_codebook_fp16(uint16_t state) { return codebook(state); }
double orc_half_to_double(uint16_t h) { return half_to_double(h); }
uint16_t orc_double_to_half(double v) { return double_to_half(v); }
uint8_t orc_double_to_e4m3(double v) { return double_to_e4m3(v); }
double orc_e4m3_to_double(uint8_t b) { return e4m3_to_double(b); }
int orc_mx_exponent(float amax) { return mx_exponent(amax); }
int orc_hardware_threads(void) { return worker_count(0); }

void orc_decode_tile_bitwise(const uint16_t* words, int bits, uint16_t* states) {
  decode_tile_bitwise(words, bits, states);
}
void orc_decode_tile_shiftreg(const uint16_t* words, int bits, uint16_t* states) {
  decode_tile_shiftreg(words, bits, states);
}
void orc_decode_matrix(const uint16_t* mat_words, int bits, int K, int N, uint16_t* codes) {
  decode_matrix(mat_words, bits, K, N, codes);
}

// Explicit blocked matrix R_n, by its definition (R4): entry (i, j) inside a block of size b
// is b^-1/2 * (-1)^popcount(i & j) in block coordinates, zero across blocks. Row-major [n][n].
int orc_hadamard_explicit(int n, double* out) {
  std::vector<std::pair<int, int>> blocks;
  if (!hadamard_blocks(n, &blocks)) return -1;
  std::fill(out, out + static_cast<size_t>(n) * n, 0.0);
  for (auto [off, b] : blocks) {
    double s = 1.0 / std::sqrt(static_cast<double>(b));
    for (int i = 0; i < b; ++i)
      for (int j = 0; j < b; ++j)
        out[static_cast<size_t>(off + i) * n + off + j] = (__builtin_popcount(i & j) & 1) ? -s : s;
  }
  return 0;
}

// Butterfly R_n applied to each of `rows` rows of length n, in place.
int orc_rotate_rows(double* v, int64_t rows, int n, int identity) {
  std::vector<std::pair<int, int>> blocks;
  if (!hadamard_blocks(n, &blocks)) return -1;
  for (int64_t r = 0; r < rows; ++r) rotate(v + r * n, n, identity != 0);
  return 0;
}

// Stable token-major route map (counting sort by expert; ties keep route order).
int orc_route_map(const int64_t* ids, int64_t R, int E, int block_m, int32_t* counts,
                  int32_t* offsets, int32_t* sorted_routes, int32_t* route_slot,
                  int32_t* tile_expert, int32_t* tile_row0, int32_t* tile_rows,
                  int32_t* num_tiles, int32_t* invalid) {
  if (E <= 0 || block_m <= 0 || R < 0) return -1;
  std::vector<int64_t> order;
  int32_t bad = 0;
  for (int64_t r = 0; r < R; ++r) {
    if (ids[r] < 0 || ids[r] >= E) {
      ++bad;
      route_slot[r] = -1;
    } else {
      order.push_back(r);
    }
  }
  std::stable_sort(order.begin(), order.end(), [&](int64_t a, int64_t b) { return ids[a] < ids[b]; });
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t r : order) ++counts[ids[r]];
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  for (size_t p = 0; p < order.size(); ++p) {
    sorted_routes[p] = static_cast<int32_t>(order[p]);
    route_slot[order[p]] = static_cast<int32_t>(p);
  }
  int32_t nt = 0;
  for (int e = 0; e < E; ++e) {
    for (int32_t r0 = 0; r0 < counts[e]; r0 += block_m) {
      tile_expert[nt] = e;
      tile_row0[nt] = offsets[e] + r0;
      tile_rows[nt] = std::min<int32_t>(block_m, counts[e] - r0);
      ++nt;
    }
  }
  *num_tiles = nt;
  *invalid = bad;
  return 0;
}

// MXFP8 quantization of rows x cols values (R6); cols must be a multiple of 32.
int orc_mxfp8_quantize(const double* in, int64_t rows, int cols, uint8_t* q, uint8_t* e8m0) {
  if (cols % 32) return -1;
  std::vector<double> tmp(32);
  for (int64_t r = 0; r < rows; ++r) {
    for (int b = 0; b < cols / 32; ++b) {
      std::copy(in + r * cols + b * 32, in + r * cols + b * 32 + 32, tmp.begin());
      mx_qdq_block(tmp.data(), 32, q + r * cols + b * 32, e8m0 + r * (cols / 32) + b);
    }
  }
  return 0;
}

// Dense trellis linear (R8). payload: C's K/16 * N/16 tiles of 16*bits words; scale, sv: fp16 [N];
// su: fp16 [K]; x: bf16 [T][K]; y: float64 [T][N]. Returns 0, or < 0 for an unsupported shape.
int orc_linear(int T, int K, int N, int bits, const uint16_t* payload, const uint16_t* scale,
               const uint16_t* su, const uint16_t* sv, const uint16_t* x, int identity, double* y) {
  if (T < 0 || K <= 0 || N <= 0 || K % 16 || N % 16 || bits < 1 || bits > 16) return -1;
  std::vector<std::pair<int, int>> blocks;
  if (!hadamard_blocks(K, &blocks) || !hadamard_blocks(N, &blocks)) return -2;
  std::vector<uint16_t> codes(static_cast<size_t>(K) * N);
  decode_matrix(payload, bits, K, N, codes.data());
  std::vector<double> c(codes.size());
  for (size_t i = 0; i < codes.size(); ++i) c[i] = half_to_double(codes[i]);
  std::vector<double> a(K), z(N);
  for (int t = 0; t < T; ++t) {
    for (int k = 0; k < K; ++k)
      a[k] = half_to_double(su[k]) * bf16_to_double(x[static_cast<size_t>(t) * K + k]);
    rotate(a.data(), K, identity != 0);
    std::fill(z.begin(), z.end(), 0.0);
    for (int k = 0; k < K; ++k) {
      const double* row = c.data() + static_cast<size_t>(k) * N;
      for (int n = 0; n < N; ++n) z[n] += a[k] * row[n];
    }
    for (int n = 0; n < N; ++n) z[n] *= half_to_double(scale[n]);
    rotate(z.data(), N, identity != 0);
    for (int n = 0; n < N; ++n) y[static_cast<size_t>(t) * N + n] = half_to_double(sv[n]) * z[n];
  }
  return 0;
}

// Full layer. y is [T][H] float64. mode 0 = W4A16, 1 = W4A8 (R7). identity != 0 replaces
// every R_n by the identity (a test mode). nthreads <= 0 uses every hardware thread.
int orc_forward(int T, int H, int I, int E, int K, const uint8_t* bits, const uint16_t* payload,
                const uint16_t* scale1, const uint16_t* scale2, const uint16_t* su1,
                const uint16_t* sv1, const uint16_t* su2, const uint16_t* sv2,
                const uint16_t* x_bf16, const int64_t* ids, const float* w, int mode,
                int identity, int nthreads, double* y) {
  Layer L{T, H, I, E, K, bits, payload, scale1, scale2, su1, sv1, su2, sv2, x_bf16, ids, w,
          mode, identity, {}};
  int rc = setup_layer(&L);
  if (rc) return rc;
  const int64_t R = static_cast<int64_t>(T) * K;
  for (int64_t r = 0; r < R; ++r)
    if (ids[r] < 0 || ids[r] >= E) return -4;
  std::vector<std::vector<int64_t>> by_expert(E);
  for (int64_t r = 0; r < R; ++r) by_expert[ids[r]].push_back(r);
  std::vector<double> o(static_cast<size_t>(R) * H, 0.0);
  std::atomic<int> next{0};
  auto work = [&]() {
    ExpertDense d;
    RouteTrace tr;
    for (int e = next++; e < E; e = next++) {
      if (by_expert[e].empty()) continue;
      decode_expert(L, e, &d);
      for (int64_t r : by_expert[e]) {
        route_forward(L, d, static_cast<int>(r / K), e, &tr);
        std::copy(tr.o.begin(), tr.o.end(), o.begin() + r * H);
      }
    }
  };
  int nw = std::min(worker_count(nthreads), std::max(1, E));
  std::vector<std::thread> pool;
  for (int i = 1; i < nw; ++i) pool.emplace_back(work);
  work();
  for (auto& th : pool) th.join();
  // Exact top-k combine: y_t = sum over j ascending of w[t, j] * o[t*K + j].
  for (int t = 0; t < T; ++t) {
    for (int m = 0; m < H; ++m) {
      double acc = 0.0;
      for (int j = 0; j < K; ++j) {
        acc += static_cast<double>(w[static_cast<size_t>(t) * K + j]) *
               o[(static_cast<size_t>(t) * K + j) * H + m];
      }
      y[static_cast<size_t>(t) * H + m] = acc;
    }
  }
  return 0;
}

// Every intermediate of one route (token t, slot j) for sampled checks at full size.
// Buffers: a[H] z[2I] h[I] b[I] v[H] o[H] (any may be null).
int orc_route_trace(int T, int H, int I, int E, int K, const uint8_t* bits, const uint16_t* payload,
                    const uint16_t* scale1, const uint16_t* scale2, const uint16_t* su1,
                    const uint16_t* sv1, const uint16_t* su2, const uint16_t* sv2,
                    const uint16_t* x_bf16, const int64_t* ids, int mode, int identity,
                    int t, int j, double* a, double* z, double* h, double* b, double* v, double* o) {
  Layer L{T, H, I, E, K, bits, payload, scale1, scale2, su1, sv1, su2, sv2, x_bf16, ids, nullptr,
          mode, identity, {}};
  int rc = setup_layer(&L);
  if (rc) return rc;
  if (t < 0 || t >= T || j < 0 || j >= K) return -5;
  int64_t e = ids[static_cast<int64_t>(t) * K + j];
  if (e < 0 || e >= E) return -4;
  ExpertDense d;
  decode_expert(L, static_cast<int>(e), &d);
  RouteTrace tr;
  route_forward(L, d, t, static_cast<int>(e), &tr);
  auto put = [](const std::vector<double>& s, double* dst) { if (dst) std::copy(s.begin(), s.end(), dst); };
  put(tr.a, a); put(tr.z, z); put(tr.h, h); put(tr.b, b); put(tr.v, v); put(tr.o, o);
  return 0;
}

}  // extern "C"
