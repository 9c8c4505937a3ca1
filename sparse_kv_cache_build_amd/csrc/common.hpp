// Device-side helpers shared by the kernels of libskv (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace skv {

constexpr int kWave = 64;
constexpr int kLshTok = 4096;       // tokens per workgroup of the soft-LSH scorer
constexpr int kLshMaxProj = 512;    // tables x hyperplanes per table (64 x 8)
constexpr int kLshMaxEntries = 16384;   // G x tables x 2^P bucket masses of one unit (64 KiB of LDS)

// Plain view of the paged cache passed by value to kernels.
// Operand and result vectors of the 16x16x32 bf16 matrix-core instruction.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte loads marked non-temporal, for data a kernel reads once per call (cache metadata, the
// rows of the selected tokens): the lines are not kept in the caches for reuse.
__device__ __forceinline__ uint4 ld_once(const uint4 *p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 ld_once(const float4 *p) {
  const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

struct CacheView {
  int32_t B, Hq, Hkv, D, S, maxP, Nphys, G;
  const void *k;
  const void *v;
  const int32_t *bt;    // [B, maxP]
  const int32_t *lens;  // [B]
};

// Valid length of sequence b, clamped to [0, maxP * S].
__device__ __forceinline__ int seq_len(const CacheView &c, int b) {
  int L = c.lens[b];
  int cap = c.maxP * c.S;
  return L < 0 ? 0 : (L > cap ? cap : L);
}

__device__ __forceinline__ int num_pages(const CacheView &c, int L) { return (L + c.S - 1) / c.S; }

// ---------------------------------------------------------------- element access
// Cache elements are float or bf16 (stored as uint16_t bit patterns). bf16 widens to f32 by a
// 16-bit shift, which is exact.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

template <typename T>
struct Elem;

template <>
struct Elem<float> {
  static __device__ __forceinline__ float get(const float *p, size_t i) { return p[i]; }
  // 8 consecutive elements (32-byte aligned)
  static __device__ __forceinline__ void load8(const float *p, float (&x)[8]) {
    float4 a = *reinterpret_cast<const float4 *>(p);
    float4 b = *reinterpret_cast<const float4 *>(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
};

template <>
struct Elem<uint16_t> {
  static __device__ __forceinline__ float get(const uint16_t *p, size_t i) { return bf16_f32(p[i]); }
  // 8 consecutive elements (16-byte aligned)
  static __device__ __forceinline__ void load8(const uint16_t *p, float (&x)[8]) {
    uint4 w = *reinterpret_cast<const uint4 *>(p);
    x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
    x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
  }
};

// 8 consecutive elements kept packed for the dot-product path: bf16 pairs as they are stored,
// float as is. dot8(q, k) = sum of the 8 products, accumulated in float32 (for bf16 with
// v_dot2c_f32_bf16: the bf16 x bf16 products are exact).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <typename T>
struct Packed8;

template <>
struct Packed8<uint16_t> {
  uint4 w;
  __device__ __forceinline__ void load(const uint16_t *p) { w = *reinterpret_cast<const uint4 *>(p); }
  __device__ __forceinline__ void load_once(const uint16_t *p) { w = ld_once(reinterpret_cast<const uint4 *>(p)); }
  __device__ __forceinline__ void zero() { w = make_uint4(0u, 0u, 0u, 0u); }
  // element j (0..7) as float; j is a compile-time constant after unrolling
  __device__ __forceinline__ float at(int j) const {
    const uint32_t x = j < 2 ? w.x : j < 4 ? w.y : j < 6 ? w.z : w.w;
    return (j & 1) ? bf16_hi(x) : bf16_lo(x);
  }
  __device__ __forceinline__ float dot(const Packed8 &k) const {
    float acc = 0.0f;
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.x), __builtin_bit_cast(bf16x2_t, k.w.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.y), __builtin_bit_cast(bf16x2_t, k.w.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.z), __builtin_bit_cast(bf16x2_t, k.w.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.w), __builtin_bit_cast(bf16x2_t, k.w.w), acc, false);
    return acc;
  }
};

template <>
struct Packed8<float> {
  float x[8];
  __device__ __forceinline__ void load(const float *p) { Elem<float>::load8(p, x); }
  __device__ __forceinline__ void load_once(const float *p) {
    const float4 a = ld_once(reinterpret_cast<const float4 *>(p)), b = ld_once(reinterpret_cast<const float4 *>(p + 4));
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = 0.0f;
  }
  __device__ __forceinline__ float at(int j) const { return x[j]; }
  __device__ __forceinline__ float dot(const Packed8 &k) const {
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = fmaf(x[j], k.x[j], acc);
    return acc;
  }
};

// Round a double to bf16, nearest-even. Normal range: round to odd at binary32 (truncate,
// then set the last bit when inexact) and round that to nearest-even at 8 significant bits;
// a round-to-odd intermediate with at least two extra bits makes the second rounding equal
// to a single one. Below 2^-126 bf16 is subnormal with quantum 2^-133: round |x| * 2^133 to an
// integer directly (it is the fraction field, and 128 carries into the smallest normal).
__device__ __forceinline__ uint16_t f64_to_bf16_edge(double x) {
  if (x != x) return 0x7fc0;
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double ax = fabs(x);
  if (ax < 0x1p-126) return sign | (uint16_t)rint(ax * 0x1p133);
  float f = (float)ax;  // round to nearest even
  uint32_t u = __float_as_uint(f);
  double back = (double)f;
  if (back != ax) {
    if (back > ax) u -= 1;  // rounded up: step back to the truncated value
    u |= 1u;                // sticky bit
  }
  if ((u & 0x7f800000u) == 0x7f800000u) return sign | 0x7f80;  // +inf
  u += 0x7fffu + ((u >> 16) & 1u);
  return sign | (uint16_t)(u >> 16);
}

// The same rounding. Results in bf16's normal range (2^-126 <= |x| < 2^128 before rounding) are
// rounded on the bit pattern: add 2^44 - 1 plus the lowest kept bit (bit 45) to the 64-bit word,
// which rounds to nearest-even at 8 significant bits (a carry out of the fraction raises the
// exponent, up to infinity), and rebias the exponent from 11 to 8 bits. Other inputs take the
// general routine above.
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint32_t hi = (uint32_t)(u >> 32), lo = (uint32_t)u;
  const uint32_t e = (hi >> 20) & 0x7ffu;
  if (e - 897u > 1150u - 897u) return f64_to_bf16_edge(x);
  const uint32_t lsb = (hi >> 13) & 1u;
  const uint32_t h = hi + 0xfffu + ((lo | lsb) != 0u ? 1u : 0u);  // carry of lo + 2^32 - 1 + lsb
  return (uint16_t)(((h >> 16) & 0x8000u) | (((h >> 13) & 0x3ffffu) - (896u << 7)));
}

// Order-preserving map float -> uint32 (larger float, larger key); -0 and +0 map alike.
__device__ __forceinline__ uint32_t f32_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Key of one projected-key row (R bf16 values, as R/8 16-byte words) for the G query heads of a
// unit: RN_f32(max_h sum_i q~_h[i] k~[i]), each sum in float64 over i ascending. The products of
// q~ (a float32 value held in float64) and a bf16 value are exact, so every kernel that calls
// this gets the same bits for the same token. qq points to q~ of the G heads, [G][R].
template <int R, int G, typename QP>
__device__ __forceinline__ float proj_row_key(const uint4 (&w)[R / 8], QP qq) {
  double acc[G];
#pragma unroll
  for (int h = 0; h < G; ++h) acc[h] = 0.0;
#pragma unroll
  for (int i0 = 0; i0 < R / 8; ++i0) {
    const uint32_t ww[4] = {w[i0].x, w[i0].y, w[i0].z, w[i0].w};
#pragma unroll
    for (int ii = 0; ii < 8; ++ii) {
      const double dx = (ii & 1) ? bf16_hi(ww[ii / 2]) : bf16_lo(ww[ii / 2]);
#pragma unroll
      for (int h = 0; h < G; ++h) acc[h] = fma(qq[h * R + i0 * 8 + ii], dx, acc[h]);
    }
  }
  double best = acc[0];
#pragma unroll
  for (int h = 1; h < G; ++h) best = fmax(best, acc[h]);
  return (float)best;
}

// The same key as proj_row_key, bit for bit (each head's float64 sum in the same order, the same
// max), with the heads taken one at a time: a quarter of the registers live, for kernels that
// evaluate it rarely next to a register-hungry main loop.
template <int R, int G>
__device__ __forceinline__ float proj_row_key_lean(const uint4 (&w)[R / 8], const double *qq) {
  double best = 0.0;
#pragma unroll 1
  for (int h = 0; h < G; ++h) {
    double acc = 0.0;
#pragma unroll
    for (int i0 = 0; i0 < R / 8; ++i0) {
      uint32_t ww[4] = {w[i0].x, w[i0].y, w[i0].z, w[i0].w};
      // opaque per head, so that the widened row is formed again for each head rather than kept
      asm volatile("" : "+v"(ww[0]), "+v"(ww[1]), "+v"(ww[2]), "+v"(ww[3]));
#pragma unroll
      for (int ii = 0; ii < 8; ++ii) {
        const double dx = (ii & 1) ? bf16_hi(ww[ii / 2]) : bf16_lo(ww[ii / 2]);
        acc = fma(qq[h * R + i0 * 8 + ii], dx, acc);
      }
    }
    best = h == 0 ? acc : fmax(best, acc);
  }
  return (float)best;
}

// Approximate projected key for the token candidate filter. With qb the bf16 rounding of q~ and
// k the bf16 row, a_h = sum_j qb_hj k_j is evaluated by v_dot2_f32_bf16 (bf16 products are exact
// in float32, the sums are float32) and n1 = sum_j |k_j| the same way. The exact key of every
// head then satisfies |key_h - a_h| <= rel * n1 + abs with the coefficients of filter_coef:
//  - rounding q~ to bf16 moves each product by at most 2^-9 |q~_j k_j|;
//  - a dot2 step rounds at most twice, so the float32 sums are off by at most (R + 2) 2^-24
//    sum_j |q~_j k_j|; the float64 sum of the exact key and its rounding to float add less
//    than 2^-23 of it; for R <= 64 all of this stays below 2^-8.9 sum_j |q~_j k_j|;
//  - sum_j |q~_j k_j| <= max|q~| n1, with n1 low by at most a factor 1 - 2^-18;
//  so rel = 2^-8 max|q~| covers the relative part with a factor of two to spare. The absolute
//  terms cover subnormal inputs, products or sums flushed to zero (below R 2^-126 (max|q~| + 1)).
// max|q~| >= 2^127 could round a bf16 q~ to infinity: rel is then infinite and every token passes.
struct FilterCoef {
  float rel, abs;
};
__device__ __forceinline__ FilterCoef filter_coef(float qmax) {
  FilterCoef f;
  f.rel = qmax < 0x1p127f ? qmax * 0x1p-8f + 0x1p-125f : INFINITY;
  f.abs = qmax * 0x1p-119f + 0x1p-100f;
  return f;
}

// Upper estimate of the projected key of one row (max over the G heads): a + rel * n1 + abs, or
// +infinity when that bound is not finite and below 2^118 (no float32 overflow is then possible in
// a) or the estimate is NaN. qp holds the unit's G * R/2 bf16 pairs of q~.
template <int R, int G>
__device__ __forceinline__ float proj_row_upper(const uint4 (&w)[R / 8], const uint32_t *qp, FilterCoef fc) {
  float acc[G], n1 = 0.0f;
#pragma unroll
  for (int h = 0; h < G; ++h) acc[h] = 0.0f;
#pragma unroll
  for (int i = 0; i < R / 8; ++i) {
    const uint32_t ww[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
#pragma unroll
      for (int h = 0; h < G; ++h)
        acc[h] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qp[h * (R / 2) + i * 4 + p]),
                                                 __builtin_bit_cast(bf16x2_t, ww[p]), acc[h], false);
      n1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, ww[p] & 0x7fff7fffu),
                                           __builtin_bit_cast(bf16x2_t, 0x3f803f80u), n1, false);
    }
  }
  float a = acc[0];
#pragma unroll
  for (int h = 1; h < G; ++h) a = fmaxf(a, acc[h]);
  const float e = fmaf(fc.rel, n1, fc.abs);
  const float hi = a + e;
  return (e < 0x1p118f && hi == hi) ? hi : INFINITY;
}

// Projected-key row of token t of unit (b, g) (t < L): R/8 16-byte loads through the block table.
template <int R>
__device__ __forceinline__ void proj_row_load(const CacheView &c, const uint16_t *kproj, int b, int g, int t,
                                              uint4 (&w)[R / 8]) {
  const int phys = c.bt[(size_t)b * c.maxP + t / c.S];
  const uint4 *row = reinterpret_cast<const uint4 *>(kproj + (((size_t)phys * c.Hkv + g) * c.S + t % c.S) * R);
#pragma unroll
  for (int i = 0; i < R / 8; ++i) w[i] = row[i];
}

// Layout of the token candidate set that the fused projected scoring writes and the token top-k
// selection reads (one buffer, regions 256-byte aligned):
//   hdr   kproj pointer (8 bytes) and the rank R (4 bytes), for the exact fallback of the selection
//   bound [U] uint32     order key T_lo of each unit (candidates are the tokens with key >= T_lo)
//   qt    [B*Hq*R] f64   projected queries q~ (float values)
//   qb    [B*Hq*R] bf16  q~ rounded to bf16, for the approximate filter of the scorer
//   qc    [U][2] float   the filter's error-bound coefficients of each unit
//   count [U][NB] int32  candidates of each group (NB = groups of kCandSegTokens tokens)
//   seg   [U][NB][kCandSegTokens] float2 (key, token index bits), in token order
constexpr int kCandSegTokens = 1024;
struct CandLayout {
  size_t hdr, bound, qt, qb, qc, count, seg, total;
  int nb;
  __host__ __device__ static size_t align(size_t x) { return (x + 255) / 256 * 256; }
  __host__ __device__ CandLayout(int B, int Hq, int Hkv, int Lmax, int R) {
    const size_t U = (size_t)B * Hkv;
    nb = (Lmax + kCandSegTokens - 1) / kCandSegTokens;
    hdr = 0;
    bound = align(hdr + 16);
    qt = align(bound + sizeof(uint32_t) * U);
    qb = align(qt + sizeof(double) * (size_t)B * Hq * R);
    qc = align(qb + sizeof(uint16_t) * (size_t)B * Hq * R);
    count = align(qc + sizeof(float) * 2 * U);
    seg = align(count + sizeof(int32_t) * U * nb);
    total = align(seg + sizeof(float2) * U * nb * kCandSegTokens);
  }
};

// ---------------------------------------------------------------- wave / block reductions
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ double wave_max(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves: row_shr 1, 2, 4, 8 scan each
// row of 16 lanes (lanes without a source add 0), row_bcast:15 adds the last lane of rows 0 and 2
// into rows 1 and 3, row_bcast:31 adds lane 31 into rows 2 and 3.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);
  return v;
}
__device__ __forceinline__ int wave_incl_scan(int v) { return (int)wave_incl_scan((uint32_t)v); }

// Wave maximum with DPP moves (row_shr 1, 2, 4, 8, then row_bcast 15 and 31 as in the scan above):
// lane 63 ends with the maximum of all 64 lanes, read back as a wave-uniform value.
__device__ __forceinline__ float wave_max_dpp(float v) {
  const int ninf = __float_as_int(-INFINITY);
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), 0x111, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), 0x112, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), 0x114, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), 0x118, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), 0x142, 0xa, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), 0x143, 0xc, 0xf, false)));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), kWave - 1));
}

// Wave sums with DPP moves in the pattern of wave_incl_scan (lane 63 ends with the total, read
// back as a wave-uniform value): a fixed order, so the result is reproducible, and no LDS round
// trips. A double moves as its two 32-bit halves; lanes without a source add +0.
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_f64(double v) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, ROWS, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, ROWS, 0xf, false);
  return __longlong_as_double((long long)(((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo));
}
__device__ __forceinline__ double wave_sum_dpp(double v) {
  v += dpp_f64<0x111, 0xf>(v);
  v += dpp_f64<0x112, 0xf>(v);
  v += dpp_f64<0x114, 0xf>(v);
  v += dpp_f64<0x118, 0xf>(v);
  v += dpp_f64<0x142, 0xa>(v);
  v += dpp_f64<0x143, 0xc>(v);
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, kWave - 1);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), kWave - 1);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
__device__ __forceinline__ int wave_sum_dpp(int v) {
  return __builtin_amdgcn_readlane((int)wave_incl_scan((uint32_t)v), kWave - 1);
}

// Unsigned wave minimum and maximum in the same DPP pattern (lanes without a source keep the
// identity), read back from lane 63.
__device__ __forceinline__ uint32_t wave_umin_dpp(uint32_t v) {
  const int id = -1;   // 0xffffffff
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x111, 0xf, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x112, 0xf, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x114, 0xf, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x118, 0xf, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x142, 0xa, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x143, 0xc, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, kWave - 1);
}
__device__ __forceinline__ uint32_t wave_umax_dpp(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, kWave - 1);
}

// Block-wide exclusive prefix sum for blocks of NT threads (NT a multiple of 64, <= 1024).
// `scratch` holds NT/64 + 1 ints of shared memory. Returns the exclusive prefix; *total gets the
// block sum. Contains __syncthreads: every thread of the block must call it.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int *scratch, int *total) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int incl = wave_incl_scan(v);
  if (lane == kWave - 1) scratch[w] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {   // independent broadcast reads of the wave totals
    const int t = scratch[i];
    before += i < w ? t : 0;
    tot += t;
  }
  *total = tot;
  __syncthreads();   // scratch is reused by the next call
  return before + incl - v;
}

template <int NT>
__device__ __forceinline__ float block_max(float v, float *scratch) {
  constexpr int NW = NT / kWave;
  v = wave_max(v);
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[threadIdx.x / kWave] = v;
  __syncthreads();
  float r = scratch[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = fmaxf(r, scratch[i]);
  __syncthreads();
  return r;
}

template <int NT>
__device__ __forceinline__ double block_sum(double v, double *scratch) {
  constexpr int NW = NT / kWave;
  v = wave_sum(v);
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[threadIdx.x / kWave] = v;
  __syncthreads();
  double r = scratch[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r += scratch[i];
  __syncthreads();
  return r;
}

// Block sums of two doubles in one reduction round (scratch: NT/64 double2).
template <int NT>
__device__ __forceinline__ void block_sum2(double &a, double &b, double2 *scratch) {
  constexpr int NW = NT / kWave;
  a = wave_sum_dpp(a);
  b = wave_sum_dpp(b);
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[threadIdx.x / kWave] = make_double2(a, b);
  __syncthreads();
  a = 0.0;
  b = 0.0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const double2 t = scratch[i];
    a += t.x;
    b += t.y;
  }
  __syncthreads();
}

// Three sums at once; scratch holds 3 * NT / kWave doubles.
template <int NT>
__device__ __forceinline__ void block_sum3(double &a, double &b, double &c, double *scratch) {
  constexpr int NW = NT / kWave;
  a = wave_sum_dpp(a);
  b = wave_sum_dpp(b);
  c = wave_sum_dpp(c);
  if ((threadIdx.x & (kWave - 1)) == 0) {
    const int w = threadIdx.x / kWave;
    scratch[w] = a;
    scratch[NW + w] = b;
    scratch[2 * NW + w] = c;
  }
  __syncthreads();
  a = 0.0;
  b = 0.0;
  c = 0.0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    a += scratch[i];
    b += scratch[NW + i];
    c += scratch[2 * NW + i];
  }
  __syncthreads();
}

template <int NT>
__device__ __forceinline__ double block_max(double v, double *scratch) {
  constexpr int NW = NT / kWave;
  v = wave_max(v);
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[threadIdx.x / kWave] = v;
  __syncthreads();
  double r = scratch[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = fmax(r, scratch[i]);
  __syncthreads();
  return r;
}

// Sum over the `width` consecutive lanes of an aligned lane group (width 2, 4, 8 or 16) with DPP
// moves: quad_perm [1,0,3,2] sums a pair, [2,3,0,1] then a quad, row_half_mirror pairs the two
// quads of 8 lanes, row_mirror the two halves of a 16-lane row. Every lane of the group gets the
// group sum, with the same bits (each step adds the same two values in either order).
template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(WIDTH == 2 || WIDTH == 4 || WIDTH == 8 || WIDTH == 16, "lane group of 2, 4, 8 or 16");
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
  if (WIDTH == 2) return v;
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
  if (WIDTH == 4) return v;
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));
  if (WIDTH == 16) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false));
  return v;
}

// group_sum of N independent values at once, one reduction level for all of them before the
// next, so that the DPP reads of one value fill the wait states after another's addition.
template <int CTL, int N>
__device__ __forceinline__ void group_sum_level(float (&v)[N]) {
  float t[N];
#pragma unroll
  for (int i = 0; i < N; ++i) t[i] = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v[i]), CTL, 0xF, 0xF, false));
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += t[i];
}
template <int WIDTH, int N>
__device__ __forceinline__ void group_sum_n(float (&v)[N]) {
  static_assert(WIDTH == 8 || WIDTH == 16, "lane group of 8 or 16");
  group_sum_level<0xB1>(v);   // the steps of group_sum
  group_sum_level<0x4E>(v);
  group_sum_level<0x141>(v);
  if (WIDTH == 16) group_sum_level<0x140>(v);
}

// Radix selection over order keys get(i), i < n: finds the r-th largest key T (1 <= r <= n) and
// need = r - #(keys > T), i.e. how many keys equal to T belong to the top r. Four 8-bit digits,
// most significant first. Each wave counts into its own 256-bin LDS histogram (the leading digits
// of float keys fall into few bins, so one shared histogram would serialize the atomics); the
// wave histograms are then summed. Integer atomics only, so the result is deterministic.
// `hist` holds NT/64 * 256 words, `bc` 2 words of shared memory. Every thread must call it.
// With digits < 4 only the leading digits are resolved: T then has its low bits cleared, which
// makes it a lower bound of the r-th largest key with at least r keys >= T.
// When every key lies in [lo, hi], the leading digits that lo and hi share are common to all keys
// and need no pass: a candidate set drawn from above a bound has one or two in front.
template <int NT, typename Get>
__device__ void radix_kth(Get get, int n, uint32_t r, uint32_t *hist, uint32_t *bc, uint32_t &T, uint32_t &need,
                          int digits = 4, uint32_t lo = 0u, uint32_t hi = 0xffffffffu) {
  constexpr int NW = NT / kWave;
  const int tid = threadIdx.x;
  uint32_t *mine = hist + (tid / kWave) * 256;
  const int last = 32 - 8 * digits;
  int first = 24;
  uint32_t mask = 0;
  while (first >= last && ((lo ^ hi) >> first) == 0) {
    mask |= 0xffu << first;
    first -= 8;
  }
  uint32_t prefix = lo & mask;
  need = r;
  for (int shift = first; shift >= last; shift -= 8) {
    for (int i = tid; i < NW * 256; i += NT) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += NT) {
      const uint32_t u = get(i);
      if ((u & mask) == prefix) atomicAdd(&mine[(u >> shift) & 0xffu], 1u);
    }
    __syncthreads();
    // the wanted digit v has count(> v) < need <= count(>= v); lane l owns digits 4l .. 4l+3
    if (tid < kWave) {
      uint32_t c4[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int w = 0; w < NW; ++w) {   // one 16-byte read per wave histogram (no bank conflicts)
        const uint4 h4 = reinterpret_cast<const uint4 *>(hist + w * 256)[tid];
        c4[0] += h4.x;
        c4[1] += h4.y;
        c4[2] += h4.z;
        c4[3] += h4.w;
      }
      const uint32_t local = c4[0] + c4[1] + c4[2] + c4[3];
      // keys in the digits of higher lanes: the wave total minus the inclusive prefix
      const uint32_t pre = wave_incl_scan(local);
      uint32_t above = __builtin_amdgcn_readlane(pre, kWave - 1) - pre;
#pragma unroll
      for (int i = 3; i >= 0; --i) {
        if (above < need && above + c4[i] >= need) {
          bc[0] = prefix | ((uint32_t)(4 * tid + i) << shift);
          bc[1] = need - above;
        }
        above += c4[i];
      }
    }
    __syncthreads();
    prefix = bc[0];
    need = bc[1];
    mask |= 0xffu << shift;
    __syncthreads();
  }
  T = prefix;
}

}  // namespace skv
