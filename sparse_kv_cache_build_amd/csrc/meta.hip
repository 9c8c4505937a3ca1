// Page metadata builder ("EntmaxKV" summary s2.A: per-page box bounds and Gaussian moments;
// "Joint Subspace Sparse Attention" abstract: keys cached in a shared low-dimensional subspace).
// Runs once per page at prefill time, and after an append for the pages holding the new tokens
// (tail > 0: only pages holding one of the last `tail` tokens of a sequence, recomputed over all
// their valid tokens, so the result equals a full build of those pages). Off the per-step path.
#include "common.hpp"
#include "launch.hpp"

namespace skv {

// One workgroup per logical page (p, b); threads sweep (KV head, coordinate) pairs so that each
// token row is read with consecutive coordinates across consecutive threads.
//   box:   exact min / max over the valid tokens, stored as the original element bits, the
//          64-byte blocks of the min row and of the max row alternating ([d / C][2][C], C = 64 bytes).
//   gauss: float64 mean (sum over t ascending, divided by n), then float64 mean squared
//          deviation, each rounded once to float32.
// First logical page a build (tail == 0) or an append of `tail` tokens covers.
__device__ __forceinline__ int first_page(const CacheView &c, int L, int tail) {
  return tail > 0 ? max(0, L - tail) / c.S : 0;
}

template <typename T>
__global__ __launch_bounds__(256) void meta_box_gauss_kernel(CacheView c, int tail, T *__restrict__ box,
                                                             float *__restrict__ gauss) {
  const int b = blockIdx.y;
  const int L = seq_len(c, b);
  const int p = first_page(c, L, tail) + blockIdx.x;
  if (p >= num_pages(c, L)) return;
  const int n = min(c.S, L - p * c.S);
  const int phys = c.bt[(size_t)b * c.maxP + p];
  const T *K = static_cast<const T *>(c.k);
  for (int idx = threadIdx.x; idx < c.Hkv * c.D; idx += blockDim.x) {
    const int g = idx / c.D, j = idx - g * c.D;
    const size_t base = ((size_t)phys * c.Hkv + g) * c.S * c.D + j;
    // 64-byte blocks of the mean and variance rows alternate, so one 128-byte line holds both
    const size_t mo = ((size_t)phys * c.Hkv + g) * 2 * c.D + (size_t)(j / 16) * 32 + (j % 16);
    if (box) {
      T lo = K[base], hi = K[base];
      float flo = Elem<T>::get(K, base), fhi = flo;
      for (int t = 1; t < n; ++t) {
        T x = K[base + (size_t)t * c.D];
        float fx = Elem<T>::get(K, base + (size_t)t * c.D);
        if (fx < flo) { flo = fx; lo = x; }
        if (fx > fhi) { fhi = fx; hi = x; }
      }
      // 64-byte blocks of the min and max rows alternate, so one 128-byte line holds both
      constexpr int C = 64 / (int)sizeof(T);
      const size_t bo = ((size_t)phys * c.Hkv + g) * 2 * c.D + (size_t)(j / C) * 2 * C + (j % C);
      box[bo] = lo;
      box[bo + C] = hi;
    }
    if (gauss) {
      double sum = 0.0;
      for (int t = 0; t < n; ++t) sum += (double)Elem<T>::get(K, base + (size_t)t * c.D);
      const double mu = sum / n;
      double ss = 0.0;
      for (int t = 0; t < n; ++t) {
        const double dv = (double)Elem<T>::get(K, base + (size_t)t * c.D) - mu;
        ss += dv * dv;
      }
      gauss[mo] = (float)mu;
      gauss[mo + 16] = (float)(ss / n);
    }
  }
}

// Pooled keys: per sub-block of pb token slots of the page, RN_f32 of the float64 mean of its
// valid keys (t ascending). One workgroup per logical page (p, b); threads sweep (KV head,
// coordinate) pairs like the box / moment kernel.
template <typename T>
__global__ __launch_bounds__(256) void meta_pool_kernel(CacheView c, int tail, int pb, float *__restrict__ pool) {
  const int b = blockIdx.y;
  const int L = seq_len(c, b);
  const int p = first_page(c, L, tail) + blockIdx.x;
  if (p >= num_pages(c, L)) return;
  const int n = min(c.S, L - p * c.S);
  const int nsb = c.S / pb;
  const int phys = c.bt[(size_t)b * c.maxP + p];
  const T *K = static_cast<const T *>(c.k);
  for (int idx = threadIdx.x; idx < c.Hkv * c.D; idx += blockDim.x) {
    const int g = idx / c.D, j = idx - g * c.D;
    const size_t base = ((size_t)phys * c.Hkv + g) * c.S * c.D + j;
    for (int sb = 0; sb < nsb && sb * pb < n; ++sb) {
      const int t1 = min(n, sb * pb + pb);
      double sum = 0.0;
      for (int t = sb * pb; t < t1; ++t) sum += (double)Elem<T>::get(K, base + (size_t)t * c.D);
      pool[(((size_t)phys * c.Hkv + g) * nsb + sb) * c.D + j] = (float)(sum / (t1 - sb * pb));
    }
  }
}

// Projected keys k~_t[i] = RN_bf16(sum_j P[i][j] k_t[j]) (float64, j ascending). One workgroup
// per (logical page, KV head): the page's keys and P are staged in LDS as float (exact), then
// each thread owns (token, i) pairs.
template <typename T>
__global__ __launch_bounds__(256) void meta_proj_kernel(CacheView c, int tail, int r, const float *__restrict__ proj,
                                                        uint16_t *__restrict__ kproj) {
  extern __shared__ float smem[];
  const int b = blockIdx.y / c.Hkv, g = blockIdx.y % c.Hkv;
  const int L = seq_len(c, b);
  const int p = first_page(c, L, tail) + blockIdx.x;
  if (p >= num_pages(c, L)) return;
  const int n = min(c.S, L - p * c.S);
  const int t0 = tail > 0 ? max(0, L - tail - p * c.S) : 0;   // first row of the page to write
  const int phys = c.bt[(size_t)b * c.maxP + p];
  const int ldp = c.D + 1;  // padded row stride of P (bank spread across i)
  float *Ps = smem;                     // [r][D+1]
  float *Ks = smem + (size_t)r * ldp;   // [n][D]
  const T *K = static_cast<const T *>(c.k) + ((size_t)phys * c.Hkv + g) * c.S * c.D;
  for (int i = threadIdx.x; i < r * c.D; i += blockDim.x) Ps[(i / c.D) * ldp + i % c.D] = proj[i];
  for (int i = t0 * c.D + threadIdx.x; i < n * c.D; i += blockDim.x) Ks[i] = Elem<T>::get(K, i);
  __syncthreads();
  uint16_t *out = kproj + ((size_t)phys * c.Hkv + g) * c.S * r;
  for (int pair = t0 * r + threadIdx.x; pair < n * r; pair += blockDim.x) {
    const int t = pair / r, i = pair - t * r;
    const float *pr = Ps + i * ldp, *kr = Ks + t * c.D;
    double acc = 0.0;
    for (int j = 0; j < c.D; ++j) acc = fma((double)pr[j], (double)kr[j], acc);
    out[(size_t)t * r + i] = f64_to_bf16(acc);
  }
}

// Soft-LSH metadata. One workgroup per logical page (p, b) covers the page's rows (KV head g,
// token t), in chunks of 64 rows staged in LDS as float (exact). Work items are (table l, row)
// pairs, with l constant over a wave in full chunks so that the hyperplanes of table l are
// wave-uniform (scalar loads); each item takes the P float64 dot products of its row in
// coordinate order, bit i of the bucket id being (dot_i > 0). Rows [t0, n) of the page are
// written: all of them for a build, the new tokens for an append. The value norm of each row is
// RN_f32(sqrt) of its float64 sum of squares.
template <typename T, int D, int P>
__global__ __launch_bounds__(256) void meta_lsh_kernel(CacheView c, int tail, int L, const float *__restrict__ planes,
                                                       uint8_t *__restrict__ bucket, float *__restrict__ vnorm) {
  constexpr int RC = 64, LDR = D + 1;
  __shared__ float Ks[RC * LDR];
  const int b = blockIdx.y;
  const int len = seq_len(c, b);
  const int p = first_page(c, len, tail) + blockIdx.x;
  if (p >= num_pages(c, len)) return;
  const int n = min(c.S, len - p * c.S);
  const int t0 = tail > 0 ? max(0, len - tail - p * c.S) : 0;
  const int cnt = n - t0, rows = c.Hkv * cnt;   // row r: KV head r / cnt, token t0 + r % cnt
  const int phys = c.bt[(size_t)b * c.maxP + p];
  const T *K = static_cast<const T *>(c.k);
  const T *V = static_cast<const T *>(c.v);
  for (int r0 = 0; r0 < rows; r0 += RC) {
    const int nr = min(RC, rows - r0);
    __syncthreads();
    for (int i = threadIdx.x; i < nr * D; i += blockDim.x) {
      const int r = r0 + i / D, j = i % D, g = r / cnt, t = t0 + r % cnt;
      Ks[(i / D) * LDR + j] = Elem<T>::get(K, (((size_t)phys * c.Hkv + g) * c.S + t) * D + j);
    }
    __syncthreads();
    for (int item = threadIdx.x; item < L * nr; item += blockDim.x) {
      // full chunks: table l is constant over each wave (scalar loads of its hyperplanes); a
      // partial chunk (an append touches a few rows) packs its (table, row) items densely
      const int l = nr == RC ? __builtin_amdgcn_readfirstlane(item / RC) : item / nr;
      const int rr = item - l * nr;
      const float *w = planes + (size_t)l * P * D;
      const float *kr = Ks + rr * LDR;
      double acc[P];
#pragma unroll
      for (int i = 0; i < P; ++i) acc[i] = 0.0;
      for (int j = 0; j < D; ++j) {
        const double kv = kr[j];
#pragma unroll
        for (int i = 0; i < P; ++i) acc[i] = fma((double)w[i * D + j], kv, acc[i]);
      }
      uint32_t id = 0;
#pragma unroll
      for (int i = 0; i < P; ++i) id |= (acc[i] > 0.0 ? 1u : 0u) << i;
      const int r = r0 + rr, g = r / cnt, t = t0 + r % cnt;
      bucket[(((size_t)phys * c.Hkv + g) * c.S + t) * L + l] = (uint8_t)id;
    }
    for (int rr = threadIdx.x; rr < nr; rr += blockDim.x) {
      const int r = r0 + rr, g = r / cnt, t = t0 + r % cnt;
      const size_t row = ((size_t)phys * c.Hkv + g) * c.S + t;
      double ss = 0.0;
      for (int j = 0; j < D; ++j) {
        const double x = Elem<T>::get(V, row * D + j);
        ss = fma(x, x, ss);
      }
      vnorm[row] = (float)sqrt(ss);
    }
  }
}

template <typename T, int D>
static hipError_t lsh_meta_d(const CacheView &c, int tail, int L, int P, const float *planes, uint8_t *bucket,
                             float *vnorm, const dim3 &grid, hipStream_t st) {
  switch (P) {
#define SKV_LSH_P(PP) \
  case PP: meta_lsh_kernel<T, D, PP><<<grid, 256, 0, st>>>(c, tail, L, planes, bucket, vnorm); break;
    SKV_LSH_P(1) SKV_LSH_P(2) SKV_LSH_P(3) SKV_LSH_P(4) SKV_LSH_P(5) SKV_LSH_P(6) SKV_LSH_P(7) SKV_LSH_P(8)
#undef SKV_LSH_P
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_build_lsh(const CacheView &c, int dtype, int tail, int L, int P, const float *planes,
                            uint8_t *bucket, float *vnorm, hipStream_t st) {
  const int np = tail > 0 ? min(c.maxP, (tail + c.S - 1) / c.S + 1) : c.maxP;
  const dim3 grid(np, c.B);
  if (c.D == 64)
    return dtype == 0 ? lsh_meta_d<float, 64>(c, tail, L, P, planes, bucket, vnorm, grid, st)
                      : lsh_meta_d<uint16_t, 64>(c, tail, L, P, planes, bucket, vnorm, grid, st);
  return dtype == 0 ? lsh_meta_d<float, 128>(c, tail, L, P, planes, bucket, vnorm, grid, st)
                    : lsh_meta_d<uint16_t, 128>(c, tail, L, P, planes, bucket, vnorm, grid, st);
}

hipError_t launch_build_meta(const CacheView &c, int dtype, int tail, void *box, float *gauss, int r,
                             const float *proj, uint16_t *kproj, int pb, float *pool, hipStream_t st) {
  // pages per sequence: all of them, or those the last `tail` tokens can touch
  const int np = tail > 0 ? min(c.maxP, (tail + c.S - 1) / c.S + 1) : c.maxP;
  const dim3 grid(np, c.B);
  if (box || gauss) {
    if (dtype == 0)
      meta_box_gauss_kernel<float><<<grid, 256, 0, st>>>(c, tail, static_cast<float *>(box), gauss);
    else
      meta_box_gauss_kernel<uint16_t><<<grid, 256, 0, st>>>(c, tail, static_cast<uint16_t *>(box), gauss);
  }
  if (pool) {
    if (dtype == 0)
      meta_pool_kernel<float><<<grid, 256, 0, st>>>(c, tail, pb, pool);
    else
      meta_pool_kernel<uint16_t><<<grid, 256, 0, st>>>(c, tail, pb, pool);
  }
  if (kproj) {
    const size_t lds = sizeof(float) * ((size_t)r * (c.D + 1) + (size_t)c.S * c.D);
    const dim3 g2(np, c.B * c.Hkv);
    if (dtype == 0)
      meta_proj_kernel<float><<<g2, 256, lds, st>>>(c, tail, r, proj, kproj);
    else
      meta_proj_kernel<uint16_t><<<g2, 256, lds, st>>>(c, tail, r, proj, kproj);
  }
  return hipGetLastError();
}

}  // namespace skv
