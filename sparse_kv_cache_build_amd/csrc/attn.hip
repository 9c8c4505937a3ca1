// Attention over the selected KV only ("EntmaxKV" summary s2.C; softmax is the comparator of
// its s1 and s3). Token-granular selections read rows in place through block_table, with no
// gathered copy ("Joint Subspace Sparse Attention" abstract).
//
// Work decomposition (split-K over the selection): block (split, unit) takes `spi` consecutive
// selected items (pages or tokens) of unit (b, g) and all G query heads of g. Inside a block a
// row (one token's d coordinates) is read by a group of D/8 lanes, 8 coordinates per lane
// (16-byte loads for bf16), so a wave covers 4 (d = 128) or 8 (d = 64) rows per step and the
// block's 4 waves 16 or 32 rows. q . k is a per-lane partial dot product summed over the lane
// group with DPP moves.
//
// softmax: every lane group keeps an online (max, sum, acc) state per head, rescaled only when a
//          logit exceeds the running reference by 2^32 (in log2 units), then the groups are
//          merged in the block and across splits by a fixed-order log-sum-exp combine.
// entmax:  pass 1 writes, per (unit, head, split), the split's maximum of z' = (alpha-1) z and the
//          (z', slot) pairs with z' > max - 1, in row order. Since the global threshold satisfies
//          tau >= max_all z' - 1, no other row can carry weight. The solve kernel (one block per
//          query head) keeps the pairs with z' > max_all - 1, bisects tau, refines it with the
//          closed form on the support (alpha = 2, 1.5), and accumulates p v reading V rows with
//          p > 0 only.
#include "common.hpp"
#include "launch.hpp"

namespace skv {

constexpr int kAttnThreads = 256;
constexpr int kCandLds = 8192;  // candidates of one head held in LDS by the solve kernel

template <int D>
struct RowLayout {
  static constexpr int LPR = D / 8;                               // lanes per row
  static constexpr int RPW = kWave / LPR;                         // rows per wave step
  static constexpr int RGB = (kAttnThreads / kWave) * RPW;        // row groups per block
};

// Resolves row r of a split (items [it0, it1)) to a K/V element offset of the row start, or -1
// when the row is past the page's valid tokens or the sequence.
struct RowMap {
  const int32_t *sel;  // selection of the unit
  const int32_t *bt;   // block table row of the sequence
  int gran, S, Hkv, g, D, L, P;
  __device__ __forceinline__ long long row_offset(int item, int t_in_page) const {
    int page, t;
    if (gran) {
      const int tok = sel[item];
      if (tok < 0 || tok >= L) return -1;
      page = tok / S;
      t = tok - page * S;
    } else {
      page = sel[item];
      if (page < 0 || page >= P) return -1;
      t = t_in_page;
      if (t >= min(S, L - page * S)) return -1;
    }
    const long long phys = bt[page];
    return ((phys * Hkv + g) * S + t) * (long long)D;
  }
};

// ---------------------------------------------------------------- softmax, split-K

template <typename T, int D, int G>
__global__ __launch_bounds__(kAttnThreads) void attn_softmax_kernel(
    CacheView c, const T *__restrict__ q, const int32_t *__restrict__ sel_idx, const int32_t *__restrict__ sel_count,
    int cap, int gran, int spi, int nsplit, float scale_log2, float *__restrict__ part, float *__restrict__ out) {
  using RL = RowLayout<D>;
  __shared__ float s_m[G][RL::RGB];
  __shared__ float s_l[G][RL::RGB];
  __shared__ float s_acc[kAttnThreads / kWave][G][D];
  const int split = blockIdx.x, unit = blockIdx.y, b = unit / c.Hkv, g = unit - b * c.Hkv;
  const int count = min(max(sel_count[unit], 0), cap);
  const int it0 = split * spi;
  if (it0 >= count && !(split == 0 && nsplit == 1)) return;  // empty split (count is known to the combine)
  const int it1 = min(count, it0 + spi);
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int lr = lane % RL::LPR, rg = wave * RL::RPW + lane / RL::LPR;
  const int L = seq_len(c, b);
  RowMap rm{sel_idx + (size_t)unit * cap, c.bt + (size_t)b * c.maxP, gran, c.S, c.Hkv, g, D, L, num_pages(c, L)};
  const int rows_per_item = gran ? 1 : c.S;
  const int NR = max(0, it1 - it0) * rows_per_item;

  float qv[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    Elem<T>::load8(q + ((size_t)b * c.Hq + g * G + h) * D + lr * 8, qv[h]);
#pragma unroll
    for (int j = 0; j < 8; ++j) qv[h][j] *= scale_log2;
  }
  float mref[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    mref[h] = -INFINITY;
    l[h] = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[h][j] = 0.0f;
  }
  const T *K = static_cast<const T *>(c.k), *V = static_cast<const T *>(c.v);
  auto row_off = [&](int r) -> long long {
    if (r >= NR) return -1;
    const int it = r / rows_per_item;
    return rm.row_offset(it0 + it, r - it * rows_per_item);
  };
  auto accumulate = [&](const float (&kx)[8], const float (&vx)[8]) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float part_dot = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) part_dot = fmaf(qv[h][j], kx[j], part_dot);
      const float z = group_sum<RL::LPR>(part_dot);
      if (z > mref[h] + 32.0f) {  // rescale the state to a new reference
        const float corr = exp2f(mref[h] - z);
        l[h] *= corr;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[h][j] *= corr;
        mref[h] = z;
      }
      const float p = exp2f(z - mref[h]);
      l[h] += p;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[h][j] = fmaf(p, vx[j], acc[h][j]);
    }
  };
  // two rows per lane group per step: both rows' loads are in flight before either is used
  for (int r = rg; r < NR; r += 2 * RL::RGB) {
    const long long o1 = row_off(r), o2 = row_off(r + RL::RGB);
    float k1[8], v1[8], k2[8], v2[8];
    if (o1 >= 0) {
      Elem<T>::load8(K + o1 + lr * 8, k1);
      Elem<T>::load8(V + o1 + lr * 8, v1);
    }
    if (o2 >= 0) {
      Elem<T>::load8(K + o2 + lr * 8, k2);
      Elem<T>::load8(V + o2 + lr * 8, v2);
    }
    if (o1 >= 0) accumulate(k1, v1);
    if (o2 >= 0) accumulate(k2, v2);
  }
  // merge the lane groups: common reference per head, then sums
  if (lr == 0)
#pragma unroll
    for (int h = 0; h < G; ++h) s_m[h][rg] = mref[h];
  __syncthreads();
  float M[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    M[h] = -INFINITY;
    for (int i = 0; i < RL::RGB; ++i) M[h] = fmaxf(M[h], s_m[h][i]);
    const float f = mref[h] == -INFINITY ? 0.0f : exp2f(mref[h] - M[h]);
    l[h] *= f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float a = acc[h][j] * f;
      // sum over the row groups of this wave (lanes lr, lr + LPR, ...)
#pragma unroll
      for (int o = RL::LPR; o < kWave; o <<= 1) a += __shfl_xor(a, o, kWave);
      acc[h][j] = a;
    }
  }
  if (lr == 0)
#pragma unroll
    for (int h = 0; h < G; ++h) s_l[h][rg] = l[h];
  if (lane < RL::LPR)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int j = 0; j < 8; ++j) s_acc[wave][h][lr * 8 + j] = acc[h][j];
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += kAttnThreads) {
    const int h = idx / D, j = idx - h * D;
    float a = 0.0f;
#pragma unroll
    for (int w = 0; w < kAttnThreads / kWave; ++w) a += s_acc[w][h][j];
    float lsum = 0.0f;
    for (int i = 0; i < RL::RGB; ++i) lsum += s_l[h][i];
    if (nsplit == 1) {
      out[((size_t)b * c.Hq + g * G + h) * D + j] = lsum > 0.0f ? a / lsum : 0.0f;
    } else {
      float *pp = part + (((size_t)unit * nsplit + split) * G + h) * (D + 2);
      if (j == 0) {
        pp[0] = M[h];
        pp[1] = lsum;
      }
      pp[2 + j] = a;
    }
  }
}

// Fixed-order log-sum-exp combine of the non-empty splits of each query head. The per-split
// (max, sum) pairs go through LDS first so that the accumulator loads are independent.
constexpr int kCombineMax = 1024;   // splits merged per LDS round
template <int D>
__global__ __launch_bounds__(D) void attn_combine_kernel(CacheView c, const int32_t *__restrict__ sel_count, int cap,
                                                        int spi, int nsplit, const float *__restrict__ part,
                                                        float *__restrict__ out) {
  __shared__ float s_w[kCombineMax];
  __shared__ float s_l[kCombineMax];
  __shared__ float red[D / kWave];
  const int bh = blockIdx.x, b = bh / c.Hq, h = bh - b * c.Hq, g = h / c.G, hh = h - g * c.G;
  const int unit = b * c.Hkv + g;
  const int count = min(max(sel_count[unit], 0), cap);
  const int ns = min(nsplit, (count + spi - 1) / spi);
  const int j = threadIdx.x;
  const size_t stride = (size_t)c.G * (D + 2);
  const float *p0 = part + ((size_t)unit * nsplit * c.G + hh) * (D + 2);
  // global max over the non-empty splits
  float M = -INFINITY;
  for (int s = j; s < ns; s += D) {
    const float *pp = p0 + s * stride;
    if (pp[1] > 0.0f) M = fmaxf(M, pp[0]);
  }
  M = block_max<D>(M, red);
  float lsum = 0.0f, a = 0.0f;
  for (int s0 = 0; s0 < ns; s0 += kCombineMax) {
    const int n = min(kCombineMax, ns - s0);
    for (int s = j; s < n; s += D) {
      const float *pp = p0 + (s0 + s) * stride;
      const float l = pp[1];
      s_w[s] = l > 0.0f ? exp2f(pp[0] - M) : 0.0f;
      s_l[s] = l;
    }
    __syncthreads();
#pragma unroll 8
    for (int s = 0; s < n; ++s) {
      const float w = s_w[s];
      lsum += s_l[s] * w;
      a += (w > 0.0f ? p0[(s0 + s) * stride + 2 + j] : 0.0f) * w;
    }
    __syncthreads();
  }
  out[(size_t)bh * D + j] = lsum > 0.0f ? a / lsum : 0.0f;
}

// ---------------------------------------------------------------- entmax pass 1

template <typename T, int D, int G>
__global__ __launch_bounds__(kAttnThreads) void attn_entmax_logits_kernel(
    CacheView c, const T *__restrict__ q, const int32_t *__restrict__ sel_idx, const int32_t *__restrict__ sel_count,
    int cap, int gran, int spi, int nsplit, float zscale, float2 *__restrict__ cand, int32_t *__restrict__ cand_cnt,
    float *__restrict__ cand_max) {
  using RL = RowLayout<D>;
  extern __shared__ float zs[];  // [G][rps]
  __shared__ int scan_scratch[kAttnThreads / kWave + 1];
  __shared__ float redf[kAttnThreads / kWave];
  const int split = blockIdx.x, unit = blockIdx.y, b = unit / c.Hkv, g = unit - b * c.Hkv;
  const int count = min(max(sel_count[unit], 0), cap);
  const int rows_per_item = gran ? 1 : c.S;
  const int rps = spi * rows_per_item;
  const int it0 = split * spi, it1 = min(count, it0 + spi);
  const int NR = max(0, it1 - it0) * rows_per_item;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int lr = lane % RL::LPR, rg = wave * RL::RPW + lane / RL::LPR;
  const int L = seq_len(c, b);
  RowMap rm{sel_idx + (size_t)unit * cap, c.bt + (size_t)b * c.maxP, gran, c.S, c.Hkv, g, D, L, num_pages(c, L)};

  float qv[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    Elem<T>::load8(q + ((size_t)b * c.Hq + g * G + h) * D + lr * 8, qv[h]);
#pragma unroll
    for (int j = 0; j < 8; ++j) qv[h][j] *= zscale;
  }
  const T *K = static_cast<const T *>(c.k);
  auto row_off = [&](int r) -> long long {
    if (r >= NR) return -1;
    const int it = r / rows_per_item;
    return rm.row_offset(it0 + it, r - it * rows_per_item);
  };
  auto logits = [&](int r, long long off, const float (&kx)[8]) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float part_dot = 0.0f;
      if (off >= 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j) part_dot = fmaf(qv[h][j], kx[j], part_dot);
        part_dot = group_sum<RL::LPR>(part_dot);
      }
      if (lr == h % RL::LPR) zs[h * rps + r] = off >= 0 ? part_dot : -INFINITY;
    }
  };
  for (int r = rg; r < NR; r += 2 * RL::RGB) {
    const int r2 = r + RL::RGB;
    const long long o1 = row_off(r), o2 = row_off(r2);
    float k1[8], k2[8];
    if (o1 >= 0) Elem<T>::load8(K + o1 + lr * 8, k1);
    if (o2 >= 0) Elem<T>::load8(K + o2 + lr * 8, k2);
    logits(r, o1, k1);
    if (r2 < NR) logits(r2, o2, k2);
  }
  __syncthreads();
  for (int h = 0; h < G; ++h) {
    float mx = -INFINITY;
    for (int r = tid; r < NR; r += kAttnThreads) mx = fmaxf(mx, zs[h * rps + r]);
    mx = block_max<kAttnThreads>(mx, redf);
    const size_t lid = ((size_t)unit * G + h) * nsplit + split;
    float2 *cl = cand + lid * rps;
    // ordered compaction of z' > mx - 1 (contiguous chunk of rows per thread)
    const int per = (NR + kAttnThreads - 1) / kAttnThreads;
    const int r0 = min(NR, tid * per), r1 = min(NR, r0 + per);
    int nk = 0;
    for (int r = r0; r < r1; ++r) nk += zs[h * rps + r] > mx - 1.0f;
    int tot;
    int pos = block_excl_scan<kAttnThreads>(nk, scan_scratch, &tot);
    for (int r = r0; r < r1; ++r) {
      const float z = zs[h * rps + r];
      if (z > mx - 1.0f) cl[pos++] = make_float2(z, __int_as_float(it0 * rows_per_item + r));
    }
    if (tid == 0) {
      cand_cnt[lid] = tot;
      cand_max[lid] = mx;
    }
  }
}

// ---------------------------------------------------------------- entmax threshold and p V

// ALPHA_KIND: 1 -> alpha = 1.5, 2 -> alpha = 2, 3 -> any alpha in (1, 2)
template <typename T, int D, int ALPHA_KIND>
__global__ __launch_bounds__(kAttnThreads) void attn_entmax_solve_kernel(
    CacheView c, const int32_t *__restrict__ sel_idx, const int32_t *__restrict__ sel_count, int cap, int gran,
    int spi, int nsplit, float alpha, const float2 *__restrict__ cand, const int32_t *__restrict__ cand_cnt,
    const float *__restrict__ cand_max, float *__restrict__ out) {
  using RL = RowLayout<D>;
  __shared__ float cz[kCandLds];
  __shared__ int cslot[kCandLds];
  __shared__ int scan_scratch[kAttnThreads / kWave + 1];
  __shared__ float redf[kAttnThreads / kWave];
  __shared__ double redd[kAttnThreads / kWave];
  __shared__ float s_acc[kAttnThreads / kWave][D];
  const int bh = blockIdx.x, b = bh / c.Hq, h = bh - b * c.Hq, g = h / c.G, hh = h - g * c.G;
  const int unit = b * c.Hkv + g;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int count = min(max(sel_count[unit], 0), cap);
  const int rows_per_item = gran ? 1 : c.S;
  const int rps = spi * rows_per_item;
  const int ns = min(nsplit, (count + spi - 1) / spi);
  const size_t lid0 = ((size_t)unit * c.G + hh) * nsplit;
  float *o = out + (size_t)bh * D;

  float mx = -INFINITY;
  for (int s = tid; s < ns; s += kAttnThreads) mx = fmaxf(mx, cand_max[lid0 + s]);
  mx = block_max<kAttnThreads>(mx, redf);
  if (mx == -INFINITY) {  // nothing selected
    for (int j = tid; j < D; j += kAttnThreads) o[j] = 0.0f;
    return;
  }
  const float lo_bound = mx - 1.0f;
  // gather the pairs with z' > max - 1 into LDS in (split, row) order
  int n = 0;
  bool overflow = false;
  for (int s0 = 0; s0 < ns; s0 += kAttnThreads) {
    const int s = s0 + tid;
    int nk = 0;
    if (s < ns) {
      const float2 *cl = cand + (lid0 + s) * rps;
      const int cnt = cand_cnt[lid0 + s];
      for (int i = 0; i < cnt; ++i) nk += cl[i].x > lo_bound;
    }
    int tot;
    int pos = n + block_excl_scan<kAttnThreads>(nk, scan_scratch, &tot);
    if (n + tot > kCandLds) overflow = true;
    if (!overflow && s < ns) {
      const float2 *cl = cand + (lid0 + s) * rps;
      const int cnt = cand_cnt[lid0 + s];
      for (int i = 0; i < cnt; ++i) {
        const float2 e = cl[i];
        if (e.x > lo_bound) {
          cz[pos] = e.x;
          cslot[pos] = __float_as_int(e.y);
          ++pos;
        }
      }
    }
    n += tot;
  }
  __syncthreads();
  if (overflow) {
    // more survivors than LDS holds: not produced by a valid bound; flag with NaN output
    for (int j = tid; j < D; j += kAttnThreads) o[j] = NAN;
    return;
  }
  // bisection: F(tau) = sum (z' - tau)_+^(1/(alpha-1)) - 1, F(mx - 1) >= 0 >= F(mx - n^(1-alpha))
  const float am1 = alpha - 1.0f, inv = 1.0f / am1;
  auto pw = [&](float x) -> float {
    if (ALPHA_KIND == 1) return x * x;
    if (ALPHA_KIND == 2) return x;
    return powf(x, inv);
  };
  float lo = lo_bound, hi = mx - powf((float)n, -am1);
  for (int it = 0; it < 40; ++it) {
    const float mid = 0.5f * (lo + hi);
    if (mid <= lo || mid >= hi) break;
    double sum = 0.0;
    for (int i = tid; i < n; i += kAttnThreads) {
      const float x = cz[i] - mid;
      if (x > 0.0f) sum += (double)pw(x);
    }
    sum = block_sum<kAttnThreads>(sum, redd);
    if (sum >= 1.0)
      lo = mid;
    else
      hi = mid;
  }
  float tau = lo;
  if (ALPHA_KIND != 3) {
    // closed form on the support S = {z' > tau}, iterated to a fixed point (shifted by mx)
    int prev = -1;
    for (int it = 0; it < 16; ++it) {
      double k = 0.0, s1 = 0.0, s2 = 0.0;
      for (int i = tid; i < n; i += kAttnThreads) {
        if (cz[i] > tau) {
          const double y = (double)cz[i] - (double)mx;
          k += 1.0;
          s1 += y;
          s2 += y * y;
        }
      }
      k = block_sum<kAttnThreads>(k, redd);
      s1 = block_sum<kAttnThreads>(s1, redd);
      s2 = block_sum<kAttnThreads>(s2, redd);
      if (k <= 0.0 || (int)k == prev) break;
      prev = (int)k;
      double ty;
      if (ALPHA_KIND == 2) {
        ty = (s1 - 1.0) / k;
      } else {
        const double Mk = s1 / k, Qk = s2 / k, dk = (1.0 - k * (Qk - Mk * Mk)) / k;
        if (dk < 0.0) break;
        ty = Mk - sqrt(dk);
      }
      tau = (float)((double)mx + ty);
    }
  }
  // weights and normalisation (alpha outside {1.5, 2}: renormalise the bisection weights)
  double psum = 0.0;
  for (int i = tid; i < n; i += kAttnThreads) {
    const float x = cz[i] - tau;
    const float p = x > 0.0f ? pw(x) : 0.0f;
    cz[i] = p;
    psum += p;
  }
  psum = block_sum<kAttnThreads>(psum, redd);
  const float norm = (ALPHA_KIND == 3 && psum > 0.0) ? (float)(1.0 / psum) : 1.0f;
  // p V over rows with p > 0; row groups take entries round-robin
  const int lr = lane % RL::LPR, rg = wave * RL::RPW + lane / RL::LPR;
  const int L = seq_len(c, b);
  RowMap rm{sel_idx + (size_t)unit * cap, c.bt + (size_t)b * c.maxP, gran, c.S, c.Hkv, g, D, L, num_pages(c, L)};
  const T *V = static_cast<const T *>(c.v);
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
  for (int i = rg; i < n; i += RL::RGB) {
    const float p = cz[i] * norm;
    if (p <= 0.0f) continue;
    const int slot = cslot[i];
    const int item = slot / rows_per_item;
    const long long off = rm.row_offset(item, slot - item * rows_per_item);
    if (off < 0) continue;
    float vx[8];
    Elem<T>::load8(V + off + lr * 8, vx);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = fmaf(p, vx[j], acc[j]);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float a = acc[j];
#pragma unroll
    for (int oo = RL::LPR; oo < kWave; oo <<= 1) a += __shfl_xor(a, oo, kWave);
    acc[j] = a;
  }
  if (lane < RL::LPR)
#pragma unroll
    for (int j = 0; j < 8; ++j) s_acc[wave][lr * 8 + j] = acc[j];
  __syncthreads();
  for (int j = tid; j < D; j += kAttnThreads) {
    float a = 0.0f;
#pragma unroll
    for (int w = 0; w < kAttnThreads / kWave; ++w) a += s_acc[w][j];
    o[j] = a;
  }
}

// ---------------------------------------------------------------- launchers

#define SKV_ATTN_DISPATCH_G(G, ...)                      \
  switch (G) {                                           \
    case 1: { constexpr int GG = 1; __VA_ARGS__; } break; \
    case 2: { constexpr int GG = 2; __VA_ARGS__; } break; \
    case 4: { constexpr int GG = 4; __VA_ARGS__; } break; \
    case 8: { constexpr int GG = 8; __VA_ARGS__; } break; \
    default: return hipErrorInvalidValue;                \
  }

template <typename T, int D>
static hipError_t attn_typed(const AttnArgs &a, hipStream_t st) {
  const CacheView &c = a.c;
  const T *q = static_cast<const T *>(a.q);
  const dim3 grid(a.nsplit, c.B * c.Hkv);
  if (a.alpha == 1.0f) {
    const float scale_log2 = a.sm_scale * 1.4426950408889634f;
    SKV_ATTN_DISPATCH_G(c.G, attn_softmax_kernel<T, D, GG><<<grid, kAttnThreads, 0, st>>>(
                                 c, q, a.sel_idx, a.sel_count, a.cap, a.gran, a.spi, a.nsplit, scale_log2, a.part, a.out))
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nsplit == 1) return e;
    attn_combine_kernel<D><<<c.B * c.Hq, D, 0, st>>>(c, a.sel_count, a.cap, a.spi, a.nsplit, a.part, a.out);
    return hipGetLastError();
  }
  const int rps = a.spi * (a.gran ? 1 : c.S);
  const size_t lds = sizeof(float) * (size_t)c.G * rps;
  const float zscale = a.sm_scale * (a.alpha - 1.0f);
  SKV_ATTN_DISPATCH_G(c.G, attn_entmax_logits_kernel<T, D, GG><<<grid, kAttnThreads, lds, st>>>(
                               c, q, a.sel_idx, a.sel_count, a.cap, a.gran, a.spi, a.nsplit, zscale, a.cand,
                               a.cand_cnt, a.cand_max))
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int kind = a.alpha == 1.5f ? 1 : (a.alpha == 2.0f ? 2 : 3);
  const dim3 g2(c.B * c.Hq);
  if (kind == 1)
    attn_entmax_solve_kernel<T, D, 1><<<g2, kAttnThreads, 0, st>>>(c, a.sel_idx, a.sel_count, a.cap, a.gran, a.spi,
                                                                    a.nsplit, a.alpha, a.cand, a.cand_cnt, a.cand_max,
                                                                    a.out);
  else if (kind == 2)
    attn_entmax_solve_kernel<T, D, 2><<<g2, kAttnThreads, 0, st>>>(c, a.sel_idx, a.sel_count, a.cap, a.gran, a.spi,
                                                                    a.nsplit, a.alpha, a.cand, a.cand_cnt, a.cand_max,
                                                                    a.out);
  else
    attn_entmax_solve_kernel<T, D, 3><<<g2, kAttnThreads, 0, st>>>(c, a.sel_idx, a.sel_count, a.cap, a.gran, a.spi,
                                                                    a.nsplit, a.alpha, a.cand, a.cand_cnt, a.cand_max,
                                                                    a.out);
  return hipGetLastError();
}

hipError_t launch_attn(const AttnArgs &a, hipStream_t st) {
  if (a.dtype == 0) return a.c.D == 64 ? attn_typed<float, 64>(a, st) : attn_typed<float, 128>(a, st);
  return a.c.D == 64 ? attn_typed<uint16_t, 64>(a, st) : attn_typed<uint16_t, 128>(a, st);
}

}  // namespace skv
