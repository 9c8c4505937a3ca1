// Attention over the selected KV only ("EntmaxKV" summary s2.C; softmax is the comparator of
// its s1 and s3). Token-granular selections read rows in place through block_table, with no
// gathered copy ("Joint Subspace Sparse Attention" abstract).
//
// Work decomposition (split-K over the selection): the unit's selected items (pages or tokens)
// are spread evenly over its nsplit splits (ceil(count / nsplit) each, never more than the
// planned `spi`, so that a selection shorter than the capacity still keeps every split busy);
// block (split, unit) takes one such run of consecutive items of unit (b, g) and all G query
// heads of g. Inside a block a
// row (one token's d coordinates) is read by a group of D/8 lanes, 8 coordinates per lane
// (16-byte loads for bf16), so a wave covers 4 (d = 128) or 8 (d = 64) rows per step and the
// block's 4 waves 16 or 32 rows. q . k is a per-lane partial dot product summed over the lane
// group with DPP moves.
//
// softmax: every lane group keeps an online (max, sum, acc) state per head, rescaled only when a
//          logit exceeds the running reference by 2^32 (in log2 units), then the groups are
//          merged in the block and across splits by a fixed-order log-sum-exp combine.
// entmax:  pass 1 writes, per (unit, head, split), the split's maximum of z' = (alpha-1) z and the
//          (z', row) pairs with z' > max - 1, in row order (row: the V row's index, so the solve
//          reads V without going back through the selection and the block table). Since the global threshold satisfies
//          tau >= max_all z' - 1, no other row can carry weight. The solve kernel (one block per
//          query head) keeps the pairs with z' > max_all - 1, bisects tau, refines it with the
//          closed form on the support (alpha = 2, 1.5), and accumulates p v reading V rows with
//          p > 0 only.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace skv {

// Items per split for a unit with `count` selected items (at most spi when count <= cap).
__device__ __forceinline__ int items_per_split(int count, int nsplit) {
  return max(1, (count + nsplit - 1) / nsplit);
}
// The same for the entmax passes, with at least two pages per split (never more than the planned
// spi, so a split stays within its LDS and list capacity): a short selection then runs as fewer,
// fuller partitions, each with fewer lists for the solve to merge.
__device__ __forceinline__ int entmax_items_per_split(int count, int nsplit, int spi, int rows_per_item) {
  const int least = min(spi, rows_per_item > 1 ? 2 : 1);
  return max(least, (count + nsplit - 1) / nsplit);
}

constexpr int kAttnThreads = 256;

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
    return offset_of(sel[item], t_in_page);
  }
  // the row's index in K / V ([Nphys, Hkv, S] rows of D elements), or -1
  __device__ __forceinline__ long long row_index(int item, int t_in_page) const {
    const long long o = offset_of(sel[item], t_in_page);
    return o < 0 ? -1 : o / D;
  }
  // the same from the selection entry e (a token, or a page) already read
  __device__ __forceinline__ long long offset_of(int e, int t_in_page) const {
    int page, t;
    if (gran) {
      if (e < 0 || e >= L) return -1;
      page = e / S;
      t = e - page * S;
    } else {
      page = e;
      if (page < 0 || page >= P) return -1;
      t = t_in_page;
      if (t >= min(S, L - page * S)) return -1;
    }
    const long long phys = bt[page];
    return ((phys * Hkv + g) * S + t) * (long long)D;
  }
};

// ---------------------------------------------------------------- softmax, split-K

// NTL: K and V rows loaded non-temporally. Page selections read runs of S consecutive rows (4 KiB
// at S = 16, d = 128), where the non-temporal hint pays; token selections read scattered 256-byte
// rows, which plain loads serve better (token128k 31.7 -> 29.6 us), as for the reference gather.
template <typename T, int D, int G, bool NTL>
__global__ __launch_bounds__(kAttnThreads) void attn_softmax_kernel(
    CacheView c, const T *__restrict__ q, const int32_t *__restrict__ sel_idx, const int32_t *__restrict__ sel_count,
    int cap, int gran, int spi, int nsplit, float scale_log2, float *__restrict__ part, float *__restrict__ out) {
  using RL = RowLayout<D>;
  constexpr int UNR = 2;   // rows per lane group in flight (three or four measured slower)
  __shared__ float s_m[G][RL::RGB];
  __shared__ float s_l[G][RL::RGB];
  __shared__ float s_acc[kAttnThreads / kWave][G][D];
  extern __shared__ long long roff[];   // element offset of each row of the partition, -1 if none
  const int split = blockIdx.x, unit = blockIdx.y, b = unit / c.Hkv, g = unit - b * c.Hkv;
  const int count = min(max(sel_count[unit], 0), cap);
  const int ipb = items_per_split(count, nsplit);
  const int it0 = split * ipb;
  if (it0 >= count && !(split == 0 && nsplit == 1)) return;  // empty split (count is known to the combine)
  const int it1 = min(count, it0 + ipb);
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int lr = lane % RL::LPR, rg = wave * RL::RPW + lane / RL::LPR;
  const int L = seq_len(c, b);
  RowMap rm{sel_idx + (size_t)unit * cap, c.bt + (size_t)b * c.maxP, gran, c.S, c.Hkv, g, D, L, num_pages(c, L)};
  const int rows_per_item = gran ? 1 : c.S;
  const int NR = max(0, it1 - it0) * rows_per_item;

  Packed8<T> qv[G];
#pragma unroll
  for (int h = 0; h < G; ++h) qv[h].load(q + ((size_t)b * c.Hq + g * G + h) * D + lr * 8);
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
  // one row's update from its G logits (the group's summed dot products); the exponents are at
  // most 32, and weights below 2^-126 of the reference (flushed to zero by v_exp_f32) add nothing
  // visible next to the reference row's weight of at least 1
  auto accumulate = [&](const float *zdot, const Packed8<T> &vp) {
    float vx[8];   // V stays packed until its row is used
#pragma unroll
    for (int j = 0; j < 8; ++j) vx[j] = vp.at(j);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float z = zdot[h] * scale_log2;
      if (z > mref[h] + 32.0f) {  // rescale the state to a new reference
        const float corr = __builtin_amdgcn_exp2f(mref[h] - z);
        l[h] *= corr;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[h][j] *= corr;
        mref[h] = z;
      }
      const float p = __builtin_amdgcn_exp2f(z - mref[h]);
      l[h] += p;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[h][j] = fmaf(p, vx[j], acc[h][j]);
    }
  };
  // row offsets first (selection entry -> block table -> row), then UNR rows per lane group per
  // step with all their loads in flight before any is used; the UNR * G dot products are summed
  // over the lane group together (one level for all of them, then the next)
  for (int r = tid; r < NR; r += kAttnThreads) roff[r] = row_off(r);
  __syncthreads();
  for (int r = rg; r < NR; r += UNR * RL::RGB) {
    long long o[UNR];
    Packed8<T> kx[UNR], vx[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int ru = r + u * RL::RGB;
      o[u] = ru < NR ? roff[ru] : -1;
      if (o[u] >= 0) {
        if constexpr (NTL) {
          kx[u].load_once(K + o[u] + lr * 8);
          vx[u].load_once(V + o[u] + lr * 8);
        } else {
          kx[u].load(K + o[u] + lr * 8);
          vx[u].load(V + o[u] + lr * 8);
        }
      } else {
        kx[u].zero();
      }
    }
    float zd[UNR * G];
#pragma unroll
    for (int u = 0; u < UNR; ++u)
#pragma unroll
      for (int h = 0; h < G; ++h) zd[u * G + h] = qv[h].dot(kx[u]);
    group_sum_n<RL::LPR>(zd);
#pragma unroll
    for (int u = 0; u < UNR; ++u)
      if (o[u] >= 0) accumulate(zd + u * G, vx[u]);
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
  const int ipb = items_per_split(count, nsplit);
  const int ns = min(nsplit, (count + ipb - 1) / ipb);
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

// Logits of an entmax partition in LDS: head h, row r at h * 4 q + (r mod 4) q + r / 4 with
// q = ceil(rps / 4). A thread of the compaction below reads a run of consecutive rows; with this
// layout the threads of a wave read consecutive words at every step, so the reads are free of
// bank conflicts (row-major, a stride of four words, they conflicted four ways).
struct ZLayout {
  int q;
  __device__ __forceinline__ explicit ZLayout(int rps) : q((rps + 3) >> 2) {}
  __device__ __forceinline__ int at(int h, int r) const { return h * 4 * q + (r & 3) * q + (r >> 2); }
  __device__ __forceinline__ int floats(int g) const { return g * 4 * q; }
};

// Per-head maximum and ordered compaction of z' > max - 1 for pass 1 (logits of the partition
// in LDS as ZLayout; rows past NR are not read). All G heads at once: every thread takes a
// contiguous chunk of rows, so the thread order is the row order; the survivor counts of the G
// heads are combined over the block with one barrier. The per-wave maxima of the heads are in
// wmax: filled by the caller when have_max (then published by a barrier before the call), else
// computed here from the LDS logits. rowid(r) is the K/V row index of partition row r (rows with a
// finite logit are valid ones). Every thread of the block must call it.
template <int G, typename RowId>
__device__ __forceinline__ void entmax_compact(const float *zs, ZLayout zl, int rps, int NR, int unit, int split,
                                               int nsplit, RowId rowid, float (*wmax)[G], bool have_max,
                                               float2 *__restrict__ cand, int32_t *__restrict__ cand_cnt,
                                               float *__restrict__ cand_max) {
  constexpr int NW = kAttnThreads / kWave;
  __shared__ int wcnt[NW][G];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const int per = (NR + kAttnThreads - 1) / kAttnThreads;
  const int r0 = min(NR, tid * per), r1 = min(NR, r0 + per);
  float mx[G];
  if (!have_max) {
#pragma unroll
    for (int h = 0; h < G; ++h) mx[h] = -INFINITY;
    for (int r = r0; r < r1; ++r)
#pragma unroll
      for (int h = 0; h < G; ++h) mx[h] = fmaxf(mx[h], zs[zl.at(h, r)]);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float m = wave_max_dpp(mx[h]);
      if (lane == 0) wmax[w][h] = m;
    }
    __syncthreads();
  }
  int nk[G], incl[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float m = wmax[0][h];
#pragma unroll
    for (int i = 1; i < NW; ++i) m = fmaxf(m, wmax[i][h]);
    mx[h] = m;
    nk[h] = 0;
  }
  for (int r = r0; r < r1; ++r)
#pragma unroll
    for (int h = 0; h < G; ++h) nk[h] += zs[zl.at(h, r)] > mx[h] - 1.0f ? 1 : 0;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    incl[h] = wave_incl_scan(nk[h]);
    if (lane == kWave - 1) wcnt[w][h] = incl[h];
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < G; ++h) {
    int before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const int t = wcnt[i][h];
      before += i < w ? t : 0;
      tot += t;
    }
    const size_t lid = ((size_t)unit * G + h) * nsplit + split;
    float2 *cl = cand + lid * rps;
    int pos = before + incl[h] - nk[h];
    for (int r = r0; r < r1; ++r) {
      const float z = zs[zl.at(h, r)];
      if (z > mx[h] - 1.0f) cl[pos++] = make_float2(z, __uint_as_float(rowid(r)));
    }
    if (tid == 0) {
      cand_cnt[lid] = tot;
      cand_max[lid] = mx[h];
    }
  }
}


template <typename T, int D, int G>
__global__ __launch_bounds__(kAttnThreads) void attn_entmax_logits_kernel(
    CacheView c, const T *__restrict__ q, const int32_t *__restrict__ sel_idx, const int32_t *__restrict__ sel_count,
    int cap, int gran, int spi, int nsplit, float zscale, float2 *__restrict__ cand, int32_t *__restrict__ cand_cnt,
    float *__restrict__ cand_max) {
  using RL = RowLayout<D>;
  extern __shared__ float zs[];  // logits (ZLayout), then [rps] row offsets (8-byte aligned)
  __shared__ float wmax[kAttnThreads / kWave][G];
  const int split = blockIdx.x, unit = blockIdx.y, b = unit / c.Hkv, g = unit - b * c.Hkv;
  const int count = min(max(sel_count[unit], 0), cap);
  const int rows_per_item = gran ? 1 : c.S;
  const int rps = spi * rows_per_item;
  const ZLayout zl(rps);
  const int ipb = entmax_items_per_split(count, nsplit, spi, rows_per_item);
  const int it0 = split * ipb, it1 = min(count, it0 + ipb);
  if (it0 >= count) return;   // past the splits in use: the solve reads none of its lists
  const int NR = max(0, it1 - it0) * rows_per_item;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int lr = lane % RL::LPR, rg = wave * RL::RPW + lane / RL::LPR;
  const int L = seq_len(c, b);
  RowMap rm{sel_idx + (size_t)unit * cap, c.bt + (size_t)b * c.maxP, gran, c.S, c.Hkv, g, D, L, num_pages(c, L)};

  Packed8<T> qv[G];
#pragma unroll
  for (int h = 0; h < G; ++h) qv[h].load(q + ((size_t)b * c.Hq + g * G + h) * D + lr * 8);
  const T *K = static_cast<const T *>(c.k);
  auto row_off = [&](int r) -> long long {
    if (r >= NR) return -1;
    const int it = r / rows_per_item;
    return rm.row_offset(it0 + it, r - it * rows_per_item);
  };
  auto logits = [&](int r, long long off, const Packed8<T> &kx) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float z = 0.0f;
      if (off >= 0) z = group_sum<RL::LPR>(qv[h].dot(kx)) * zscale;
      if (lr == h % RL::LPR) zs[zl.at(h, r)] = off >= 0 ? z : -INFINITY;
    }
  };
  long long *roff = reinterpret_cast<long long *>(zs + ((zl.floats(G) + 1) & ~1));
  for (int r = tid; r < NR; r += kAttnThreads) roff[r] = row_off(r);
  __syncthreads();
  constexpr int UNR = 4;
  for (int r = rg; r < NR; r += UNR * RL::RGB) {
    long long o[UNR];
    Packed8<T> kx[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int ru = r + u * RL::RGB;
      o[u] = ru < NR ? roff[ru] : -1;
      if (o[u] >= 0) kx[u].load_once(K + o[u] + lr * 8);
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u)
      if (r + u * RL::RGB < NR) logits(r + u * RL::RGB, o[u], kx[u]);
  }
  __syncthreads();
  auto rowid = [&](int r) { return (uint32_t)(roff[r] / D); };
  entmax_compact<G>(zs, zl, rps, NR, unit, split, nsplit, rowid, wmax, false, cand, cand_cnt, cand_max);
}

// Entmax pass 1 for bf16 caches on the matrix cores, on tiles of 8 rows. A dot product may take
// its coordinates in any order, so each v_mfma_f32_16x16x32_bf16 covers 64 coordinates of 8 rows:
// A row m = 2 p + s holds coordinates 64 kb + 32 s + [0, 32) of tile row p, B column c = n + 8 s'
// holds the same slice (s') of head n's q (heads past G zero), and C[2 p + s][n + 8 s'] is a
// partial dot product. The logit of row p and head n is C[2p][n] + C[2p + 1][n + 8]: the two
// halves sit in lanes c and c + 8 of the same row of 16 lanes and are added with one DPP move.
// Lane l supplies A[l % 16][8 (l / 16) ..], so the 8 lanes of tile row p read 128 consecutive
// bytes and one load instruction reads 8 whole rows of 128-byte lines (a 16-row tile would split
// every line over two instructions), and since every line is then read whole by one instruction
// the loads are marked non-temporal. d/64 products per tile. Each wave takes every fourth tile,
// with the K loads of UNR tiles in flight before their products. bf16 products are exact and the
// sums are float32, as on the VALU path.

template <int D, int G>
__global__ __launch_bounds__(kAttnThreads) void attn_entmax_logits_mfma_kernel(
    CacheView c, const uint16_t *__restrict__ q, const int32_t *__restrict__ sel_idx,
    const int32_t *__restrict__ sel_count, int cap, int gran, int spi, int nsplit, float zscale,
    float2 *__restrict__ cand, int32_t *__restrict__ cand_cnt, float *__restrict__ cand_max) {
  static_assert(G <= 8, "the B columns hold 8 heads times two coordinate halves");
  constexpr int KB = D / 64, UNR = 4, NWV = kAttnThreads / kWave;
  extern __shared__ float zs[];  // logits (ZLayout), then [rps] row offsets (8-byte aligned)
  __shared__ float wmax[kAttnThreads / kWave][G];
  const int split = blockIdx.x, unit = blockIdx.y, b = unit / c.Hkv, g = unit - b * c.Hkv;
  const int count = min(max(sel_count[unit], 0), cap);
  const int rows_per_item = gran ? 1 : c.S;
  const int rps = spi * rows_per_item;
  const ZLayout zl(rps);
  const int ipb = entmax_items_per_split(count, nsplit, spi, rows_per_item);
  const int it0 = split * ipb, it1 = min(count, it0 + ipb);
  if (it0 >= count) return;   // past the splits in use: the solve reads none of its lists
  const int NR = max(0, it1 - it0) * rows_per_item;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int L = seq_len(c, b);
  RowMap rm{sel_idx + (size_t)unit * cap, c.bt + (size_t)b * c.maxP, gran, c.S, c.Hkv, g, D, L, num_pages(c, L)};
  // this lane's column of B: head n, coordinate half hs; its A row: tile row pr, half hs too
  // (m = lane % 16 = 2 pr + hs); its 8 coordinates of the 32 of a half start at kq
  const int col = lane & 15, n = col & 7, hs = col >> 3, kq = 8 * (lane >> 4);
  const int pr = col >> 1, ha = col & 1;
  bf16x8_t qb[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    uint4 w = make_uint4(0u, 0u, 0u, 0u);
    if (n < G)
      w = *reinterpret_cast<const uint4 *>(q + ((size_t)b * c.Hq + g * G + n) * D + 64 * kb + 32 * hs + kq);
    qb[kb] = __builtin_bit_cast(bf16x8_t, w);
  }
  // row indices (not element offsets: half the LDS, which keeps four workgroups per CU at G = 8);
  // every row of a cache that fits in memory has an index below 2^32 - 1
  uint32_t *ridx = reinterpret_cast<uint32_t *>(zs + zl.floats(G));
  for (int r = tid; r < NR; r += kAttnThreads) {
    const int it = r / rows_per_item;
    const long long ri = rm.row_index(it0 + it, r - it * rows_per_item);
    ridx[r] = ri < 0 ? 0xffffffffu : (uint32_t)ri;
  }
  __syncthreads();
  const uint16_t *K = static_cast<const uint16_t *>(c.k);
  const int ntile = (NR + 7) / 8;
  float mxl = -INFINITY;   // the largest logit of head n among this lane's rows (lanes col < G)
  for (int t0 = wave; t0 < ntile; t0 += NWV * UNR) {
    bf16x8_t a[UNR][KB];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int row = (t0 + u * NWV) * 8 + pr;
      const uint32_t ri = row < NR ? ridx[row] : 0xffffffffu;
      const uint16_t *kr = K + (size_t)ri * D + 32 * ha + kq;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        uint4 w = make_uint4(0u, 0u, 0u, 0u);
        if (ri != 0xffffffffu) w = ld_once(reinterpret_cast<const uint4 *>(kr + 64 * kb));
        a[u][kb] = __builtin_bit_cast(bf16x8_t, w);
      }
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int tb = (t0 + u * NWV) * 8;
      if (tb >= NR) break;
      f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][kb], qb[kb], acc, 0, 0, 0);
      // acc[i] = C[4 (lane / 16) + i][col]: tile row 2 (lane / 16) + i / 2, A half i % 2. The
      // second half of head n's dot product is in lane col + 8 (row_ror:8 within the 16 lanes),
      // taken by every lane so that each source lane is active
      float z[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        z[i] = acc[2 * i] +
               __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(acc[2 * i + 1]), 0x128, 0xf, 0xf, false));
      if (col < G) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int r = tb + 2 * (lane >> 4) + i;
          if (r < NR) {
            const float v = ridx[r] != 0xffffffffu ? z[i] * zscale : -INFINITY;
            zs[zl.at(n, r)] = v;
            mxl = fmaxf(mxl, v);
          }
        }
      }
    }
  }
  // the lanes of head n (n, n + 16, n + 32, n + 48) hold disjoint row sets
  mxl = fmaxf(mxl, __shfl_xor(mxl, 16, kWave));
  mxl = fmaxf(mxl, __shfl_xor(mxl, 32, kWave));
  if (lane < G) wmax[wave][lane] = mxl;
  __syncthreads();
  auto rowid = [&](int r) { return ridx[r]; };
  entmax_compact<G>(zs, zl, rps, NR, unit, split, nsplit, rowid, wmax, true, cand, cand_cnt, cand_max);
}

// ---------------------------------------------------------------- entmax threshold and p V

// One wave per query head. ALPHA_KIND: 1 -> alpha = 1.5, 2 -> alpha = 2, 3 -> any alpha in (1, 2).
//  1. max_all = max of the split maxima; only z' > max_all - 1 can carry weight.
//  2. The per-split pair lists are read as one flat list (split-major, row order) through prefix
//     offsets in LDS, and the survivors are compacted into LDS in that order (ballots). Splits
//     whose maximum is at most max_all - 1 are skipped.
//  3. Bisection on tau over [max_all - 1, max_all - n^(1-alpha)], then the closed form on the
//     support {z' > tau}, iterated until the support size repeats (alpha = 2: tau = (sum z' - 1) / k;
//     alpha = 1.5: tau = mean - sqrt((1 - k var) / k), the smaller root of sum (z' - tau)^2 = 1).
//     For alpha = 1.5 and 2 the bisection stops once no survivor lies in (lo, hi]: the support is
//     then settled. Up to 256 survivors are held in registers; sums over lanes use DPP.
//  4. p = (z' - tau)_+^(1/(alpha-1)) (renormalized for other alpha), out = sum p v over rows with
//     p > 0, read in place at the V rows pass 1 recorded with each pair.
// When the survivors do not fit in LDS, steps 3-4 read the flat list from global memory instead.
constexpr int kSolveCap = 1024;     // survivors staged in LDS
constexpr int kSolveSplits = 2048;  // split offsets staged in LDS (the planner keeps nsplit below)
constexpr int kStageU = 8;          // pair-list entries per lane and staging round

template <typename T, int D, int ALPHA_KIND>
__global__ __launch_bounds__(kWave) void attn_entmax_solve_kernel(
    CacheView c, const int32_t *__restrict__ sel_idx, const int32_t *__restrict__ sel_count, int cap, int gran,
    int spi, int nsplit, float alpha, const float2 *__restrict__ cand, const int32_t *__restrict__ cand_cnt,
    const float *__restrict__ cand_max, float *__restrict__ out) {
  using RL = RowLayout<D>;
  constexpr int RG = kWave / RL::LPR;  // row groups in the wave
  __shared__ float cz[kSolveCap];
  __shared__ uint32_t crow[kSolveCap];   // the survivors' V rows
  __shared__ __align__(8) int soff[kSolveSplits + 1];   // later reused as the support's row offsets
  const int bh = blockIdx.x, b = bh / c.Hq, h = bh - b * c.Hq, g = h / c.G, hh = h - g * c.G;
  const int unit = b * c.Hkv + g;
  const int lane = threadIdx.x;
  const int count = min(max(sel_count[unit], 0), cap);
  const int rows_per_item = gran ? 1 : c.S;
  const int rps = spi * rows_per_item;
  const int ipb = entmax_items_per_split(count, nsplit, spi, rows_per_item);
  const int ns = min(nsplit, (count + ipb - 1) / ipb);
  const size_t lid0 = ((size_t)unit * c.G + hh) * nsplit;
  float *o = out + (size_t)bh * D;

  // the maxima and counts of the first 64 splits are read together (most units have no more)
  float mx = -INFINITY, mx0 = -INFINITY;
  int cnt0 = 0;
  if (lane < ns) {
    mx0 = cand_max[lid0 + lane];
    cnt0 = cand_cnt[lid0 + lane];
  }
  mx = mx0;
  for (int s = lane + kWave; s < ns; s += kWave) mx = fmaxf(mx, cand_max[lid0 + s]);
  mx = wave_max_dpp(mx);
  if (mx == -INFINITY) {  // nothing selected
    for (int j = lane; j < D; j += kWave) o[j] = 0.0f;
    return;
  }
  const float lo_bound = mx - 1.0f;
  // prefix offsets of the split lists (exclusive), 64 splits per step; a split whose maximum is
  // at most max_all - 1 holds no survivor and is left out
  int run = 0;
  for (int s0 = 0; s0 < ns; s0 += kWave) {
    const int s = s0 + lane;
    int cnt = 0;
    if (s0 == 0)
      cnt = mx0 > lo_bound ? cnt0 : 0;
    else if (s < ns && cand_max[lid0 + s] > lo_bound)
      cnt = cand_cnt[lid0 + s];
    const int incl = wave_incl_scan(cnt);
    if (s < ns) soff[s] = run + incl - cnt;
    run += __shfl(incl, kWave - 1, kWave);
  }
  if (lane == 0) soff[ns] = run;
  __syncthreads();
  const int nraw = run;
  // flat entry f -> (split, row) through a binary search of the offsets
  auto entry = [&](int f) -> float2 {
    int lo = 0, hi = ns - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (soff[mid] <= f) lo = mid; else hi = mid - 1;
    }
    return cand[(lid0 + lo) * rps + (f - soff[lo])];
  };
  // survivors into LDS, in flat order; U entries per lane and round (1 when the list fits one
  // round, else kStageU), their splits found by binary searches run side by side (a fixed number
  // of halving steps), then all their loads in flight
  int top = 1;
  while (top < ns) top <<= 1;
  int n = 0;
  auto stage = [&](auto uu) {
    constexpr int U = decltype(uu)::value;
    for (int f0 = 0; f0 < nraw; f0 += U * kWave) {
      int sp[U];
#pragma unroll
      for (int u = 0; u < U; ++u) sp[u] = 0;
      for (int step = top >> 1; step > 0; step >>= 1) {
#pragma unroll
        for (int u = 0; u < U; ++u) {   // soff[ns] = nraw exceeds every entry index read below
          const int f = f0 + u * kWave + lane, m = sp[u] + step;
          sp[u] = soff[min(m, ns)] <= f ? m : sp[u];
        }
      }
      float2 e[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int f = f0 + u * kWave + lane;
        e[u] = f < nraw ? cand[(lid0 + sp[u]) * rps + (f - soff[sp[u]])] : make_float2(-INFINITY, 0.0f);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool keep = e[u].x > lo_bound;
        const uint64_t bal = __ballot(keep);
        const int pos = n + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
        if (keep && pos < kSolveCap) {
          cz[pos] = e[u].x;
          crow[pos] = __float_as_uint(e[u].y);
        }
        n += __popcll(bal);
      }
    }
  };
  if (nraw <= kWave)
    stage(std::integral_constant<int, 1>{});
  else
    stage(std::integral_constant<int, kStageU>{});
  __syncthreads();
  const bool in_lds = n <= kSolveCap;
  const int nn = in_lds ? n : nraw;   // in global mode the unfiltered list is walked (z' <= max - 1 weighs 0)
  auto z_at = [&](int i) -> float { return in_lds ? cz[i] : entry(i).x; };

  const float am1 = alpha - 1.0f, inv = 1.0f / am1;
  auto pw = [&](float x) -> float {
    if (ALPHA_KIND == 1) return x * x;
    if (ALPHA_KIND == 2) return x;
    return powf(x, inv);
  };
  // up to ZR * 64 survivors (the usual case) are also held in registers, lane-strided like cz;
  // empty slots hold -inf and add nothing
  constexpr int ZR = 4;
  const bool in_regs = n <= ZR * kWave;
  float zr[ZR];
#pragma unroll
  for (int j = 0; j < ZR; ++j) {
    const int i = lane + j * kWave;
    zr[j] = (in_regs && i < n) ? cz[i] : -INFINITY;
  }
  // the V row offsets of the register-held survivors
  long long offr[ZR];
#pragma unroll
  for (int j = 0; j < ZR; ++j) {
    const int i = lane + j * kWave;
    offr[j] = (in_regs && i < n) ? (long long)crow[i] * D : -1;
  }
  // 3. bisection; for alpha = 1.5 and 2 it stops as soon as no survivor lies in (lo, hi]: the
  //    support {z' > tau} is then settled and the closed form below gives tau from it
  float lo = lo_bound, hi = mx - powf((float)n, -am1);
  int klo = n, khi = -1;   // survivors above lo and above hi (-1: not counted)
  if (ALPHA_KIND != 3 && in_regs) {   // every survivor above hi: the support is all of them
    int c0 = 0;
#pragma unroll
    for (int j = 0; j < ZR; ++j) c0 += zr[j] > hi ? 1 : 0;
    khi = wave_sum_dpp(c0);
  }
  for (int it = 0; it < 40; ++it) {
    if (ALPHA_KIND != 3 && klo == khi) break;
    if (ALPHA_KIND != 3 && in_regs && khi >= 0 && klo - khi == 1) {
      // one survivor z_j left in (lo, hi]: F at z_j says which side of it tau lies on, and the
      // interval then holds no survivor inside: lo = z_j (tau >= z_j) or hi = z_j (tau < z_j)
      float zj = -INFINITY;
#pragma unroll
      for (int j = 0; j < ZR; ++j) zj = (zr[j] > lo && zr[j] <= hi) ? fmaxf(zj, zr[j]) : zj;
      zj = wave_max_dpp(zj);
      double sj = 0.0;
#pragma unroll
      for (int j = 0; j < ZR; ++j) {
        const float x = zr[j] - zj;
        if (x > 0.0f) sj += (double)pw(x);
      }
      if (wave_sum_dpp(sj) >= 1.0) {
        lo = zj;
        klo = khi;
      } else {
        hi = zj;
      }
      break;
    }
    const float mid = 0.5f * (lo + hi);
    if (mid <= lo || mid >= hi) break;
    double sum = 0.0;
    int cnt = 0;
    if (in_regs) {
#pragma unroll
      for (int j = 0; j < ZR; ++j) {
        const float x = zr[j] - mid;
        if (x > 0.0f) {
          sum += (double)pw(x);
          ++cnt;
        }
      }
    } else {
      for (int i = lane; i < nn; i += kWave) {
        const float x = z_at(i) - mid;
        if (x > 0.0f) {
          sum += (double)pw(x);
          ++cnt;
        }
      }
    }
    sum = wave_sum_dpp(sum);
    cnt = wave_sum_dpp(cnt);
    if (sum >= 1.0) {
      lo = mid;
      klo = cnt;
    } else {
      hi = mid;
      khi = cnt;
    }
  }
  float tau = lo;
  if (ALPHA_KIND != 3) {
    int prev = -1;
    for (int it = 0; it < 16; ++it) {
      double k = 0.0, s1 = 0.0, s2 = 0.0;
      auto add = [&](float z) {
        const double y = (double)z - (double)mx;
        k += 1.0;
        s1 += y;
        s2 += y * y;
      };
      if (in_regs) {
#pragma unroll
        for (int j = 0; j < ZR; ++j)
          if (zr[j] > tau) add(zr[j]);
      } else {
        for (int i = lane; i < nn; i += kWave) {
          const float z = z_at(i);
          if (z > tau) add(z);
        }
      }
      k = wave_sum_dpp(k);
      s1 = wave_sum_dpp(s1);
      s2 = wave_sum_dpp(s2);
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
  float norm = 1.0f;
  if (ALPHA_KIND == 3) {
    double psum = 0.0;
    if (in_regs) {
#pragma unroll
      for (int j = 0; j < ZR; ++j) {
        const float x = zr[j] - tau;
        if (x > 0.0f) psum += pw(x);
      }
    } else {
      for (int i = lane; i < nn; i += kWave) {
        const float x = z_at(i) - tau;
        if (x > 0.0f) psum += pw(x);
      }
    }
    psum = wave_sum_dpp(psum);
    norm = psum > 0.0 ? (float)(1.0 / psum) : 1.0f;
  }
  // p V over rows with p > 0
  const int lr = lane % RL::LPR, rg = lane / RL::LPR;
  const T *V = static_cast<const T *>(c.v);
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
  if (in_lds) {
    // 1. every lane at once: p and the row offset of each survivor, the support compacted in order
    //    (p over cz, offsets over the split offsets, which are no longer needed); entries are read
    //    before any write of the round, and a write position never passes the entries read so far
    long long *voff = reinterpret_cast<long long *>(soff);
    int m = 0;
    if (in_regs) {   // the same from the registers (offsets already resolved)
#pragma unroll
      for (int j = 0; j < ZR; ++j) {
        const float x = zr[j] - tau;
        const bool keep = x > 0.0f && offr[j] >= 0;
        const uint64_t bal = __ballot(keep);
        if (keep) {
          const int pos = m + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
          cz[pos] = pw(x) * norm;
          voff[pos] = offr[j];
        }
        m += __popcll(bal);
      }
    }
    for (int i0 = 0; i0 < (in_regs ? 0 : n); i0 += kWave) {
      const int i = i0 + lane;
      float pv = 0.0f;
      long long off = -1;
      if (i < n) {
        const float x = cz[i] - tau;
        if (x > 0.0f) {
          off = (long long)crow[i] * D;
          pv = pw(x) * norm;
        }
      }
      const bool keep = off >= 0;
      const uint64_t bal = __ballot(keep);
      if (keep) {
        const int pos = m + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
        cz[pos] = pv;
        voff[pos] = off;
      }
      m += __popcll(bal);
    }
    __syncthreads();
    // 2. row groups take the support round-robin, eight rows' V loads in flight per group
    constexpr int UV = 8;
    for (int j0 = rg; j0 < m; j0 += UV * RG) {
      float vx[UV][8];
      float pj[UV];
#pragma unroll
      for (int u = 0; u < UV; ++u) {
        const int j = j0 + u * RG;
        pj[u] = j < m ? cz[j] : 0.0f;
        if (j < m) Elem<T>::load8(V + voff[j] + lr * 8, vx[u]);
      }
#pragma unroll
      for (int u = 0; u < UV; ++u)
        if (j0 + u * RG < m)
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) acc[jj] = fmaf(pj[u], vx[u][jj], acc[jj]);
    }
  } else {
    for (int i = rg; i < nn; i += RG) {   // survivors beyond LDS: walk the flat list
      const float2 e = entry(i);
      const float x = e.x - tau;
      if (!(x > 0.0f)) continue;
      const float p = pw(x) * norm;
      const long long off = (long long)__float_as_uint(e.y) * D;
      float vx[8];
      Elem<T>::load8(V + off + lr * 8, vx);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = fmaf(p, vx[j], acc[j]);
    }
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
    for (int j = 0; j < 8; ++j) o[lr * 8 + j] = acc[j];
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
    const int rps_s = a.spi * (a.gran ? 1 : c.S);
    const size_t lds_s = sizeof(long long) * (size_t)rps_s;
    hipError_t e0 = a.ev.before(st);
    if (e0 != hipSuccess) return e0;
    if (a.gran)
      SKV_ATTN_DISPATCH_G(c.G, attn_softmax_kernel<T, D, GG, false><<<grid, kAttnThreads, lds_s, st>>>(
                                   c, q, a.sel_idx, a.sel_count, a.cap, a.gran, a.spi, a.nsplit, scale_log2, a.part, a.out))
    else
      SKV_ATTN_DISPATCH_G(c.G, attn_softmax_kernel<T, D, GG, true><<<grid, kAttnThreads, lds_s, st>>>(
                                   c, q, a.sel_idx, a.sel_count, a.cap, a.gran, a.spi, a.nsplit, scale_log2, a.part, a.out))
    hipError_t e = a.ev.after(st);
    if (e != hipSuccess || a.nsplit == 1) return e;
    attn_combine_kernel<D><<<c.B * c.Hq, D, 0, st>>>(c, a.sel_count, a.cap, a.spi, a.nsplit, a.part, a.out);
    return hipGetLastError();
  }
  const int rps = a.spi * (a.gran ? 1 : c.S);
  const int zq = (rps + 3) / 4;   // ZLayout of the logits
  const size_t lds = sizeof(float) * (size_t)((c.G * 4 * zq + 1) & ~1) + sizeof(long long) * (size_t)rps;
  const size_t lds_mfma = sizeof(float) * (size_t)(c.G * 4 * zq) + sizeof(uint32_t) * (size_t)rps;   // 32-bit row indices
  const float zscale = a.sm_scale * (a.alpha - 1.0f);
  hipError_t e0 = a.ev.before(st);
  if (e0 != hipSuccess) return e0;
  if constexpr (std::is_same<T, uint16_t>::value) {   // bf16: logits on the matrix cores
    SKV_ATTN_DISPATCH_G(c.G, attn_entmax_logits_mfma_kernel<D, GG><<<grid, kAttnThreads, lds_mfma, st>>>(
                                 c, q, a.sel_idx, a.sel_count, a.cap, a.gran, a.spi, a.nsplit, zscale, a.cand,
                                 a.cand_cnt, a.cand_max))
  } else {
    SKV_ATTN_DISPATCH_G(c.G, attn_entmax_logits_kernel<T, D, GG><<<grid, kAttnThreads, lds, st>>>(
                                 c, q, a.sel_idx, a.sel_count, a.cap, a.gran, a.spi, a.nsplit, zscale, a.cand,
                                 a.cand_cnt, a.cand_max))
  }
  hipError_t e = a.ev.after(st);
  if (e != hipSuccess) return e;
  const int kind = a.alpha == 1.5f ? 1 : (a.alpha == 2.0f ? 2 : 3);
  const dim3 g2(c.B * c.Hq);
  if (kind == 1)
    attn_entmax_solve_kernel<T, D, 1><<<g2, kWave, 0, st>>>(c, a.sel_idx, a.sel_count, a.cap, a.gran, a.spi,
                                                                    a.nsplit, a.alpha, a.cand, a.cand_cnt, a.cand_max,
                                                                    a.out);
  else if (kind == 2)
    attn_entmax_solve_kernel<T, D, 2><<<g2, kWave, 0, st>>>(c, a.sel_idx, a.sel_count, a.cap, a.gran, a.spi,
                                                                    a.nsplit, a.alpha, a.cand, a.cand_cnt, a.cand_max,
                                                                    a.out);
  else
    attn_entmax_solve_kernel<T, D, 3><<<g2, kWave, 0, st>>>(c, a.sel_idx, a.sel_count, a.cap, a.gran, a.spi,
                                                                    a.nsplit, a.alpha, a.cand, a.cand_cnt, a.cand_max,
                                                                    a.out);
  return hipGetLastError();
}

hipError_t launch_attn(const AttnArgs &a, hipStream_t st) {
  if (a.dtype == 0) return a.c.D == 64 ? attn_typed<float, 64>(a, st) : attn_typed<float, 128>(a, st);
  return a.c.D == 64 ? attn_typed<uint16_t, 64>(a, st) : attn_typed<uint16_t, 128>(a, st);
}

}  // namespace skv
