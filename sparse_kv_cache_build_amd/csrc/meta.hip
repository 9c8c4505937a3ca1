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

// Projected keys ("Joint Subspace Sparse Attention": keys kept in the shared rank-r subspace),
// kproj[row][i] = RN_bf16(sum_j P[i][j] * K[row][j]), the float64 sum taken over j = 0..d-1 in
// that order from 0 (each product of a float and a cache element is exact in float64).
// Register-blocked: a wave owns 8 outputs i and 512 tokens of one (sequence, KV head), token
// u * 64 + lane in slot u of each lane, and keeps the 64 float64 accumulators in registers. Per
// coordinate it reads its 8 P values as float64 broadcasts from LDS and converts each token's K
// value once, so every conversion feeds 8 fma and every P read feeds 8 tokens. The workgroup's
// waves share one tile of tokens (SUB tiles of 512 for r = 16, whose 16 outputs take two waves per
// tile). K goes from global memory straight to LDS (global_load_lds, 16 bytes a lane, so that each
// instruction's lanes fill consecutive LDS slots) in chunks of 32 bytes per row, double-buffered;
// each lane picks the piece for its slot such that the two pieces of a row trade places in every
// other group of four rows, which lets 8 consecutive rows read their pieces conflict-free. Tokens
// covered: [0, L) for a build, the last `tail` of them for an append. The P slab in LDS holds up
// to 32 outputs; r = 64 takes two slabs per tile.
constexpr int kProjTok = 8, kProjOut = 8, kProjSlab = 32, kProjTilesPerWg = 4;

template <typename T>
__device__ __forceinline__ float proj_elem(const uint4 &w, int e) {
  const uint32_t x = e / 2 == 0 ? w.x : e / 2 == 1 ? w.y : e / 2 == 2 ? w.z : w.w;
  return (e & 1) ? bf16_hi(x) : bf16_lo(x);
}
template <>
__device__ __forceinline__ float proj_elem<float>(const uint4 &w, int e) {
  return __uint_as_float(e == 0 ? w.x : e == 1 ? w.y : e == 2 ? w.z : w.w);
}

// 16 bytes per lane from global memory into LDS: lane i of the wave writes lds_base + 16 i
// (lds_base uniform over the wave). The operands go through void pointers: with typed pointers the
// host pass of a kernel template drops the launch stub.
__device__ __forceinline__ void skv_load_lds16(const void *src, void *lds_base) {
  __builtin_amdgcn_global_load_lds(const_cast<void *>(src), lds_base, 16, 0, 0);
}

// piece (0 or 1) of tile row rho that sits in its LDS slot `bit` (and, the map being its own
// inverse, the slot that piece `bit` of the row sits in)
__device__ __forceinline__ int proj_piece(int rho, int bit) { return bit ^ ((rho >> 2) & 1); }

// row index (into K and kproj, in rows of the cache) of token tau of sequence b, KV head g
__device__ __forceinline__ uint32_t proj_row(const CacheView &c, int b, int g, int tau) {
  const int p = tau / c.S, t = tau - p * c.S;
  return ((uint32_t)c.bt[(size_t)b * c.maxP + p] * c.Hkv + g) * c.S + t;
}

template <typename T, int D, int SUB>
__global__ __launch_bounds__(256, 2) void meta_proj_kernel(CacheView c, int tail, int r, const float *__restrict__ proj,
                                                           uint16_t *__restrict__ kproj) {
  constexpr int PPJ = 16 / sizeof(T);          // coordinates per 16-byte piece
  constexpr int CC = 2 * PPJ;                  // coordinates per staged chunk (32 bytes per row)
  constexpr int NCH = D / CC;                  // chunks per row
  constexpr int TT = SUB * 64 * kProjTok;      // tokens per tile
  constexpr int NL = TT * 2 / 256;             // staging loads per thread and chunk
  constexpr int SLAB = SUB == 2 ? 16 : kProjSlab;
  __shared__ uint4 ks[2][TT * 2];                      // [buffer][row * 2 + slot]
  __shared__ double2 pslab[SLAB / kProjOut][D][kProjOut / 2];
  const int b = blockIdx.y / c.Hkv, g = blockIdx.y % c.Hkv;
  const int L = seq_len(c, b);
  const int lo = tail > 0 ? max(0, L - tail) : 0, ntok = L - lo;
  const int nslab = r / SLAB, obs = SLAB / kProjOut;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64), lane = threadIdx.x % 64;
  const int ob = wave % obs, sub = wave / obs;
  const T *K = static_cast<const T *>(c.k);
  for (int it = 0; it < kProjTilesPerWg; ++it) {
    const int tile0 = (blockIdx.x * kProjTilesPerWg + it) * TT;
    if (tile0 >= ntok) break;  // uniform over the workgroup
    // staging load k of this thread fills slot threadIdx.x % 2 of tile row threadIdx.x / 2 + 128 k
    // (LDS slots 64 (wave + 4 k) + lane); a missing token stages the tile's first row instead
    const T *src[NL];
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      const int rho = (int)threadIdx.x / 2 + 128 * k, tok = tile0 + rho;
      src[k] = K + (size_t)proj_row(c, b, g, lo + (tok < ntok ? tok : tile0)) * D + proj_piece(rho, threadIdx.x & 1) * PPJ;
    }
    const int tbase = tile0 + sub * 64 * kProjTok;
    const bool live = tbase < ntok;
    const int rbase = sub * 64 * kProjTok + lane;  // tile row of slot u: rbase + 64 u
    for (int s = 0; s < nslab; ++s) {
      __syncthreads();  // the previous tile's or slab's LDS contents are no longer read
      if (nslab > 1 || it == 0) {
        double *pd = &pslab[0][0][0].x;
        for (int e = threadIdx.x; e < SLAB * D; e += blockDim.x) {
          const int i = e / D, j = e - i * D;
          pd[((i / kProjOut) * D + j) * kProjOut + i % kProjOut] = proj[(size_t)(s * SLAB + i) * D + j];
        }
      }
#pragma unroll
      for (int k = 0; k < NL; ++k) skv_load_lds16(src[k], &ks[0][64 * (wave + 4 * k)]);
      double acc[kProjTok][kProjOut];
#pragma unroll
      for (int u = 0; u < kProjTok; ++u)
#pragma unroll
        for (int i = 0; i < kProjOut; ++i) acc[u][i] = 0.0;
#pragma unroll 1
      for (int ch = 0; ch < NCH; ++ch) {
        __builtin_amdgcn_s_waitcnt(0);  // this thread's loads of chunk ch are in LDS
        __syncthreads();                // everyone's are, and chunk ch - 1 is no longer read
        if (ch + 1 < NCH) {
#pragma unroll
          for (int k = 0; k < NL; ++k)
            skv_load_lds16(src[k] + (ch + 1) * CC, &ks[(ch + 1) & 1][64 * (wave + 4 * k)]);
        }
        if (!live) continue;
        const uint4 *kb = ks[ch & 1];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          uint4 raw[kProjTok];
#pragma unroll
          for (int u = 0; u < kProjTok; ++u) {
            const int rho = rbase + 64 * u;
            raw[u] = kb[rho * 2 + proj_piece(rho, q)];
          }
#pragma unroll
          for (int e = 0; e < PPJ; ++e) {
            const int j = ch * CC + q * PPJ + e;
            double pv[kProjOut];
#pragma unroll
            for (int i = 0; i < kProjOut / 2; ++i) {
              const double2 w = pslab[ob][j][i];
              pv[2 * i] = w.x;
              pv[2 * i + 1] = w.y;
            }
#pragma unroll
            for (int u = 0; u < kProjTok; ++u) {
              const double kv = (double)proj_elem<T>(raw[u], e);
#pragma unroll
              for (int i = 0; i < kProjOut; ++i) acc[u][i] = fma(pv[i], kv, acc[u][i]);
            }
          }
        }
      }
      if (!live) continue;
#pragma unroll
      for (int u = 0; u < kProjTok; ++u) {
        const int tok = tbase + u * 64 + lane;
        if (tok >= ntok) continue;
        uint32_t w[kProjOut / 2];
#pragma unroll
        for (int i = 0; i < kProjOut / 2; ++i)
          w[i] = (uint32_t)f64_to_bf16(acc[u][2 * i]) | ((uint32_t)f64_to_bf16(acc[u][2 * i + 1]) << 16);
        *reinterpret_cast<uint4 *>(kproj + (size_t)proj_row(c, b, g, lo + tok) * r + s * SLAB + ob * kProjOut) =
            make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
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
    const int slab = min(r, kProjSlab);
    const int sub = 4 / (slab / kProjOut);  // 512-token tiles per workgroup tile: 2 for r = 16
    const int tile_tok = sub * 64 * kProjTok;
    const long maxtok = tail > 0 ? min((long)tail, (long)c.maxP * c.S) : (long)c.maxP * c.S;
    const long tiles = (maxtok + tile_tok - 1) / tile_tok;
    const dim3 g2((unsigned)((tiles + kProjTilesPerWg - 1) / kProjTilesPerWg), c.B * c.Hkv);
#define SKV_PROJ(TT, DD, SS) meta_proj_kernel<TT, DD, SS><<<g2, 256, 0, st>>>(c, tail, r, proj, kproj)
#define SKV_PROJ_D(TT, SS) \
  if (c.D == 64) SKV_PROJ(TT, 64, SS); else SKV_PROJ(TT, 128, SS);
    if (dtype == 0) {
      if (sub == 2) { SKV_PROJ_D(float, 2) } else { SKV_PROJ_D(float, 1) }
    } else {
      if (sub == 2) { SKV_PROJ_D(uint16_t, 2) } else { SKV_PROJ_D(uint16_t, 1) }
    }
#undef SKV_PROJ_D
#undef SKV_PROJ
  }
  return hipGetLastError();
}

}  // namespace skv
