// Page metadata builder ("EntmaxKV" summary s2.A: per-page box bounds and Gaussian moments;
// "Joint Subspace Sparse Attention" abstract: keys cached in a shared low-dimensional subspace).
// Runs once per page at prefill time, and after an append for the pages holding the new tokens
// (tail > 0: only pages holding one of the last `tail` tokens of a sequence, recomputed over all
// their valid tokens, so the result equals a full build of those pages). Off the per-step path.
#include "common.hpp"
#include "launch.hpp"

namespace skv {

// Box, moment and pooled-key builders. Work items are (page, KV head g, 16-byte slice o of the
// key row): V = 16 / sizeof(T) consecutive coordinates, so 64 consecutive items read whole rows
// (256 bytes for d = 128 bf16) and a wave instruction covers several rows. A workgroup takes
// `ppw` consecutive pages of one sequence; each item walks its page's valid tokens in ascending
// order, kMetaRows rows in flight.
//   box:   min / max over the valid tokens from +inf / -inf with strict comparisons, stored as
//          the element bits, the 64-byte blocks of the min row and of the max row alternating
//          ([d / C][2][C], C = 64 bytes).
//   gauss: float64 mean (sum over t ascending, divided by n), then float64 mean squared
//          deviation (each square rounded, then added), each rounded once to float32; the 64-byte
//          blocks of the mean row and of the variance row alternate ([d / 16][2][16]).
// First logical page a build (tail == 0) or an append of `tail` tokens covers.
__device__ __forceinline__ int first_page(const CacheView &c, int L, int tail) {
  return tail > 0 ? max(0, L - tail) / c.S : 0;
}

template <typename T>
struct Slice;
template <>
struct Slice<uint16_t> {
  static constexpr int V = 8;
  static __device__ __forceinline__ void unpack(const uint4 &w, float (&x)[8]) {
    x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
    x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
  }
  // element bits of two values (exact: a bf16 widened to float keeps its bits in the top half)
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xffff0000u);
  }
  static __device__ __forceinline__ uint4 pack(const float (&x)[8]) {
    return make_uint4(pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]), pack2(x[6], x[7]));
  }
};
template <>
struct Slice<float> {
  static constexpr int V = 4;
  static __device__ __forceinline__ void unpack(const uint4 &w, float (&x)[4]) {
    x[0] = __uint_as_float(w.x); x[1] = __uint_as_float(w.y); x[2] = __uint_as_float(w.z); x[3] = __uint_as_float(w.w);
  }
  static __device__ __forceinline__ uint4 pack(const float (&x)[4]) {
    return make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3]));
  }
};

// ss + dv * dv with the square rounded before the addition (no fused multiply-add)
__device__ __forceinline__ double add_square(double ss, double dv) {
#pragma clang fp contract(off)
  return ss + dv * dv;
}

// Item `it` of a workgroup that covers pages [p0, p0 + ppw): page p, KV head g, slice o; returns
// false past the sequence's last page. Rows of the item start at `row` (in rows of the cache).
struct MetaItem {
  int p, g, o, n;
  size_t row;
};
__device__ __forceinline__ bool meta_item(const CacheView &c, int b, int L, int p0, int it, int spr, MetaItem &m) {
  const int per_page = c.Hkv * spr;
  const int pp = it / per_page, rem = it - pp * per_page;
  m.p = p0 + pp;
  if (m.p >= num_pages(c, L)) return false;
  m.g = rem / spr;
  m.o = rem - m.g * spr;
  m.n = min(c.S, L - m.p * c.S);
  m.row = ((size_t)c.bt[(size_t)b * c.maxP + m.p] * c.Hkv + m.g) * c.S;
  return true;
}

constexpr int kMetaRows = 8;  // rows in flight per item

template <typename T, bool BOX, bool GAUSS>
__global__ __launch_bounds__(256) void meta_box_gauss_kernel(CacheView c, int tail, int ppw, T *__restrict__ box,
                                                             float *__restrict__ gauss) {
  constexpr int V = Slice<T>::V;
  const int b = blockIdx.y;
  const int L = seq_len(c, b);
  const int p0 = first_page(c, L, tail) + blockIdx.x * ppw;
  const int spr = c.D / V;  // slices per row
  const T *K = static_cast<const T *>(c.k);
  for (int it = threadIdx.x; it < ppw * c.Hkv * spr; it += blockDim.x) {
    MetaItem m;
    if (!meta_item(c, b, L, p0, it, spr, m)) break;  // items are page-major: the rest are past too
    const uint4 *src = reinterpret_cast<const uint4 *>(K + m.row * c.D) + m.o;
    const int rs = c.D / V;  // row stride in slices
    float lo[V], hi[V];
    double sum[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      lo[v] = __builtin_inff();
      hi[v] = -__builtin_inff();
      sum[v] = 0.0;
    }
    for (int t0 = 0; t0 < m.n; t0 += kMetaRows) {
      uint4 w[kMetaRows];
#pragma unroll
      for (int r = 0; r < kMetaRows; ++r)
        if (t0 + r < m.n) w[r] = GAUSS ? src[(size_t)(t0 + r) * rs] : ld_once(src + (size_t)(t0 + r) * rs);
#pragma unroll
      for (int r = 0; r < kMetaRows; ++r) {
        if (t0 + r >= m.n) break;
        float x[V];
        Slice<T>::unpack(w[r], x);
#pragma unroll
        for (int v = 0; v < V; ++v) {
          if (BOX) {
            if (x[v] < lo[v]) lo[v] = x[v];
            if (x[v] > hi[v]) hi[v] = x[v];
          }
          if (GAUSS) sum[v] += (double)x[v];
        }
      }
    }
    const int j0 = m.o * V;
    const size_t ob = (m.row / c.S) * 2 * c.D;  // (phys * Hkv + g) * 2d
    if (BOX) {
      constexpr int C = 64 / (int)sizeof(T);
      uint4 *dst = reinterpret_cast<uint4 *>(box + ob + (size_t)(j0 / C) * 2 * C + (j0 % C));
      dst[0] = Slice<T>::pack(lo);
      dst[C / V] = Slice<T>::pack(hi);
    }
    if (GAUSS) {
      double mu[V], ss[V];
#pragma unroll
      for (int v = 0; v < V; ++v) {
        mu[v] = sum[v] / m.n;
        ss[v] = 0.0;
      }
      for (int t0 = 0; t0 < m.n; t0 += kMetaRows) {
        uint4 w[kMetaRows];
#pragma unroll
        for (int r = 0; r < kMetaRows; ++r)
          if (t0 + r < m.n) w[r] = src[(size_t)(t0 + r) * rs];
#pragma unroll
        for (int r = 0; r < kMetaRows; ++r) {
          if (t0 + r >= m.n) break;
          float x[V];
          Slice<T>::unpack(w[r], x);
#pragma unroll
          for (int v = 0; v < V; ++v) ss[v] = add_square(ss[v], (double)x[v] - mu[v]);
        }
      }
      float mf[V], vf[V];
#pragma unroll
      for (int v = 0; v < V; ++v) {
        mf[v] = (float)mu[v];
        vf[v] = (float)(ss[v] / m.n);
      }
      float *gm = gauss + ob + (size_t)(j0 / 16) * 32 + (j0 % 16);
#pragma unroll
      for (int v = 0; v < V; v += 4) {
        *reinterpret_cast<float4 *>(gm + v) = make_float4(mf[v], mf[v + 1], mf[v + 2], mf[v + 3]);
        *reinterpret_cast<float4 *>(gm + 16 + v) = make_float4(vf[v], vf[v + 1], vf[v + 2], vf[v + 3]);
      }
    }
  }
}

// Pooled keys: per sub-block of pb token slots of the page, RN_f32 of the float64 mean of its
// valid keys (t ascending). Items as for the box / moment builder.
template <typename T>
__global__ __launch_bounds__(256) void meta_pool_kernel(CacheView c, int tail, int ppw, int pb, float *__restrict__ pool) {
  constexpr int V = Slice<T>::V;
  const int b = blockIdx.y;
  const int L = seq_len(c, b);
  const int p0 = first_page(c, L, tail) + blockIdx.x * ppw;
  const int spr = c.D / V, nsb = c.S / pb;
  const T *K = static_cast<const T *>(c.k);
  for (int it = threadIdx.x; it < ppw * c.Hkv * spr; it += blockDim.x) {
    MetaItem m;
    if (!meta_item(c, b, L, p0, it, spr, m)) break;
    const uint4 *src = reinterpret_cast<const uint4 *>(K + m.row * c.D) + m.o;
    const int j0 = m.o * V;
    for (int sb = 0; sb < nsb && sb * pb < m.n; ++sb) {
      const int t1 = min(m.n, sb * pb + pb);
      double sum[V];
#pragma unroll
      for (int v = 0; v < V; ++v) sum[v] = 0.0;
      for (int t0 = sb * pb; t0 < t1; t0 += kMetaRows) {
        uint4 w[kMetaRows];
#pragma unroll
        for (int r = 0; r < kMetaRows; ++r)
          if (t0 + r < t1) w[r] = ld_once(src + (size_t)(t0 + r) * spr);
#pragma unroll
        for (int r = 0; r < kMetaRows; ++r) {
          if (t0 + r >= t1) break;
          float x[V];
          Slice<T>::unpack(w[r], x);
#pragma unroll
          for (int v = 0; v < V; ++v) sum[v] += (double)x[v];
        }
      }
      float *dst = pool + ((m.row / c.S) * nsb + sb) * c.D + j0;
      const double cnt = t1 - sb * pb;
#pragma unroll
      for (int v = 0; v < V; v += 4)
        *reinterpret_cast<float4 *>(dst + v) = make_float4((float)(sum[v] / cnt), (float)(sum[v + 1] / cnt),
                                                           (float)(sum[v + 2] / cnt), (float)(sum[v + 3] / cnt));
    }
  }
}

// Float64 row dots of the projected-key and soft-LSH builders: every valid token row k of a
// (sequence, KV head) against the rows w_i of a float matrix, dot_i = sum_j w_i[j] * k[j] taken in
// float64 over j = 0..d-1 in that order from 0 (each product of a float and a cache element is
// exact in float64).
//   projected keys ("Joint Subspace Sparse Attention": keys kept in the shared rank-r subspace):
//     the r rows of P, kproj[row][i] = RN_bf16(dot_i).
//   soft LSH ("SOCKET" Methodology, soft LSH step 1): table l takes rows 8 l .. 8 l + 7, its P
//     hyperplanes then zero rows; bucket[row][l] has bit i set iff dot_i > 0.
// Register-blocked: a wave owns an output block of 8 rows (NOUT of them computed: 8, or P rounded
// up to even) and 512 tokens, token u * 64 + lane in slot u of each lane, and keeps the float64
// accumulators in registers. Per coordinate it reads its matrix values as float64 broadcasts from
// LDS and converts each token's K value once, so every conversion feeds NOUT fma and every matrix
// read feeds 8 tokens. The workgroup's waves share one tile of tokens (SUB tiles of 512 for r =
// 16, whose 16 outputs take two waves per tile). K goes from global memory straight to LDS
// (global_load_lds, 16 bytes a lane, so that each instruction's lanes fill consecutive LDS slots)
// in chunks of 32 bytes per row, double-buffered; each lane picks the piece for its slot such that
// the two pieces of a row trade places in every other group of four rows, which lets 8
// consecutive rows read their pieces conflict-free. Tokens covered: [0, L) for a build, the last
// `tail` of them for an append. The matrix slab in LDS holds up to 32 rows (4 output blocks);
// larger matrices take several slabs per tile.
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

struct RowDotJob {
  int nrows;            // matrix rows in output blocks of 8: r, or 8 L
  const float *mat;     // P [r][d], or the hyperplanes [L][P][d]
  int lsh_L, lsh_P;     // soft LSH only
  uint16_t *kproj;      // projected keys: [rows of the cache][r]
  uint8_t *bucket;      // soft LSH: [rows of the cache][L]
};

template <typename T, int D, int SUB, int NOUT, bool LSH>
__global__ __launch_bounds__(256, 2) void meta_rowdot_kernel(CacheView c, int tail, RowDotJob job) {
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
  const int nslab = job.nrows / SLAB, obs = SLAB / kProjOut;
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
          const int i = e / D, j = e - i * D, row = s * SLAB + i;
          float w;
          if (LSH)
            w = (row & 7) < job.lsh_P ? job.mat[((size_t)(row >> 3) * job.lsh_P + (row & 7)) * D + j] : 0.0f;
          else
            w = job.mat[(size_t)row * D + j];
          pd[((i / kProjOut) * D + j) * kProjOut + i % kProjOut] = w;
        }
      }
#pragma unroll
      for (int k = 0; k < NL; ++k) skv_load_lds16(src[k], &ks[0][64 * (wave + 4 * k)]);
      double acc[kProjTok][NOUT];
#pragma unroll
      for (int u = 0; u < kProjTok; ++u)
#pragma unroll
        for (int i = 0; i < NOUT; ++i) acc[u][i] = 0.0;
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
            double pv[NOUT];
#pragma unroll
            for (int i = 0; i < NOUT / 2; ++i) {
              const double2 w = pslab[ob][j][i];
              pv[2 * i] = w.x;
              pv[2 * i + 1] = w.y;
            }
#pragma unroll
            for (int u = 0; u < kProjTok; ++u) {
              const double kv = (double)proj_elem<T>(raw[u], e);
#pragma unroll
              for (int i = 0; i < NOUT; ++i) acc[u][i] = fma(pv[i], kv, acc[u][i]);
            }
          }
        }
      }
      if (!live) continue;
#pragma unroll
      for (int u = 0; u < kProjTok; ++u) {
        const int tok = tbase + u * 64 + lane;
        if (tok >= ntok) continue;
        const size_t row = proj_row(c, b, g, lo + tok);
        if (LSH) {
          uint32_t id = 0;
#pragma unroll
          for (int i = 0; i < NOUT; ++i) id |= (i < job.lsh_P && acc[u][i] > 0.0 ? 1u : 0u) << i;
          job.bucket[row * job.lsh_L + s * obs + ob] = (uint8_t)id;
        } else {
          uint32_t w[NOUT / 2];
#pragma unroll
          for (int i = 0; i < NOUT / 2; ++i)
            w[i] = (uint32_t)f64_to_bf16(acc[u][2 * i]) | ((uint32_t)f64_to_bf16(acc[u][2 * i + 1]) << 16);
          *reinterpret_cast<uint4 *>(job.kproj + row * job.nrows + s * SLAB + ob * kProjOut) =
              make_uint4(w[0], w[1], w[2], w[3]);
        }
      }
    }
  }
}

// The same row dots for few tokens (an append of up to kPairMaxTok tokens per sequence), where a
// tile would compute 512 tokens for a handful: one thread per (token, output row) for projected
// keys, per (token, table) for soft LSH (its P chains side by side), each chain the float64 sum
// over j = 0..d-1 from 0 as above, so that the results equal the tile kernel's.
constexpr int kPairMaxTok = 128;
template <typename T, int D, int P>   // P hyperplanes per table (soft LSH), 0 for projected keys
__global__ __launch_bounds__(256) void meta_rowdot_pairs_kernel(CacheView c, int tail, RowDotJob job) {
  const int b = blockIdx.y / c.Hkv, g = blockIdx.y % c.Hkv;
  const int L = seq_len(c, b);
  const int lo = tail > 0 ? max(0, L - tail) : 0, ntok = L - lo;
  const int outs = P ? job.lsh_L : job.nrows;  // outputs per token: tables, or rows of P
  const int pair = blockIdx.x * blockDim.x + threadIdx.x;
  if (pair >= ntok * outs) return;
  const int tok = pair / outs, o = pair - tok * outs;
  const size_t row = proj_row(c, b, g, lo + tok);
  const T *k = static_cast<const T *>(c.k) + row * D;
  constexpr int NA = P ? P : 1;
  const float *w = job.mat + (size_t)o * NA * D;
  double acc[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) acc[i] = 0.0;
#pragma unroll 8
  for (int j = 0; j < D; ++j) {
    const double kv = (double)Elem<T>::get(k, j);
#pragma unroll
    for (int i = 0; i < NA; ++i) acc[i] = fma((double)w[(size_t)i * D + j], kv, acc[i]);
  }
  if (P) {
    uint32_t id = 0;
#pragma unroll
    for (int i = 0; i < NA; ++i) id |= (acc[i] > 0.0 ? 1u : 0u) << i;
    job.bucket[row * job.lsh_L + o] = (uint8_t)id;
  } else {
    job.kproj[row * job.nrows + o] = f64_to_bf16(acc[0]);
  }
}

// Value norms for soft LSH: vnorm[row] = RN_f32(sqrt(sum_j v_j^2)), the float64 sum over j
// ascending (the square of a cache element is exact in float64, so the fma rounds once as the
// addition alone would). One thread per token row of a (sequence, KV head), 16-byte loads.
template <typename T, int D>
__global__ __launch_bounds__(256) void meta_vnorm_kernel(CacheView c, int tail, float *__restrict__ vnorm) {
  constexpr int V = Slice<T>::V;
  const int b = blockIdx.y / c.Hkv, g = blockIdx.y % c.Hkv;
  const int L = seq_len(c, b);
  const int lo = tail > 0 ? max(0, L - tail) : 0, ntok = L - lo;
  const int tok = blockIdx.x * blockDim.x + threadIdx.x;
  if (tok >= ntok) return;
  const size_t row = proj_row(c, b, g, lo + tok);
  const uint4 *src = reinterpret_cast<const uint4 *>(static_cast<const T *>(c.v) + row * D);
  uint4 w[D / V];
#pragma unroll
  for (int q = 0; q < D / V; ++q) w[q] = src[q];
  double ss = 0.0;
#pragma unroll
  for (int q = 0; q < D / V; ++q) {
    float x[V];
    Slice<T>::unpack(w[q], x);
#pragma unroll
    for (int v = 0; v < V; ++v) ss = fma((double)x[v], (double)x[v], ss);
  }
  vnorm[row] = (float)sqrt(ss);
}

// tokens per sequence a call covers at most
static long rowdot_tokens(const CacheView &c, int tail) {
  return tail > 0 ? min((long)tail, (long)c.maxP * c.S) : (long)c.maxP * c.S;
}

// Launch geometry of the row-dot kernel: 512-token tiles (two per workgroup tile for a 16-row
// matrix), kProjTilesPerWg tiles per workgroup, one grid row per (sequence, KV head).
static dim3 rowdot_grid(const CacheView &c, int tail, int sub) {
  const int tile_tok = sub * 64 * kProjTok;
  const long maxtok = rowdot_tokens(c, tail);
  const long tiles = (maxtok + tile_tok - 1) / tile_tok;
  return dim3((unsigned)((tiles + kProjTilesPerWg - 1) / kProjTilesPerWg), c.B * c.Hkv);
}

template <typename T, int D, int P>
static void rowdot_pairs(const CacheView &c, int tail, const RowDotJob &job, hipStream_t st) {
  const long pairs = rowdot_tokens(c, tail) * (P ? job.lsh_L : job.nrows);
  meta_rowdot_pairs_kernel<T, D, P><<<dim3((unsigned)((pairs + 255) / 256), c.B * c.Hkv), 256, 0, st>>>(c, tail, job);
}

template <typename T, int D>
static void lsh_pairs(const CacheView &c, int tail, const RowDotJob &job, hipStream_t st) {
  switch (job.lsh_P) {
    case 1: rowdot_pairs<T, D, 1>(c, tail, job, st); break;
    case 2: rowdot_pairs<T, D, 2>(c, tail, job, st); break;
    case 3: rowdot_pairs<T, D, 3>(c, tail, job, st); break;
    case 4: rowdot_pairs<T, D, 4>(c, tail, job, st); break;
    case 5: rowdot_pairs<T, D, 5>(c, tail, job, st); break;
    case 6: rowdot_pairs<T, D, 6>(c, tail, job, st); break;
    case 7: rowdot_pairs<T, D, 7>(c, tail, job, st); break;
    default: rowdot_pairs<T, D, 8>(c, tail, job, st); break;
  }
}

template <typename T, int D>
static void lsh_meta_d(const CacheView &c, int tail, const RowDotJob &job, float *vnorm, hipStream_t st) {
  const dim3 g2 = rowdot_grid(c, tail, 1);
  const int P = job.lsh_P;
  if (rowdot_tokens(c, tail) <= kPairMaxTok)
    lsh_pairs<T, D>(c, tail, job, st);
  else if (P <= 2) meta_rowdot_kernel<T, D, 1, 2, true><<<g2, 256, 0, st>>>(c, tail, job);
  else if (P <= 4) meta_rowdot_kernel<T, D, 1, 4, true><<<g2, 256, 0, st>>>(c, tail, job);
  else if (P <= 6) meta_rowdot_kernel<T, D, 1, 6, true><<<g2, 256, 0, st>>>(c, tail, job);
  else meta_rowdot_kernel<T, D, 1, 8, true><<<g2, 256, 0, st>>>(c, tail, job);
  const long maxtok = rowdot_tokens(c, tail);
  meta_vnorm_kernel<T, D><<<dim3((unsigned)((maxtok + 255) / 256), c.B * c.Hkv), 256, 0, st>>>(c, tail, vnorm);
}

hipError_t launch_build_lsh(const CacheView &c, int dtype, int tail, int L, int P, const float *planes,
                            uint8_t *bucket, float *vnorm, hipStream_t st) {
  const RowDotJob job{8 * L, planes, L, P, nullptr, bucket};
  if (c.D == 64) {
    if (dtype == 0) lsh_meta_d<float, 64>(c, tail, job, vnorm, st); else lsh_meta_d<uint16_t, 64>(c, tail, job, vnorm, st);
  } else {
    if (dtype == 0) lsh_meta_d<float, 128>(c, tail, job, vnorm, st); else lsh_meta_d<uint16_t, 128>(c, tail, job, vnorm, st);
  }
  return hipGetLastError();
}

hipError_t launch_build_meta(const CacheView &c, int dtype, int tail, void *box, float *gauss, int r,
                             const float *proj, uint16_t *kproj, int pb, float *pool, hipStream_t st) {
  // pages per sequence: all of them, or those the last `tail` tokens can touch
  const int np = tail > 0 ? min(c.maxP, (tail + c.S - 1) / c.S + 1) : c.maxP;
  // box / moments / pooled keys: pages per workgroup so that its 256 threads have an item each
  const int items = c.Hkv * c.D / (dtype == 0 ? Slice<float>::V : Slice<uint16_t>::V);
  const int ppw = max(1, 256 / items);
  const dim3 gridw((np + ppw - 1) / ppw, c.B);
#define SKV_BG(TT, BX, GS) \
  meta_box_gauss_kernel<TT, BX, GS><<<gridw, 256, 0, st>>>(c, tail, ppw, static_cast<TT *>(box), gauss)
  if (box || gauss) {
    if (dtype == 0) {
      if (box && gauss) SKV_BG(float, true, true); else if (box) SKV_BG(float, true, false); else SKV_BG(float, false, true);
    } else {
      if (box && gauss) SKV_BG(uint16_t, true, true);
      else if (box) SKV_BG(uint16_t, true, false);
      else SKV_BG(uint16_t, false, true);
    }
  }
#undef SKV_BG
  if (pool) {
    if (dtype == 0)
      meta_pool_kernel<float><<<gridw, 256, 0, st>>>(c, tail, ppw, pb, pool);
    else
      meta_pool_kernel<uint16_t><<<gridw, 256, 0, st>>>(c, tail, ppw, pb, pool);
  }
  if (kproj) {
    const int sub = r == 16 ? 2 : 1;  // 512-token tiles per workgroup tile
    const dim3 g2 = rowdot_grid(c, tail, sub);
    const RowDotJob job{r, proj, 0, 0, kproj, nullptr};
#define SKV_PROJ(TT, DD, SS) meta_rowdot_kernel<TT, DD, SS, 8, false><<<g2, 256, 0, st>>>(c, tail, job)
#define SKV_PROJ_D(TT, SS) \
  if (c.D == 64) SKV_PROJ(TT, 64, SS); else SKV_PROJ(TT, 128, SS);
    const bool pairs = rowdot_tokens(c, tail) <= kPairMaxTok;
    if (dtype == 0) {
      if (pairs) { if (c.D == 64) rowdot_pairs<float, 64, 0>(c, tail, job, st); else rowdot_pairs<float, 128, 0>(c, tail, job, st); }
      else if (sub == 2) { SKV_PROJ_D(float, 2) } else { SKV_PROJ_D(float, 1) }
    } else {
      if (pairs) { if (c.D == 64) rowdot_pairs<uint16_t, 64, 0>(c, tail, job, st); else rowdot_pairs<uint16_t, 128, 0>(c, tail, job, st); }
      else if (sub == 2) { SKV_PROJ_D(uint16_t, 2) } else { SKV_PROJ_D(uint16_t, 1) }
    }
#undef SKV_PROJ_D
#undef SKV_PROJ
  }
  return hipGetLastError();
}

}  // namespace skv
