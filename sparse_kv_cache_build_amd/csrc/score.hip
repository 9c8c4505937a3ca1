// Query-aware page / token scores ("EntmaxKV" summary s2.A; "Joint Subspace Sparse Attention"
// abstract for token scores in the shared subspace).
//
// Exactness: every score sum runs in float64 over the coordinate index in ascending order, one
// lane per page (or token), so that the float32 key is the rounding of the same float64 value
// a plain sequential loop produces; all products involved are exact in float64. The projected-key
// query terms, and the box terms at G = 8, are staged once per step in a float64 workspace, read by
// uniform (scalar) loads; the other scorers stage theirs in LDS from q.
#include "common.hpp"
#include "launch.hpp"

namespace skv {

// BOX: per query head and coordinate, the two float64 terms (max(q_j, 0), min(q_j, 0)), so that
// max(q kmin, q kmax) = q+ kmax + q- kmin term by term. Layout [B, Hq, D, 2].
template <typename T>
__global__ void qprep_pair_kernel(const T *__restrict__ q, int n, double *__restrict__ out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const double x = (double)Elem<T>::get(q, i);
  out[2 * i] = fmax(x, 0.0);
  out[2 * i + 1] = fmin(x, 0.0);
}

// PROJ: q~_h[i] = RN_f32(sum_j P[i][j] q_hj) (float64 sum, j ascending), stored as float64 values.
// One block per query head, thread i owns row i of P: its row is read with independent 16-byte
// loads while q_h is read with uniform (scalar) loads. Layout [B, Hq, r].
template <typename T, int D>
__global__ __launch_bounds__(64) void qprep_proj_kernel(const T *__restrict__ q, int r,
                                                        const float *__restrict__ proj, double *__restrict__ out) {
  const int bh = blockIdx.x, i = threadIdx.x;
  if (i >= r) return;
  const T *qh = q + (size_t)bh * D;
  const float4 *pr = reinterpret_cast<const float4 *>(proj + (size_t)i * D);
  double acc = 0.0;
#pragma unroll
  for (int j0 = 0; j0 < D; j0 += 4) {
    const float4 pv = pr[j0 / 4];
    acc = fma((double)pv.x, (double)Elem<T>::get(qh, j0), acc);
    acc = fma((double)pv.y, (double)Elem<T>::get(qh, j0 + 1), acc);
    acc = fma((double)pv.z, (double)Elem<T>::get(qh, j0 + 2), acc);
    acc = fma((double)pv.w, (double)Elem<T>::get(qh, j0 + 3), acc);
  }
  out[(size_t)bh * r + i] = (double)(float)acc;
}

// element jj of a row slice held as 16-byte words (jj a compile-time constant after unrolling)
template <typename T, int N>
__device__ __forceinline__ float box_elem(const uint4 (&r)[N], int jj) {
  const int w = sizeof(T) == 4 ? jj : jj >> 1;
  const uint4 v = r[w >> 2];
  const uint32_t x = (w & 3) == 0 ? v.x : (w & 3) == 1 ? v.y : (w & 3) == 2 ? v.z : v.w;
  if constexpr (sizeof(T) == 4) return __uint_as_float(x);
  else return (jj & 1) ? bf16_hi(x) : bf16_lo(x);
}

// BOX key: one lane per page. key[b][g][p] = RN_f32(max_h sum_j (q+_hj kmax_j + q-_hj kmin_j)).
// The query terms q+, q- are read as block-uniform values: at G <= 4 from LDS, where the block
// stages them from q itself (no preparation launch); at G = 8, where their LDS broadcasts would
// saturate LDS, by scalar loads from the workspace that qprep_pair_kernel fills.
// For each coordinate exactly one of the two products is nonzero (or both are zero), so the
// float64 running sum equals sum_j max(q_hj kmin_j, q_hj kmax_j) accumulated in order.
template <typename T, int D, int G>
__global__ __launch_bounds__(256) void score_box_kernel(CacheView c, const T *__restrict__ box,
                                                        const double *__restrict__ qpm, const T *__restrict__ qraw,
                                                        float *__restrict__ key) {
  const int g = blockIdx.x % c.Hkv, b = blockIdx.y, unit = b * c.Hkv + g;
  constexpr bool LQ = G <= 4;   // query terms staged in LDS from q
  __shared__ double qsl[LQ ? G * D * 2 : 2];
  if constexpr (LQ) {
    const T *qg = qraw + (size_t)(b * c.Hq + g * G) * D;
    for (int i = threadIdx.x; i < G * D; i += blockDim.x) {
      const double x = (double)Elem<T>::get(qg, i);
      qsl[2 * i] = fmax(x, 0.0);
      qsl[2 * i + 1] = fmin(x, 0.0);
    }
    __syncthreads();
  }
  const int p = (blockIdx.x / c.Hkv) * blockDim.x + threadIdx.x;
  if (p >= c.maxP) return;
  float *out = key + (size_t)unit * c.maxP + p;
  const int P = num_pages(c, seq_len(c, b));
  if (p >= P) {
    *out = -INFINITY;
    return;
  }
  const int phys = c.bt[(size_t)b * c.maxP + p];
  // the page's box: 128-byte lines, each the min row's and the max row's values of the same C
  // coordinates (64 bytes each)
  const uint4 *row = reinterpret_cast<const uint4 *>(box + ((size_t)phys * c.Hkv + g) * 2 * D);
  const double *qq = LQ ? qsl : qpm + (size_t)(b * c.Hq + g * G) * D * 2;
  // The lines are read in groups of NL whole lines, their 16-byte loads issued together, so that
  // each line is fetched once. Left to the scheduler, the loads of a line were spread over the
  // arithmetic, and the line was often evicted in between. One line per group at G = 8, where the
  // registers of two would cost more occupancy than they save.
  constexpr int NL = G >= 8 ? 1 : 2, NV = 4 * NL, EPV = 16 / (int)sizeof(T), GC = NV * EPV;
  static_assert(D % GC == 0, "a group of coordinates must divide the row");
  double acc[G];
#pragma unroll
  for (int h = 0; h < G; ++h) acc[h] = 0.0;
#pragma unroll
  for (int j0 = 0; j0 < D; j0 += GC) {
    uint4 rl[NV], rh[NV];   // the group's min values, then its max values, coordinates in order
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      const uint4 *ln = row + (size_t)(j0 / GC * NL + l) * 8;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        rl[4 * l + i] = ln[i];
        rh[4 * l + i] = ln[4 + i];
      }
    }
    __builtin_amdgcn_sched_barrier(0);   // keep the group's loads together (no wait is implied)
#pragma unroll
    for (int jj = 0; jj < GC; ++jj) {
      const double dl = box_elem<T>(rl, jj), dh = box_elem<T>(rh, jj);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        acc[h] = fma(qq[((size_t)h * D + j0 + jj) * 2], dh, acc[h]);
        acc[h] = fma(qq[((size_t)h * D + j0 + jj) * 2 + 1], dl, acc[h]);
      }
    }
  }
  double best = acc[0];
#pragma unroll
  for (int h = 1; h < G; ++h) best = fmax(best, acc[h]);
  *out = (float)best;
}

// POOL key. A row is one (page, sub-block) pair; a wave takes tiles of 64 rows: 64 >> lw pages with
// 2^lw rows each (a power of two covering the page's S/pb sub-blocks, at most 64; more sub-blocks
// than that take several tiles). Each tile is read in chunks of 32 coordinates: every lane loads
// 16 bytes of eight rows, so one load instruction covers eight whole 128-byte lines, and the chunk
// goes through LDS to the lane that owns the row. That lane sums q_hi pool_j[i] in float64 with i
// ascending (the query terms are staged in LDS from q itself), takes the largest over the heads and
// its valid sub-blocks (those holding a token), the page's lanes combine, and key[b][g][p] is the
// float32 rounding of the result; -inf past the sequence. The next chunk is loaded while the current
// one is summed. Every line is read once and whole by one instruction, so the loads are marked
// non-temporal.
template <typename QT, int D, int G>
__global__ __launch_bounds__(256) void score_pool_kernel(CacheView c, int pb, int lw, const float *__restrict__ pool,
                                                         const QT *__restrict__ q, float *__restrict__ key) {
  constexpr int CW = 32, NC = D / CW, LDR = CW + 4;   // chunk width, chunks per row, padded LDS row
  __shared__ double qs[G * D];
  __shared__ float xs[4][64 * LDR];
  const int unit = blockIdx.y, b = unit / c.Hkv, g = unit - b * c.Hkv;
  const int bx = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int W = 1 << lw, PT = 64 >> lw;
  const int p0 = (bx * 4 + wave) * PT;
  const int L = seq_len(c, b), np = num_pages(c, L), nsb = c.S / pb;
  if (bx * 4 * PT >= np) {   // every page of the block lies past the sequence
    for (int i = threadIdx.x; i < 4 * PT; i += blockDim.x)
      if (bx * 4 * PT + i < c.maxP) key[(size_t)unit * c.maxP + bx * 4 * PT + i] = -INFINITY;
    return;
  }
  const int T = (nsb + W - 1) >> lw;
  const QT *qg = q + (size_t)(b * c.Hq + g * G) * D;   // the G heads of the group are adjacent
  for (int i = threadIdx.x; i < G * D; i += blockDim.x) qs[i] = (double)Elem<QT>::get(qg, i);
  const int *bt = c.bt + (size_t)b * c.maxP;
  // element offset of a tile row in the pool array, -1 for rows without a valid token
  auto row_off = [&](int row, int t) -> long long {
    const int p = p0 + (row >> lw), sb = t * W + (row & (W - 1));
    if (p >= np || sb >= nsb || sb * pb >= min(c.S, L - p * c.S)) return -1;
    return (((long long)bt[p] * c.Hkv + g) * nsb + sb) * D;
  };
  const int lrow = lane >> 3, lcol = (lane & 7) * 4;   // load side: rows lrow + 8k, 4 columns
  const int my_p = p0 + (lane >> lw), my_j = lane & (W - 1);
  const int my_n = my_p < np ? min(c.S, L - my_p * c.S) : 0;
  float *xw = xs[wave];
  long long off[8];
  float4 r[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    off[k] = row_off(lrow + 8 * k, 0);
    r[k] = off[k] >= 0 ? ld_once(reinterpret_cast<const float4 *>(pool + off[k] + lcol)) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  double best = -INFINITY, acc[G];
  const int total = T * NC;
  __syncthreads();   // qs is staged; from here on each wave uses only its own rows in LDS
  for (int s = 0; s < total; ++s) {
    const int t = s / NC, ch = s - t * NC;
    __builtin_amdgcn_wave_barrier();   // the wave has read the previous chunk
#pragma unroll
    for (int k = 0; k < 8; ++k) *reinterpret_cast<float4 *>(xw + (lrow + 8 * k) * LDR + lcol) = r[k];
    if (s + 1 < total) {
      const int t1 = (s + 1) / NC, c1 = s + 1 - t1 * NC;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (c1 == 0) off[k] = row_off(lrow + 8 * k, t1);
        r[k] = off[k] >= 0 ? ld_once(reinterpret_cast<const float4 *>(pool + off[k] + c1 * CW + lcol))
                           : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    __builtin_amdgcn_wave_barrier();   // the chunk is in LDS for every lane of the wave
    if (ch == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) acc[h] = 0.0;
    }
    const float *xr = xw + lane * LDR;
    const double *qc = qs + ch * CW;
#pragma unroll 1   // not unrolled: the query terms of 4 coordinates live at a time (4 waves per SIMD)
    for (int i = 0; i < CW; i += 4) {
      const float4 x = *reinterpret_cast<const float4 *>(xr + i);
      const float xv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int h = 0; h < G; ++h) acc[h] = fma(qc[h * D + i + e], (double)xv[e], acc[h]);
    }
    if (ch == NC - 1) {
      const int sb = t * W + my_j;
      if (my_p < np && sb < nsb && sb * pb < my_n) {
#pragma unroll
        for (int h = 0; h < G; ++h) best = fmax(best, acc[h]);
      }
    }
  }
  for (int o = W >> 1; o > 0; o >>= 1) best = fmax(best, __shfl_xor(best, o));
  if (my_j == 0 && my_p < c.maxP) key[(size_t)unit * c.maxP + my_p] = my_p < np ? (float)best : -INFINITY;
}

constexpr int kLshPrepThreads = kLshMaxProj;   // one thread per hyperplane of the largest table set
// Soft-LSH bucket masses of one query head, one workgroup per (b, h): z_i = w_{l,i} . q / ||q||
// (float64 sums in coordinate order; 0 for q = 0), the two sigmoids sigma(+-2 z_i / tau) of every
// hyperplane, then for each table l and bucket beta the product over the bits (ascending) of the
// sigmoid the bit's sign picks, stored as the integer p * 2^24 rounded to nearest even. Layout
// [B, Hkv, L, 2^P, G]: the G heads of one bucket are adjacent for the scorer.
template <typename T, int D>
__global__ __launch_bounds__(kLshPrepThreads) void lsh_prep_kernel(CacheView c, const T *__restrict__ q, int L, int P,
                                                       const float *__restrict__ planes, double tau,
                                                       uint32_t *__restrict__ tab) {
  __shared__ double qs[D];
  __shared__ double sg[2 * kLshMaxProj];   // [l * P + i][+, -]
  __shared__ double nq;
  const int bh = blockIdx.x, b = bh / c.Hq, h = bh - b * c.Hq, g = h / c.G, hh = h - g * c.G;
  // the hyperplane rows do not depend on q: each thread's first chunk is requested before q is
  // staged, and ||q|| (thread 0, a sequential float64 sum) is taken while the others sum their dots
  constexpr int CH = 8, NCH = D / 4 / CH;
  const int m0 = threadIdx.x;   // L P <= kLshMaxProj = blockDim.x: at most one hyperplane per thread
  const float4 *w4 = reinterpret_cast<const float4 *>(planes + (size_t)min(m0, L * P - 1) * D);
  float4 wa[CH], wb[CH];
  if (m0 < L * P)
#pragma unroll
    for (int j = 0; j < CH; ++j) wa[j] = w4[j];
  for (int j = threadIdx.x; j < D; j += blockDim.x) qs[j] = (double)Elem<T>::get(q, (size_t)bh * D + j);
  __syncthreads();
  if (threadIdx.x == 0) {
    double ss = 0.0;
    for (int j = 0; j < D; ++j) ss = fma(qs[j], qs[j], ss);
    nq = sqrt(ss);
  }
  double dot = 0.0;
  if (m0 < L * P) {
    // the hyperplane streams in chunks of 32 coordinates, the next chunk loading while one is
    // summed; each chunk's query terms are read from LDS into registers before its sum, so the
    // sequential FMA chain never waits on LDS
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      if (k + 1 < NCH)
#pragma unroll
        for (int j = 0; j < CH; ++j) wb[j] = w4[(k + 1) * CH + j];
      double qc[4 * CH];
#pragma unroll
      for (int j = 0; j < 4 * CH; ++j) qc[j] = qs[4 * CH * k + j];
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        dot = fma((double)wa[j].x, qc[4 * j], dot);
        dot = fma((double)wa[j].y, qc[4 * j + 1], dot);
        dot = fma((double)wa[j].z, qc[4 * j + 2], dot);
        dot = fma((double)wa[j].w, qc[4 * j + 3], dot);
      }
#pragma unroll
      for (int j = 0; j < CH; ++j) wa[j] = wb[j];
    }
  }
  __syncthreads();   // nq is ready
  if (m0 < L * P) {
    const double z = nq > 0.0 ? dot / nq : 0.0;
    sg[2 * m0] = 1.0 / (1.0 + exp(-((2.0 * z) / tau)));
    sg[2 * m0 + 1] = 1.0 / (1.0 + exp(-((-2.0 * z) / tau)));
  }
  __syncthreads();
  const int nb = 1 << P;
  uint32_t *out = tab + (size_t)(b * c.Hkv + g) * L * nb * c.G;
  for (int e = threadIdx.x; e < L * nb; e += blockDim.x) {
    const int l = e >> P, beta = e & (nb - 1);
    double pr = 1.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {   // P <= 8; the reads go out together (index clamped in range)
      const int m = min(l * P + i, L * P - 1);
      const double v = sg[2 * m + (((beta >> i) & 1) ? 0 : 1)];
      pr = i < P ? pr * v : pr;
    }
    out[(size_t)e * c.G + hh] = (uint32_t)rint(ldexp(pr, 24));
  }
}

// Soft-collision token keys: one workgroup per (kLshTok tokens, unit). The unit's bucket masses
// [L, 2^P, G] and the block-table entries of the workgroup's pages are copied into LDS. A token's
// L bucket ids (L bytes, the tokens of a page adjacent rows) are read by L/16 lanes (4 when L = 48,
// the fourth idle), 16 tables each, so one load instruction reads 64/lpt consecutive tokens' ids:
// whole 128-byte lines, read once (non-temporal). Each lane adds up the G heads' masses of its
// tables' buckets (uint32, exact, so the order of the sums does not matter), the token's lanes
// combine their sums with DPP moves, and key = RN_f32(vnorm * (largest sum) * 2^-24), one float64
// product. A lane takes 4 tokens per step, and the next step's ids are loaded while the current
// ones are summed. Tokens past the sequence get -inf.
constexpr int kLshUnr = 4;   // tokens per lane and step
template <int G>
__global__ __launch_bounds__(256) void score_lsh_kernel(CacheView c, int L, int P, const uint8_t *__restrict__ bucket,
                                                        const float *__restrict__ vnorm,
                                                        const uint32_t *__restrict__ tab, float *__restrict__ key) {
  extern __shared__ uint4 ts4[];   // masses, then the block-table entries of the workgroup's pages
  const uint32_t *ts = reinterpret_cast<const uint32_t *>(ts4);
  const int unit = blockIdx.y, b = unit / c.Hkv, g = unit - b * c.Hkv;
  const int len = seq_len(c, b);
  const int ntok = c.maxP * c.S;
  const int t0 = blockIdx.x * kLshTok, t1 = min(ntok, t0 + kLshTok);
  float *out = key + (size_t)unit * ntok;
  const int tend = min(t1, len);   // tokens [t0, tend) are scored, [tend, t1) get -inf
  for (int t = max(t0, tend) + threadIdx.x; t < t1; t += blockDim.x) out[t] = -INFINITY;
  if (t0 >= tend) return;
  const int ne = (L << P) * G;   // a multiple of 16 (L is)
  const uint4 *src = reinterpret_cast<const uint4 *>(tab + (size_t)unit * ne);
  for (int i = threadIdx.x; i < ne / 4; i += blockDim.x) ts4[i] = src[i];
  int *sbt = reinterpret_cast<int *>(ts4 + ne / 4);
  const int p0 = t0 / c.S, np = (tend - 1) / c.S - p0 + 1;
  const int *bt = c.bt + (size_t)b * c.maxP + p0;
  for (int i = threadIdx.x; i < np; i += blockDim.x) sbt[i] = bt[i];
  __syncthreads();
  const int lpt = L == 16 ? 1 : (L == 32 ? 2 : 4);   // lanes per token
  const int tpw = kWave / lpt;                        // tokens per wave and load instruction
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int piece = lane & (lpt - 1);
  const bool has = piece * 16 < L;
  const uint32_t nbm = (1u << P) - 1;
  const int per_step = (256 / kWave) * kLshUnr * tpw;   // tokens of the workgroup per step
  const int nstep = (tend - t0 + per_step - 1) / per_step;
  // token u of this lane in step s
  auto tok = [&](int s, int u) { return t0 + s * per_step + (u * (256 / kWave) + wave) * tpw + lane / lpt; };
  auto load = [&](int s, uint4 (&w)[kLshUnr], float (&vn)[kLshUnr]) {
#pragma unroll
    for (int u = 0; u < kLshUnr; ++u) {
      const int t = tok(s, u);
      w[u] = make_uint4(0u, 0u, 0u, 0u);
      vn[u] = 0.0f;
      if (t < tend) {
        const int p = t / c.S;
        const size_t row = ((size_t)sbt[p - p0] * c.Hkv + g) * c.S + (t - p * c.S);
        if (has) w[u] = ld_once(reinterpret_cast<const uint4 *>(bucket + row * L) + piece);
        if (piece == 0) vn[u] = vnorm[row];
      }
    }
  };
  uint4 wc[kLshUnr], wn[kLshUnr];
  float vc[kLshUnr], vnx[kLshUnr];
  load(0, wc, vc);
  for (int s = 0; s < nstep; ++s) {   // uniform over the workgroup: every lane takes part in the DPP sums
    if (s + 1 < nstep) load(s + 1, wn, vnx);
#pragma unroll
    for (int u = 0; u < kLshUnr; ++u) {
      uint32_t sum[G];
#pragma unroll
      for (int hh = 0; hh < G; ++hh) sum[hh] = 0;
      if (has) {
        const uint32_t w4[4] = {wc[u].x, wc[u].y, wc[u].z, wc[u].w};
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const uint32_t bb = (w4[k >> 2] >> (8 * (k & 3))) & nbm;   // ids are < 2^P; the mask keeps LDS in range
          const uint32_t *e = ts + (((size_t)(piece * 16 + k) << P) + bb) * G;
          if constexpr (G >= 4) {
#pragma unroll
            for (int h4 = 0; h4 < G; h4 += 4) {
              const uint4 v = *reinterpret_cast<const uint4 *>(e + h4);
              sum[h4] += v.x;
              sum[h4 + 1] += v.y;
              sum[h4 + 2] += v.z;
              sum[h4 + 3] += v.w;
            }
          } else {
#pragma unroll
            for (int hh = 0; hh < G; ++hh) sum[hh] += e[hh];
          }
        }
      }
      // the token's lanes are adjacent: add their sums (quad_perm xor 1, then xor 2)
      if (lpt >= 2)
#pragma unroll
        for (int hh = 0; hh < G; ++hh) sum[hh] += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)sum[hh], 0xb1, 0xf, 0xf, false);
      if (lpt >= 4)
#pragma unroll
        for (int hh = 0; hh < G; ++hh) sum[hh] += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)sum[hh], 0x4e, 0xf, 0xf, false);
      uint32_t best = sum[0];
#pragma unroll
      for (int hh = 1; hh < G; ++hh) best = max(best, sum[hh]);
      const int t = tok(s, u);
      if (piece == 0 && t < tend) out[t] = (float)((double)vc[u] * ldexp((double)best, -24));
    }
#pragma unroll
    for (int u = 0; u < kLshUnr; ++u) {
      wc[u] = wn[u];
      vc[u] = vnx[u];
    }
  }
}

// GAUSS scores. m = scale sum_j q_j mean_j, s = scale sqrt(sum_j q_j^2 var_j), shat = m + s sqrt(2 ln
// n_p) (or the quantile maximum); outputs [B, Hq, maxP], NaN past the sequence. The sums run in
// float32, j ascending: the scores feed only the threshold estimate, whose decisions are compared
// with a tolerance (a float32 sum of d terms is within about d 2^-24 of the sum of the absolute
// terms). A block first stages the (q, q^2) pairs of its G query heads in LDS from q itself. A wave
// owns 64 pages (a lane each, G heads); their rows are read in chunks of 16 coordinates, one whole
// 128-byte line of the metadata (64 bytes of means, then the 64 bytes of variances of the same
// coordinates: 8 lanes per page, eight pages per load instruction) into LDS, where each lane sums
// its page with the (q, q^2) pairs read as broadcasts (8 bytes per head and coordinate). The next
// chunk is loaded while the current one is summed; the loads are non-temporal, each line being read
// once and whole by one instruction.
template <typename T, int D, int G>
__global__ __launch_bounds__(256) void score_gauss_kernel(CacheView c, const T *__restrict__ q,
                                                          const float *__restrict__ gauss, float scale, int quantile,
                                                          float *__restrict__ m_out, float *__restrict__ s_out,
                                                          float *__restrict__ shat_out) {
  constexpr int CW = 16, NC = D / CW, LDR = 2 * CW + 4, NK = 8;   // 64 rows, 8 per load instruction
  __shared__ float2 qs[G * D];
  __shared__ float xs[4][64 * LDR];
  const int unit = blockIdx.y, b = unit / c.Hkv, g = unit - b * c.Hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int pblk = blockIdx.x * 256, p0 = pblk + wave * 64;
  const int L = seq_len(c, b), np = num_pages(c, L);
  const size_t ob = (size_t)(b * c.Hq + g * G) * c.maxP;
  if (pblk >= np) {   // every page of the block lies past the sequence
    for (int i = threadIdx.x; i < 256 * G; i += blockDim.x) {
      const int p = pblk + i % 256, h = i / 256;
      if (p < c.maxP) m_out[ob + (size_t)h * c.maxP + p] = s_out[ob + (size_t)h * c.maxP + p] =
          shat_out[ob + (size_t)h * c.maxP + p] = NAN;
    }
    return;
  }
  const T *qg = q + (size_t)(b * c.Hq + g * G) * D;   // the G heads of the group are adjacent
  for (int i = threadIdx.x; i < G * D; i += blockDim.x) {
    const float x = Elem<T>::get(qg, i);
    qs[i] = make_float2(x, x * x);
  }
  const int *bt = c.bt + (size_t)b * c.maxP;
  // load side: lane -> page lrow + 8k, half (mean or variance row) and 4 of the 16 columns
  const int lrow = lane >> 3, half = (lane >> 2) & 1, lcol = (lane & 3) * 4;
  long long off[NK];
  float4 r[NK];
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    const int p = p0 + lrow + 8 * k;
    off[k] = p < np ? ((long long)bt[p] * c.Hkv + g) * 2 * D + half * CW + lcol : -1;
    r[k] = off[k] >= 0 ? ld_once(reinterpret_cast<const float4 *>(gauss + off[k])) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float *xw = xs[wave];
  float sm[G], sv[G];
#pragma unroll
  for (int h = 0; h < G; ++h) sm[h] = sv[h] = 0.0f;
  __syncthreads();   // qs is staged; from here on each wave uses only its own rows in LDS
  for (int ch = 0; ch < NC; ++ch) {
    __builtin_amdgcn_wave_barrier();   // the wave has read the previous chunk
#pragma unroll
    for (int k = 0; k < NK; ++k) *reinterpret_cast<float4 *>(xw + (lrow + 8 * k) * LDR + half * CW + lcol) = r[k];
    if (ch + 1 < NC) {
#pragma unroll
      for (int k = 0; k < NK; ++k)
        r[k] = off[k] >= 0 ? ld_once(reinterpret_cast<const float4 *>(gauss + off[k] + (ch + 1) * 2 * CW))
                           : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __builtin_amdgcn_wave_barrier();   // the chunk is in LDS for every lane of the wave
    const float *xm = xw + lane * LDR, *xv = xm + CW;
    const float2 *qc = qs + ch * CW;
#pragma unroll 4
    for (int j = 0; j < CW; ++j) {
      const float dm = xm[j], dv = xv[j];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float2 qp = qc[h * D + j];
        sm[h] = fmaf(qp.x, dm, sm[h]);
        sv[h] = fmaf(qp.y, dv, sv[h]);
      }
    }
  }
  const int p = p0 + lane;
  if (p >= c.maxP) return;
  const size_t o0 = ob + p;
  if (p >= np) {
#pragma unroll
    for (int h = 0; h < G; ++h) m_out[o0 + (size_t)h * c.maxP] = s_out[o0 + (size_t)h * c.maxP] =
        shat_out[o0 + (size_t)h * c.maxP] = NAN;
    return;
  }
  const int n = min(c.S, L - p * c.S);
  // estimated maximum of the page's n scores: m + s sqrt(2 ln n), or (quantile) m + s Phi^-1(1 - 1/n)
  // = m + s sqrt(2) erfcinv(2 / n)
  const float lg =
      n <= 1 ? 0.0f : (float)(quantile ? 1.4142135623730951 * erfcinv(2.0 / n) : sqrt(2.0 * log((double)n)));
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float m = scale * sm[h], s = scale * sqrtf(sv[h]);
    m_out[o0 + (size_t)h * c.maxP] = m;
    s_out[o0 + (size_t)h * c.maxP] = s;
    shat_out[o0 + (size_t)h * c.maxP] = fmaf(s, lg, m);
  }
}

// PROJ key: one lane per token t. u_h(t) = sum_i q~_h[i] k~_t[i] (float64, i ascending; the
// products of a float32 and a bf16 value are exact), key = RN_f32(max_h u_h(t)). Each thread
// scores TPT tokens (t, t + 256, ...) with all their row loads issued before the arithmetic.
constexpr int kProjTPT = 2;
template <int R, int G>
__global__ __launch_bounds__(256) void score_proj_kernel(CacheView c, const uint16_t *__restrict__ kproj,
                                                         const double *__restrict__ qt, float *__restrict__ key) {
  const int unit = blockIdx.y, b = unit / c.Hkv, g = unit - b * c.Hkv;
  const int Lmax = c.maxP * c.S, L = seq_len(c, b);
  const int t0 = blockIdx.x * (256 * kProjTPT) + threadIdx.x;
  const double *qq = qt + (size_t)(b * c.Hq + g * G) * R;
  uint4 w[kProjTPT][R / 8];
#pragma unroll
  for (int u = 0; u < kProjTPT; ++u)
    if (t0 + u * 256 < L) proj_row_load<R>(c, kproj, b, g, t0 + u * 256, w[u]);
#pragma unroll
  for (int u = 0; u < kProjTPT; ++u) {
    const int t = t0 + u * 256;
    if (t >= Lmax) break;
    key[(size_t)unit * Lmax + t] = t < L ? proj_row_key<R, G>(w[u], qq) : -INFINITY;
  }
}

// Fused PROJ scoring for a token top-k. Only tokens whose exact key has order key >= the unit's
// bound T_lo are written, as (key, token) pairs in token order into the candidate segment of
// their group, with the group's count. One wave per group of kCandSegTokens consecutive tokens,
// in chunks of 64 tokens; the next two chunks' rows are loaded while the current one is filtered:
//  1. load: a row of R bf16 values is R/8 lanes of 16 bytes, so one load instruction reads 512/R
//     consecutive rows, whole 128-byte lines (runs of S R 2 bytes inside a page). The loads are
//     marked non-temporal, as every row is read once. When S is a power of two and a multiple of
//     512/R, the rows of one load lie in one page, whose block-table entry is wave-uniform;
//  2. the chunk goes through the wave's LDS staging area, from which every lane reads one row;
//  3. filter: the row's upper estimate of its key (proj_row_upper, q~ as scalar operands)
//     against T_lo; rows that pass join the wave's LDS list of pending candidates, with their rows;
//  4. exact: when a chunk would overflow the 64-entry list, and after the last chunk, the pending
//     candidates (one lane each) get the exact key, and the ones with order key >= T_lo are
//     appended to the segment with ballots.
// The estimate never falls below the exact key, so the filter loses no token of the exact set;
// it only spares the float64 arithmetic for the tokens that cannot reach T_lo.
template <int R, int G, bool UNI>
__global__ __launch_bounds__(256) void score_proj_cand_kernel(CacheView c, const uint16_t *__restrict__ kproj,
                                                              const double *__restrict__ qt,
                                                              const uint32_t *__restrict__ qb,
                                                              const float2 *__restrict__ qc,
                                                              const uint32_t *__restrict__ bound,
                                                              int32_t *__restrict__ count, float2 *__restrict__ segs,
                                                              int nb) {
  constexpr int GT = kCandSegTokens, CH = kWave;                   // tokens per group, per chunk
  constexpr int LPR = R / 8, TPI = kWave / LPR, NI = CH / TPI;     // lanes per row, rows per load, loads per chunk
  constexpr int SROW = LPR + 1;   // staged row stride in 16-byte words (the pad spreads a row read over the banks)
  __shared__ uint4 stg[256 / kWave][CH * SROW];
  __shared__ uint4 rc[256 / kWave][kWave][LPR];   // rows of the pending candidates
  __shared__ int cl[256 / kWave][kWave];          // their tokens
  const int g = blockIdx.x % c.Hkv, b = blockIdx.y, unit = b * c.Hkv + g;
  const int L = seq_len(c, b);
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  const int gid = (blockIdx.x / c.Hkv) * (256 / kWave) + wv;   // group of this wave
  const int tg = gid * GT;
  if (tg >= L || gid >= nb) return;
  const uint32_t *qp = qb + (size_t)(b * c.Hq + g * G) * (R / 2);
  const uint32_t Tlo = bound[unit];
  const float2 cf = qc[unit];
  const FilterCoef fc{cf.x, cf.y};
  const int *btb = c.bt + (size_t)b * c.maxP;
  const int sh = 31 - __clz(c.S);                   // log2 S when S is a power of two
  const int part = lane % LPR, lrow = lane / LPR;   // the lane's 16 bytes of row lrow of a load
  // UNI: the block-table entries of the group's pages, one per lane (pages past the sequence: 0)
  constexpr int NV = (GT / TPI + kWave - 1) / kWave;
  int vbt[NV];
  if (UNI) {
    const int pg0 = tg >> sh, npg = num_pages(c, L);
#pragma unroll
    for (int v = 0; v < NV; ++v) vbt[v] = pg0 + v * kWave + lane < npg ? btb[pg0 + v * kWave + lane] : 0;
  }
  auto load = [&](int ch, uint4 (&x)[NI]) {
    const int ts = tg + ch * CH;
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const int t = min(ts + k * TPI + lrow, L - 1);   // rows past the sequence repeat the last one
      int pg, phys;
      if (UNI) {   // S is a power of two and a multiple of TPI: the load's rows share one page
        pg = __builtin_amdgcn_readfirstlane(min(ts + k * TPI, L - 1)) >> sh;
        const int pl = pg - (tg >> sh);   // the page's index in the group, below GT / S
        phys = NV == 1 || pl < kWave ? __builtin_amdgcn_readlane(vbt[0], pl & (kWave - 1))
                                     : __builtin_amdgcn_readlane(vbt[NV - 1], pl & (kWave - 1));
      } else {
        pg = t / c.S;
        phys = btb[pg];
      }
      const uint4 *row =
          reinterpret_cast<const uint4 *>(kproj + (((size_t)phys * c.Hkv + g) * c.S + (t - pg * c.S)) * R);
      x[k] = ld_once(row + part);
    }
  };
  const double *qq = qt + (size_t)(b * c.Hq + g * G) * R;
  float2 *seg = segs + ((size_t)unit * nb + gid) * GT;
  int pend = 0, base = 0;
  auto flush = [&]() {
    __builtin_amdgcn_wave_barrier();
    uint4 x[LPR];
#pragma unroll
    for (int j = 0; j < LPR; ++j) x[j] = rc[wv][lane][j];
    const int t = lane < pend ? cl[wv][lane] : tg;
    const float kv = proj_row_key_lean<R, G>(x, qq);
    const bool keep = lane < pend && f32_order_key(kv) >= Tlo;
    const uint64_t bal = __ballot(keep);
    if (keep)
      seg[base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u))] =
          make_float2(kv, __int_as_float(t));
    base += __popcll(bal);
    pend = 0;
    __builtin_amdgcn_wave_barrier();   // the list is read before it is refilled
  };
  auto filter = [&](int ch, const uint4 (&x)[NI]) {
    uint4 *sw = stg[wv];
    __builtin_amdgcn_wave_barrier();   // the previous chunk's rows have been read
#pragma unroll
    for (int k = 0; k < NI; ++k) sw[(k * TPI + lrow) * SROW + part] = x[k];
    __builtin_amdgcn_wave_barrier();
    uint4 row[LPR];
#pragma unroll
    for (int j = 0; j < LPR; ++j) row[j] = sw[lane * SROW + j];
    const int t = tg + ch * CH + lane;
    int zero = 0;
    asm volatile("" : "+s"(zero));   // q~ is read again per chunk (scalar loads), not held in registers
    const bool keep = t < L && f32_order_key(proj_row_upper<R, G>(row, qp + zero, fc)) >= Tlo;
    const uint64_t bal = __ballot(keep);
    const int n = __popcll(bal);
    if (pend + n > kWave) flush();
    if (keep) {
      const int slot = pend + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
      cl[wv][slot] = t;
#pragma unroll
      for (int j = 0; j < LPR; ++j) rc[wv][slot][j] = row[j];
    }
    pend += n;
  };
  const int nch = min(GT / CH, (L - tg + CH - 1) / CH);
  uint4 w0[NI], w1[NI], w2[NI];   // two chunks in flight while a third is filtered
  load(0, w0);
  if (1 < nch) load(1, w1);
  for (int ch = 0; ch < nch; ch += 3) {   // three buffers in rotation: no dynamic register indexing
    if (ch + 2 < nch) load(ch + 2, w2);
    filter(ch, w0);
    if (ch + 1 >= nch) break;
    if (ch + 3 < nch) load(ch + 3, w0);
    filter(ch + 1, w1);
    if (ch + 2 >= nch) break;
    if (ch + 4 < nch) load(ch + 4, w1);
    filter(ch + 2, w2);
  }
  if (pend > 0) flush();
  if (lane == 0) count[(size_t)unit * nb + gid] = base;
}

// ---------------------------------------------------------------- launchers

template <typename T>
static hipError_t qprep_pair(const void *q, int n, double *ws, hipStream_t st) {
  qprep_pair_kernel<T><<<(n + 255) / 256, 256, 0, st>>>(static_cast<const T *>(q), n, ws);
  return hipGetLastError();
}

#define SKV_DISPATCH_G(G, ...)                      \
  switch (G) {                                      \
    case 1: { constexpr int GG = 1; __VA_ARGS__; } break; \
    case 2: { constexpr int GG = 2; __VA_ARGS__; } break; \
    case 4: { constexpr int GG = 4; __VA_ARGS__; } break; \
    case 8: { constexpr int GG = 8; __VA_ARGS__; } break; \
    default: return hipErrorInvalidValue;           \
  }

template <typename T, int D>
static hipError_t box_d(const CacheView &c, const void *q, const void *box, const double *qpm, float *key, hipStream_t st,
                        const KernelEvents &ev) {
  // the Hkv blocks of one page range are adjacent in launch order (page block = x / Hkv), so the
  // KV heads' boxes of a physical page (adjacent in memory) are read at about the same time
  const dim3 grid(((c.maxP + 255) / 256) * c.Hkv, c.B);
  hipError_t e0 = ev.before(st);
  if (e0 != hipSuccess) return e0;
  SKV_DISPATCH_G(c.G, score_box_kernel<T, D, GG><<<grid, 256, 0, st>>>(c, static_cast<const T *>(box), qpm,
                                                                         static_cast<const T *>(q), key))
  return ev.after(st);
}

hipError_t launch_score_box(const CacheView &c, int dtype, const void *q, const void *box, float *key, double *ws,
                            hipStream_t st, const KernelEvents &ev) {
  const int n = c.B * c.Hq * c.D;
  if (c.G > 4) {   // at G = 8 the terms are read by scalar loads from the workspace
    hipError_t e = dtype == 0 ? qprep_pair<float>(q, n, ws, st) : qprep_pair<uint16_t>(q, n, ws, st);
    if (e != hipSuccess) return e;
  }
  if (c.D == 64) return dtype == 0 ? box_d<float, 64>(c, q, box, ws, key, st, ev) : box_d<uint16_t, 64>(c, q, box, ws, key, st, ev);
  return dtype == 0 ? box_d<float, 128>(c, q, box, ws, key, st, ev) : box_d<uint16_t, 128>(c, q, box, ws, key, st, ev);
}

template <typename T, int D>
static hipError_t gauss_d(const CacheView &c, const void *q, const float *gauss, float scale, int quantile, float *m,
                          float *s, float *shat, hipStream_t st, const KernelEvents &ev) {
  const dim3 grid((c.maxP + 255) / 256, c.B * c.Hkv);
  const T *qt = static_cast<const T *>(q);
  hipError_t e0 = ev.before(st);
  if (e0 != hipSuccess) return e0;
  SKV_DISPATCH_G(c.G, score_gauss_kernel<T, D, GG><<<grid, 256, 0, st>>>(c, qt, gauss, scale, quantile, m, s, shat))
  return ev.after(st);
}

hipError_t launch_score_gauss(const CacheView &c, int dtype, const void *q, const float *gauss, float scale,
                              int quantile, float *m, float *s, float *shat, hipStream_t st, const KernelEvents &ev) {
  if (dtype == 0)
    return c.D == 64 ? gauss_d<float, 64>(c, q, gauss, scale, quantile, m, s, shat, st, ev)
                     : gauss_d<float, 128>(c, q, gauss, scale, quantile, m, s, shat, st, ev);
  return c.D == 64 ? gauss_d<uint16_t, 64>(c, q, gauss, scale, quantile, m, s, shat, st, ev)
                   : gauss_d<uint16_t, 128>(c, q, gauss, scale, quantile, m, s, shat, st, ev);
}

template <typename T, int D>
static hipError_t pool_d(const CacheView &c, int pb, const T *q, const float *pool, float *key, hipStream_t st,
                         const KernelEvents &ev) {
  int lw = 0;
  while ((1 << lw) < c.S / pb && lw < 6) ++lw;
  const int pages_per_block = 4 * (64 >> lw);
  const dim3 grid((c.maxP + pages_per_block - 1) / pages_per_block, c.B * c.Hkv);
  hipError_t e0 = ev.before(st);
  if (e0 != hipSuccess) return e0;
  SKV_DISPATCH_G(c.G, score_pool_kernel<T, D, GG><<<grid, 256, 0, st>>>(c, pb, lw, pool, q, key))
  return ev.after(st);
}

hipError_t launch_score_pool(const CacheView &c, int dtype, const void *q, int pb, const float *pool, float *key,
                             hipStream_t st, const KernelEvents &ev) {
  if (dtype == 0) {
    const float *qf = static_cast<const float *>(q);
    return c.D == 64 ? pool_d<float, 64>(c, pb, qf, pool, key, st, ev) : pool_d<float, 128>(c, pb, qf, pool, key, st, ev);
  }
  const uint16_t *qb = static_cast<const uint16_t *>(q);
  return c.D == 64 ? pool_d<uint16_t, 64>(c, pb, qb, pool, key, st, ev)
                   : pool_d<uint16_t, 128>(c, pb, qb, pool, key, st, ev);
}

template <int R>
static hipError_t proj_r(const CacheView &c, const uint16_t *kproj, const double *qt, float *key, hipStream_t st,
                         const KernelEvents &ev) {
  const dim3 grid((c.maxP * c.S + 256 * kProjTPT - 1) / (256 * kProjTPT), c.B * c.Hkv);
  hipError_t e0 = ev.before(st);
  if (e0 != hipSuccess) return e0;
  SKV_DISPATCH_G(c.G, score_proj_kernel<R, GG><<<grid, 256, 0, st>>>(c, kproj, qt, key))
  return ev.after(st);
}

template <int R, bool UNI>
static hipError_t proj_cand_r(const CacheView &c, const uint16_t *kproj, char *cand, const CandLayout &lay,
                              hipStream_t st, const KernelEvents &ev) {
  // the Hkv blocks of one token range are adjacent in launch order: the KV heads' rows of a
  // physical page (adjacent in memory) are read at about the same time
  const dim3 grid(((lay.nb + 3) / 4) * c.Hkv, c.B);
  hipError_t e0 = ev.before(st);
  if (e0 != hipSuccess) return e0;
  SKV_DISPATCH_G(c.G, score_proj_cand_kernel<R, GG, UNI><<<grid, 256, 0, st>>>(
                          c, kproj, reinterpret_cast<const double *>(cand + lay.qt),
                          reinterpret_cast<const uint32_t *>(cand + lay.qb),
                          reinterpret_cast<const float2 *>(cand + lay.qc),
                          reinterpret_cast<const uint32_t *>(cand + lay.bound),
                          reinterpret_cast<int32_t *>(cand + lay.count), reinterpret_cast<float2 *>(cand + lay.seg),
                          lay.nb))
  return ev.after(st);
}

hipError_t launch_score_proj_cand(const CacheView &c, int r, const uint16_t *kproj, char *cand, hipStream_t st,
                                  const KernelEvents &ev) {
  const CandLayout lay(c.B, c.Hq, c.Hkv, c.maxP * c.S, 64);   // layout independent of the rank
  // rows of one load instruction: 512 / r; they share a page when S is a power-of-two multiple
  const bool uni = (c.S & (c.S - 1)) == 0 && c.S % (512 / r) == 0;
  switch (r) {
    case 16: return uni ? proj_cand_r<16, true>(c, kproj, cand, lay, st, ev) : proj_cand_r<16, false>(c, kproj, cand, lay, st, ev);
    case 32: return uni ? proj_cand_r<32, true>(c, kproj, cand, lay, st, ev) : proj_cand_r<32, false>(c, kproj, cand, lay, st, ev);
    case 64: return uni ? proj_cand_r<64, true>(c, kproj, cand, lay, st, ev) : proj_cand_r<64, false>(c, kproj, cand, lay, st, ev);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_score_proj(const CacheView &c, int dtype, const void *q, int r, const float *proj,
                             const uint16_t *kproj, float *key, double *ws, hipStream_t st,
                             const KernelEvents &ev) {
  const int BH = c.B * c.Hq;
  if (dtype == 0) {
    if (c.D == 64)
      qprep_proj_kernel<float, 64><<<BH, 64, 0, st>>>(static_cast<const float *>(q), r, proj, ws);
    else
      qprep_proj_kernel<float, 128><<<BH, 64, 0, st>>>(static_cast<const float *>(q), r, proj, ws);
  } else {
    if (c.D == 64)
      qprep_proj_kernel<uint16_t, 64><<<BH, 64, 0, st>>>(static_cast<const uint16_t *>(q), r, proj, ws);
    else
      qprep_proj_kernel<uint16_t, 128><<<BH, 64, 0, st>>>(static_cast<const uint16_t *>(q), r, proj, ws);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (r) {
    case 16: return proj_r<16>(c, kproj, ws, key, st, ev);
    case 32: return proj_r<32>(c, kproj, ws, key, st, ev);
    case 64: return proj_r<64>(c, kproj, ws, key, st, ev);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
static hipError_t lsh_d(const CacheView &c, int dtype, const void *q, int L, int P, const float *planes, double tau,
                        const uint8_t *bucket, const float *vnorm, float *key, uint32_t *tab, hipStream_t st,
                        const KernelEvents &ev) {
  if (dtype == 0)
    lsh_prep_kernel<float, D><<<c.B * c.Hq, kLshPrepThreads, 0, st>>>(c, static_cast<const float *>(q), L, P, planes, tau, tab);
  else
    lsh_prep_kernel<uint16_t, D><<<c.B * c.Hq, kLshPrepThreads, 0, st>>>(c, static_cast<const uint16_t *>(q), L, P, planes, tau,
                                                             tab);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((c.maxP * c.S + kLshTok - 1) / kLshTok, c.B * c.Hkv);
  // masses, then the block-table entries of the pages of kLshTok tokens (at most kLshTok / S + 2)
  const size_t lds = sizeof(uint32_t) * ((size_t)L << P) * c.G + sizeof(int) * (size_t)(kLshTok / c.S + 2);
  hipError_t e0 = ev.before(st);
  if (e0 != hipSuccess) return e0;
  SKV_DISPATCH_G(c.G, score_lsh_kernel<GG><<<grid, 256, lds, st>>>(c, L, P, bucket, vnorm, tab, key))
  return ev.after(st);
}

hipError_t launch_score_lsh(const CacheView &c, int dtype, const void *q, int L, int P, const float *planes,
                            float tau, const uint8_t *bucket, const float *vnorm, float *key, void *ws,
                            hipStream_t st, const KernelEvents &ev) {
  uint32_t *tab = static_cast<uint32_t *>(ws);
  return c.D == 64 ? lsh_d<64>(c, dtype, q, L, P, planes, (double)tau, bucket, vnorm, key, tab, st, ev)
                   : lsh_d<128>(c, dtype, q, L, P, planes, (double)tau, bucket, vnorm, key, tab, st, ev);
}

}  // namespace skv
