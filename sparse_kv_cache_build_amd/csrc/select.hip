// Candidate selection ("EntmaxKV" summary s2.B: top-k pages by bound, Gaussian-aware entmax
// threshold; "Joint Subspace Sparse Attention" abstract: top-k tokens per KV head).
// One selection per (sequence, KV head); indices are emitted in ascending order.
#include "common.hpp"
#include "launch.hpp"

namespace skv {

constexpr int kSelThreads = 512;
constexpr int kSelLds = 16384;   // page keys held in LDS when n <= kSelLds (64 KiB)
constexpr int kTokThreads = 1024;
constexpr int kTokCand = 8192;   // token candidates held in LDS (key + index: 64 KiB)
constexpr int kTokSample = 8192; // keys sampled to place the candidate threshold

// Number of candidates and how many to keep for unit (b, g).
struct SelSize {
  int n, k;
};

__device__ __forceinline__ SelSize sel_size(const CacheView &c, int b, int policy, int k, int pct) {
  const int L = seq_len(c, b);
  const int P = num_pages(c, L);
  SelSize s;
  if (policy == 3) {  // TOKEN_TOPK
    s.n = L;
    s.k = min(k, L);
  } else if (policy == 1) {  // BUDGET: ceil(pct * P / 100), at least 1
    s.n = P;
    const long long kb = ((long long)pct * P + 99) / 100;
    s.k = P == 0 ? 0 : (int)min((long long)P, max(1LL, kb));
  } else {  // TOPK
    s.n = P;
    s.k = min(k, P);
  }
  return s;
}

// radix_kth over keys a thread holds in registers: slot j of thread t is key i = t + j * NT (valid
// when i < n). The keys are read once, not per pass, and within a wave the lanes whose digit
// equals the first active lane's are counted with one atomic (the leading digits of a candidate
// set fall into few bins, where per-lane atomics on one address serialize).
template <int NT, int KPT>
__device__ void radix_kth_regs(const uint32_t (&u)[KPT], int n, uint32_t r, uint32_t *hist, uint32_t *bc,
                               uint32_t &T, uint32_t &need, int digits, uint32_t lo, uint32_t hi) {
  constexpr int NW = NT / kWave;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
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
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const bool in = tid + j * NT < n && (u[j] & mask) == prefix;
      const uint32_t d = (u[j] >> shift) & 0xffu;
      const uint64_t act = __ballot(in);
      if (act != 0) {
        const int leader = __ffsll((unsigned long long)act) - 1;
        const uint32_t ld = __builtin_amdgcn_readlane(d, leader);
        const uint64_t same = __ballot(in && d == ld);
        if (lane == leader) atomicAdd(&mine[ld], (uint32_t)__popcll(same));
        if (in && d != ld) atomicAdd(&mine[d], 1u);
      }
    }
    __syncthreads();
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

// Ordered take over i in [0, n): keeps keys > T and the first `need` keys == T (lowest i), and
// writes out[rank] = idx(i) in increasing i. Each thread walks a contiguous chunk; block scans
// give the ranks (one scan of both counts packed in a word when n < 2^15). Every thread of the
// block must call it.
template <int NT, typename Get, typename Idx>
__device__ void ordered_take(Get get, Idx idx, int n, uint32_t T, uint32_t need, int32_t *out, int *scan_scratch) {
  const int per = (n + NT - 1) / NT;
  const int i0 = min(n, (int)threadIdx.x * per), i1 = min(n, i0 + per);
  int ngt = 0, neq = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t u = get(i);
    ngt += u > T;
    neq += u == T;
  }
  int tot, gt_before, eq_before;
  if (n < 32768) {   // both counts in one word (each below 2^15): one scan gives both prefixes
    const int both = block_excl_scan<NT>((ngt << 16) | neq, scan_scratch, &tot);
    gt_before = both >> 16;
    eq_before = both & 0xffff;
  } else {
    gt_before = block_excl_scan<NT>(ngt, scan_scratch, &tot);
    eq_before = block_excl_scan<NT>(neq, scan_scratch, &tot);
  }
  for (int i = i0; i < i1; ++i) {
    const uint32_t u = get(i);
    if (u > T || (u == T && (uint32_t)eq_before < need)) out[gt_before + min((uint32_t)eq_before, need)] = idx(i);
    gt_before += u > T;
    eq_before += u == T;
  }
}

// Page top-k / budget: one block per unit; the unit's page keys sit in LDS when they fit.
__global__ __launch_bounds__(kSelThreads) void select_topk_kernel(CacheView c, const float *__restrict__ key,
                                                                  int key_stride, int policy, int k, int pct,
                                                                  int32_t *__restrict__ sel_idx,
                                                                  int32_t *__restrict__ sel_count, int cap) {
  __shared__ uint32_t skeys[kSelLds];
  __shared__ __align__(16) uint32_t hist[kSelThreads / kWave * 256];
  __shared__ uint32_t bc[2];
  __shared__ int scan_scratch[kSelThreads / kWave + 1];
  const int unit = blockIdx.x, b = unit / c.Hkv;
  const SelSize sz = sel_size(c, b, policy, k, pct);
  const float *kr = key + (size_t)unit * key_stride;
  int32_t *out = sel_idx + (size_t)unit * cap;
  const int tid = threadIdx.x;
  if (tid == 0) sel_count[unit] = sz.k;
  if (sz.k <= 0) return;
  if (sz.k >= sz.n) {  // everything is kept
    for (int i = tid; i < sz.n; i += kSelThreads) out[i] = i;
    return;
  }
  uint32_t T, need;
  auto ident = [](int i) { return i; };
  if (sz.n <= kSelLds) {
    // the keys' range comes with the load: radix passes over the leading digits that every key
    // shares are skipped (page keys of a unit share their leading byte as a rule)
    uint32_t kmin = 0xffffffffu, kmax = 0u;
    for (int i = tid; i < sz.n; i += kSelThreads) {
      const uint32_t u = f32_order_key(kr[i]);
      skeys[i] = u;
      kmin = min(kmin, u);
      kmax = max(kmax, u);
    }
    kmin = wave_umin_dpp(kmin);
    kmax = wave_umax_dpp(kmax);
    if ((tid & (kWave - 1)) == 0) {
      hist[tid / kWave] = kmin;   // hist is free until the radix passes clear it
      hist[kSelThreads / kWave + tid / kWave] = kmax;
    }
    __syncthreads();
    for (int w = 0; w < kSelThreads / kWave; ++w) {
      kmin = min(kmin, hist[w]);
      kmax = max(kmax, hist[kSelThreads / kWave + w]);
    }
    __syncthreads();   // every thread has read the range before the first pass clears hist
    auto get = [&](int i) { return skeys[i]; };
    radix_kth<kSelThreads>(get, sz.n, (uint32_t)sz.k, hist, bc, T, need, 4, kmin, kmax);
    ordered_take<kSelThreads>(get, ident, sz.n, T, need, out, scan_scratch);
  } else {
    auto get = [&](int i) { return f32_order_key(kr[i]); };
    radix_kth<kSelThreads>(get, sz.n, (uint32_t)sz.k, hist, bc, T, need);
    ordered_take<kSelThreads>(get, ident, sz.n, T, need, out, scan_scratch);
  }
}

// Token top-k over long sequences: one block of 1024 threads per unit.
//  1. Sample 8192 keys (64 evenly spaced runs of 128) and take the r-th largest sampled key,
//     r = k * 8192 / n plus a 4-sigma margin, as the candidate bound T_lo.
//  2. One pass over all keys keeps (key, index) with key >= T_lo in LDS, in index order: wave w
//     scans the w-th contiguous sixteenth of the keys and compacts into its own LDS segment with
//     ballots (no block barrier per tile); the next tile's loads are issued before the current
//     tile is compacted.
//  3. If at least k candidates were kept (and every segment fit), the top k all lie among them (the
//     k-th largest key is >= T_lo, so every key that ties with it is a candidate too): select
//     exactly in LDS. Otherwise fall back to the radix selection over all keys in global memory.
constexpr int kTokWaves = kTokThreads / kWave;
constexpr int kTokSeg = kTokCand / kTokWaves;   // candidates per wave segment

__global__ __launch_bounds__(kTokThreads) void select_topk_large_kernel(CacheView c, const float *__restrict__ key,
                                                                        int key_stride, int k,
                                                                        int32_t *__restrict__ sel_idx,
                                                                        int32_t *__restrict__ sel_count, int cap) {
  __shared__ uint32_t ckey[kTokCand];
  __shared__ int32_t cidx[kTokCand];
  __shared__ __align__(16) uint32_t hist[kTokWaves * 256];
  __shared__ uint32_t bc[2];
  __shared__ int scan_scratch[kTokWaves + 1];
  __shared__ int seg_cnt[kTokWaves];
  const int unit = blockIdx.x, b = unit / c.Hkv;
  const int n = seq_len(c, b);
  const int kk = min(k, n);
  const float *kr = key + (size_t)unit * key_stride;
  int32_t *out = sel_idx + (size_t)unit * cap;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  if (tid == 0) sel_count[unit] = kk;
  if (kk <= 0) return;
  if (kk >= n) {
    for (int i = tid; i < n; i += kTokThreads) out[i] = i;
    return;
  }
  uint32_t T, need;
  auto lget = [&](int i) { return ckey[i]; };
  auto lidx = [&](int i) { return cidx[i]; };
  if (n <= kTokCand) {
    for (int i = tid; i < n; i += kTokThreads) {
      ckey[i] = f32_order_key(kr[i]);
      cidx[i] = i;
    }
    __syncthreads();
    radix_kth<kTokThreads>(lget, n, (uint32_t)kk, hist, bc, T, need);
    ordered_take<kTokThreads>(lget, lidx, n, T, need, out, scan_scratch);
    return;
  }
  // 1. sample
  const int run = kTokSample / 64, stride = n / 64;
  for (int s = tid; s < kTokSample; s += kTokThreads) ckey[s] = f32_order_key(kr[(s / run) * stride + s % run]);
  __syncthreads();
  const double expect = (double)kk * kTokSample / n;
  const double rs = ceil(expect + 4.0 * sqrt(expect) + 16.0);
  uint32_t Tlo = 0;
  if (rs < kTokSample) {
    radix_kth<kTokThreads>(lget, kTokSample, (uint32_t)rs, hist, bc, T, need, 2);   // a lower bound suffices
    Tlo = T;
  }
  __syncthreads();
  // 2. filtered pass: wave w owns keys [w * span, (w + 1) * span). Per step a wave covers kSub
  //    tiles of 256 keys (4 consecutive keys per lane per tile), all loads issued up front.
  constexpr int kSub = 8;
  const int span = ((n + kTokWaves - 1) / kTokWaves + 255) / 256 * 256;
  const int w0 = min(n, wave * span), w1 = min(n, w0 + span);
  const bool vec = (key_stride & 3) == 0;
  uint32_t *sk = ckey + wave * kTokSeg;
  int32_t *si = cidx + wave * kTokSeg;
  int cnt = 0;   // candidates of this wave (uniform across the wave)
  for (int t0 = w0; t0 < w1; t0 += kSub * 4 * kWave) {
    uint32_t u[kSub][4];
#pragma unroll
    for (int j = 0; j < kSub; ++j) {
      const int i = t0 + j * 4 * kWave + 4 * lane;
      if (vec && i + 3 < w1) {
        const float4 f = *reinterpret_cast<const float4 *>(kr + i);
        u[j][0] = f32_order_key(f.x);
        u[j][1] = f32_order_key(f.y);
        u[j][2] = f32_order_key(f.z);
        u[j][3] = f32_order_key(f.w);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) u[j][e] = i + e < w1 ? f32_order_key(kr[i + e]) : 0u;
      }
    }
#pragma unroll
    for (int j = 0; j < kSub; ++j) {
      const int i = t0 + j * 4 * kWave + 4 * lane;
      bool f[4];
      uint64_t bal[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[e] = (i + e < w1) && u[j][e] >= Tlo;
        bal[e] = __ballot(f[e]);
      }
      // index order is lane-major within a tile: rank = keys of lower lanes + lower e in this lane
      int pos = cnt;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        pos += __builtin_amdgcn_mbcnt_hi((uint32_t)(bal[e] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal[e], 0u));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (f[e]) {
          if (pos < kTokSeg) {
            sk[pos] = u[j][e];
            si[pos] = i + e;
          }
          ++pos;
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) cnt += __popcll(bal[e]);
    }
  }
  if (lane == 0) seg_cnt[wave] = cnt;
  __syncthreads();
  int total = 0;
  bool overflow = false;
  for (int w = 0; w < kTokWaves; ++w) {
    total += seg_cnt[w];
    overflow |= seg_cnt[w] > kTokSeg;
  }
  if (!overflow && total >= kk) {
    // gather the segments into one contiguous list (in place, front to back) so the list is
    // ordered by index; wave w's entries move to the prefix of the earlier segments
    int off = 0;
    for (int w = 0; w < kTokWaves; ++w) {
      const int m = seg_cnt[w];
      uint32_t tk = 0;
      int32_t ti = 0;
      const bool has = tid < m;
      if (has) {
        tk = ckey[w * kTokSeg + tid];
        ti = cidx[w * kTokSeg + tid];
      }
      __syncthreads();
      if (has) {
        ckey[off + tid] = tk;
        cidx[off + tid] = ti;
      }
      __syncthreads();
      off += m;
    }
    radix_kth<kTokThreads>(lget, total, (uint32_t)kk, hist, bc, T, need);
    ordered_take<kTokThreads>(lget, lidx, total, T, need, out, scan_scratch);
    return;
  }
  // 3. fallback: exact radix selection over all keys in global memory
  auto gget = [&](int i) { return f32_order_key(kr[i]); };
  auto gidx = [](int i) { return i; };
  radix_kth<kTokThreads>(gget, n, (uint32_t)kk, hist, bc, T, need);
  ordered_take<kTokThreads>(gget, gidx, n, T, need, out, scan_scratch);
}

// ---------------------------------------------------------------- fused token top-k

constexpr int kBoundSample = 2048;   // tokens scored per unit to place the candidate bound
constexpr int kMaxCandBlocks = 8192; // candidate segments per unit the selection can gather (1M tokens)

// Step 1 of the fused token top-k, one block per unit:
//  - q~ of the unit's G heads (the same float64 sums as the projected-query prep), into the
//    candidate set;
//  - q~ rounded to bf16 and the error-bound coefficients of the approximate key (filter_coef),
//    for the scorer's filter;
//  - 2048 sampled tokens (64 evenly spaced runs of 32) get a lower estimate of their key: the
//    approximate key minus its error bound;
//  - T_lo = the r-th largest estimate with its low 16 bits cleared, r = k * 2048 / L plus a
//    4-sigma margin. Short sequences (L <= 8192) or k >= L keep every token.
// T_lo only steers how many candidates the scorer keeps: the selection certifies it by counting
// (at least k exact keys >= T_lo) and otherwise recomputes the unit exactly.
constexpr int kBoundThreads = 1024;
template <typename T, int D, int R, int G>
__global__ __launch_bounds__(kBoundThreads) void token_bound_kernel(CacheView c, const T *__restrict__ q, int k,
                                                                   const float *__restrict__ proj,
                                                                   const uint16_t *__restrict__ kproj,
                                                                   char *__restrict__ cand, CandLayout lay) {
  constexpr int NT = kBoundThreads;
  constexpr int PER = kBoundSample / NT;    // sampled tokens per thread
  constexpr int PPT = R * D / NT;           // elements of P per thread (R * D is a multiple of NT)
  static_assert(PPT >= 1 && PPT * NT == R * D, "P tile");
  static_assert(G * R <= NT, "one thread per projected query element");
  __shared__ float ps[R][D + 1];            // P, padded rows
  __shared__ float qf[G][D];
  __shared__ uint16_t qh[G * R];            // bf16 q~
  __shared__ uint32_t qmax_bits;
  __shared__ __align__(16) uint32_t hist[NT / kWave * 256];
  __shared__ uint32_t bc[2];
  const int unit = blockIdx.x, b = unit / c.Hkv, g = unit - b * c.Hkv;
  const int tid = threadIdx.x;
  if (unit == 0 && tid == 0) {
    *reinterpret_cast<const uint16_t **>(cand + lay.hdr) = kproj;
    *reinterpret_cast<int32_t *>(cand + lay.hdr + 8) = R;
  }
  if (tid == 0) qmax_bits = 0u;
  // P and q are staged first, so that the barrier waits for them only; the block-table entries
  // of the sampled tokens are then in flight while q~ is formed, and the sampled rows while the
  // filter coefficients are settled
  float pv[PPT];
#pragma unroll
  for (int u = 0; u < PPT; ++u) pv[u] = proj[u * NT + tid];
  const T *qb = q + ((size_t)b * c.Hq + g * G) * D;
  const float qv = tid < G * D ? Elem<T>::get(qb, tid) : 0.0f;
  const int L = seq_len(c, b);
#pragma unroll
  for (int u = 0; u < PPT; ++u) ps[(u * NT + tid) / D][(u * NT + tid) % D] = pv[u];
  if (tid < G * D) qf[tid / D][tid % D] = qv;
  __syncthreads();
  const int kk = min(k, L);
  const bool sample = !(kk >= L || L <= kTokCand);
  const int run = kBoundSample / 64, stride = L / 64;
  int tok[PER], phys[PER];
  uint4 w[PER][R / 8];
  if (sample) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int s = u * NT + tid;
      tok[u] = (s / run) * stride + s % run;
      phys[u] = c.bt[(size_t)b * c.maxP + tok[u] / c.S];
    }
  }
  // q~ of the unit's G heads: the float64 sum over j ascending of P[i][j] q[j], rounded to float
  double *qt = reinterpret_cast<double *>(cand + lay.qt) + (size_t)(b * c.Hq + g * G) * R;
  if (tid < G * R) {
    const int h = tid / R, ii = tid - h * R;
    double acc = 0.0;
#pragma unroll 8
    for (int j = 0; j < D; ++j) acc = fma((double)ps[ii][j], (double)qf[h][j], acc);
    const float qf32 = (float)acc;
    qt[tid] = (double)qf32;
    const uint32_t bits = __float_as_uint(qf32);
    const uint16_t hb = (uint16_t)((bits + 0x7fffu + ((bits >> 16) & 1u)) >> 16);   // nearest even
    qh[tid] = hb;
    reinterpret_cast<uint16_t *>(cand + lay.qb)[(size_t)(b * c.Hq + g * G) * R + tid] = hb;
    const float am = wave_max(fabsf(qf32));
    if ((tid & (kWave - 1)) == 0) atomicMax(&qmax_bits, __float_as_uint(am));
  }
  if (sample) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const uint4 *row = reinterpret_cast<const uint4 *>(
          kproj + (((size_t)phys[u] * c.Hkv + g) * c.S + tok[u] % c.S) * R);
#pragma unroll
      for (int i = 0; i < R / 8; ++i) w[u][i] = row[i];
    }
  }
  __syncthreads();
  const FilterCoef fc = filter_coef(__uint_as_float(qmax_bits));
  uint32_t *bound = reinterpret_cast<uint32_t *>(cand + lay.bound);
  if (tid == 0) reinterpret_cast<float2 *>(cand + lay.qc)[unit] = make_float2(fc.rel, fc.abs);
  if (!sample) {
    if (tid == 0) bound[unit] = 0u;
    return;
  }
  const uint32_t *qp = reinterpret_cast<const uint32_t *>(qh);
  float acc[PER][G], n1[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    n1[u] = 0.0f;
#pragma unroll
    for (int h = 0; h < G; ++h) acc[u][h] = 0.0f;
  }
#pragma unroll
  for (int i = 0; i < R / 8; ++i) {
    int zero = 0;
    asm volatile("" : "+s"(zero));   // keeps each chunk's q~ reads from LDS within the chunk
    const uint32_t *qpi = qp + zero;
#pragma unroll
    for (int pr = 0; pr < 4; ++pr) {
      uint32_t kw[PER];
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        kw[u] = pr == 0 ? w[u][i].x : pr == 1 ? w[u][i].y : pr == 2 ? w[u][i].z : w[u][i].w;
        n1[u] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, kw[u] & 0x7fff7fffu),
                                                __builtin_bit_cast(bf16x2_t, 0x3f803f80u), n1[u], false);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const bf16x2_t qq = __builtin_bit_cast(bf16x2_t, qpi[h * (R / 2) + i * 4 + pr]);
#pragma unroll
        for (int u = 0; u < PER; ++u)
          acc[u][h] = __builtin_amdgcn_fdot2_f32_bf16(qq, __builtin_bit_cast(bf16x2_t, kw[u]), acc[u][h], false);
      }
    }
  }
  uint32_t sk[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    float a = acc[u][0];
#pragma unroll
    for (int h = 1; h < G; ++h) a = fmaxf(a, acc[u][h]);
    sk[u] = f32_order_key(a - fmaf(fc.rel, n1[u], fc.abs));
  }
  const double expect = (double)kk * kBoundSample / L;
  const double rs = ceil(expect + 4.0 * sqrt(expect) + 16.0);
  uint32_t Tlo = 0, need;
  if (rs < kBoundSample) radix_kth_regs<NT, PER>(sk, kBoundSample, (uint32_t)rs, hist, bc, Tlo, need, 2, 0u, 0xffffffffu);
  if (tid == 0) bound[unit] = Tlo;
}

// Token top-k over dense keys on many workgroups (the caller gave the selection a workspace laid
// out like the fused candidate set): the bound of step 1 of select_topk_large_kernel, one block
// per unit; then one wave per group of kCandSegTokens keys writes the keys >= T_lo as (key, token)
// into its segment, in token order, with the count; then select_token_cand_kernel selects exactly.
__global__ __launch_bounds__(kTokThreads) void dense_bound_kernel(CacheView c, const float *__restrict__ key,
                                                                  int key_stride, int k, uint32_t *__restrict__ bound) {
  __shared__ uint32_t ckey[kTokSample];
  __shared__ __align__(16) uint32_t hist[kTokWaves * 256];
  __shared__ uint32_t bc[2];
  const int unit = blockIdx.x, b = unit / c.Hkv;
  const int n = seq_len(c, b);
  const int kk = min(k, n);
  uint32_t Tlo = 0;   // short sequences: every key is a candidate
  if (kk >= 1 && kk < n && n > kTokCand) {
    const float *kr = key + (size_t)unit * key_stride;
    const int run = kTokSample / 64, stride = n / 64;
    for (int s = threadIdx.x; s < kTokSample; s += kTokThreads)
      ckey[s] = f32_order_key(kr[(s / run) * stride + s % run]);
    __syncthreads();
    const double expect = (double)kk * kTokSample / n;
    const double rs = ceil(expect + 4.0 * sqrt(expect) + 16.0);
    if (rs < kTokSample) {
      uint32_t T, need;
      auto lget = [&](int i) { return ckey[i]; };
      radix_kth<kTokThreads>(lget, kTokSample, (uint32_t)rs, hist, bc, T, need, 2);   // a lower bound suffices
      Tlo = T;
    }
  }
  if (threadIdx.x == 0) bound[unit] = Tlo;
}

__global__ __launch_bounds__(256) void dense_filter_kernel(CacheView c, const float *__restrict__ key, int key_stride,
                                                           int vec, const uint32_t *__restrict__ bound,
                                                           int32_t *__restrict__ count, float2 *__restrict__ segs,
                                                           int nb) {
  constexpr int GT = kCandSegTokens, NT = GT / (4 * kWave);   // tiles of 4 keys per lane
  const int unit = blockIdx.y, b = unit / c.Hkv;
  const int n = seq_len(c, b);
  const int lane = threadIdx.x & (kWave - 1), gid = blockIdx.x * 4 + threadIdx.x / kWave;
  const int tg = gid * GT;
  if (tg >= n || gid >= nb) return;
  const uint32_t Tlo = bound[unit];
  const float *kr = key + (size_t)unit * key_stride;
  float2 *seg = segs + ((size_t)unit * nb + gid) * GT;
  float x[NT][4];
#pragma unroll
  for (int j = 0; j < NT; ++j) {   // every load in flight before any compaction
    const int i = tg + j * 4 * kWave + 4 * lane;
    if (vec && i + 3 < n) {
      const float4 f = *reinterpret_cast<const float4 *>(kr + i);
      x[j][0] = f.x;
      x[j][1] = f.y;
      x[j][2] = f.z;
      x[j][3] = f.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[j][e] = i + e < n ? kr[i + e] : 0.0f;
    }
  }
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int i = tg + j * 4 * kWave + 4 * lane;
    bool f[4];
    uint64_t bal[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[e] = i + e < n && f32_order_key(x[j][e]) >= Tlo;
      bal[e] = __ballot(f[e]);
    }
    // token order is lane-major within a tile: rank = keys of lower lanes + lower e in this lane
    int pos = cnt;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      pos += __builtin_amdgcn_mbcnt_hi((uint32_t)(bal[e] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal[e], 0u));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (f[e]) seg[pos] = make_float2(x[j][e], __int_as_float(i + e));
      pos += f[e] ? 1 : 0;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) cnt += __popcll(bal[e]);
  }
  if (lane == 0) count[(size_t)unit * nb + gid] = cnt;
}

// Step 3 of the fused token top-k, one block per unit: gather the unit's candidate segments in
// segment order (so in token order) into LDS and select exactly there.
// When fewer than k candidates arrived, or more than LDS holds, every key of the unit is
// recomputed from the projected keys (same arithmetic), or read from the dense keys (DENSE), and
// selected by radix over global memory.
template <int G, bool DENSE>
__global__ __launch_bounds__(kTokThreads) void select_token_cand_kernel(CacheView c, int k,
                                                                        const char *__restrict__ cand, CandLayout lay,
                                                                        const float *__restrict__ dkey, int dstride,
                                                                        int32_t *__restrict__ sel_idx,
                                                                        int32_t *__restrict__ sel_count, int cap) {
  __shared__ uint32_t ckey[kTokCand];
  __shared__ int32_t cidx[kTokCand];
  __shared__ int soff[kMaxCandBlocks + 1];
  __shared__ __align__(16) uint32_t hist[kTokWaves * 256];
  __shared__ uint32_t bc[2];
  __shared__ int scan_scratch[kTokWaves + 1];
  __shared__ uint32_t range[2 * kTokWaves];
  const int unit = blockIdx.x, b = unit / c.Hkv, g = unit - b * c.Hkv;
  const int n = seq_len(c, b);
  const int kk = min(k, n);
  int32_t *out = sel_idx + (size_t)unit * cap;
  const int tid = threadIdx.x;
  if (tid == 0) sel_count[unit] = kk;
  if (kk <= 0) return;
  if (kk >= n) {
    for (int i = tid; i < n; i += kTokThreads) out[i] = i;
    return;
  }
  const int nb = (n + kCandSegTokens - 1) / kCandSegTokens;
  const int32_t *cnt = reinterpret_cast<const int32_t *>(cand + lay.count) + (size_t)unit * lay.nb;
  const float2 *seg = reinterpret_cast<const float2 *>(cand + lay.seg) + (size_t)unit * lay.nb * kCandSegTokens;
  int base = 0;
  for (int s0 = 0; s0 < nb; s0 += kTokThreads) {
    const int s = s0 + tid;
    const int v = s < nb ? cnt[s] : 0;
    int tot;
    const int ex = block_excl_scan<kTokThreads>(v, scan_scratch, &tot);
    if (s < nb) soff[s] = base + ex;
    base += tot;
  }
  if (tid == 0) soff[nb] = base;
  __syncthreads();
  const int total = base;
  uint32_t T, need;
  if (total >= kk && total <= kTokCand) {
    // candidate f sits in the segment s with soff[s] <= f < soff[s + 1]: eight independent
    // fixed-depth binary searches per thread, then all eight loads in flight at once
    constexpr int GPT = kTokCand / kTokThreads;
    int sg[GPT];
#pragma unroll
    for (int j = 0; j < GPT; ++j) sg[j] = 0;
    // slots past the end load the last candidate (total >= kk >= 1) and are dropped.
    // soff[nb] = total exceeds every f searched, so m >= nb needs no test of its own: the eight
    // LDS reads of a step are unconditional and overlap
    int fs[GPT];
#pragma unroll
    for (int j = 0; j < GPT; ++j) fs[j] = min(tid + j * kTokThreads, total - 1);
    for (int step = 1 << (31 - __clz(nb)); step > 0; step >>= 1) {
      int v[GPT];
#pragma unroll
      for (int j = 0; j < GPT; ++j) v[j] = soff[min(sg[j] + step, nb)];
#pragma unroll
      for (int j = 0; j < GPT; ++j) sg[j] = v[j] <= fs[j] ? sg[j] + step : sg[j];
    }
    float2 e[GPT];
#pragma unroll
    for (int j = 0; j < GPT; ++j) e[j] = seg[(size_t)sg[j] * kCandSegTokens + (fs[j] - soff[sg[j]])];
    uint32_t u[GPT], kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
    for (int j = 0; j < GPT; ++j) {
      const int f = tid + j * kTokThreads;
      u[j] = f32_order_key(e[j].x);
      if (f < total) {
        ckey[f] = u[j];
        cidx[f] = __float_as_int(e[j].y);
        kmin = min(kmin, u[j]);
        kmax = max(kmax, u[j]);
      }
    }
    kmin = wave_umin_dpp(kmin);
    kmax = wave_umax_dpp(kmax);
    if ((tid & (kWave - 1)) == 0) {
      range[tid / kWave] = kmin;
      range[kTokWaves + tid / kWave] = kmax;
    }
    __syncthreads();
    kmin = 0xffffffffu;
    kmax = 0u;
#pragma unroll
    for (int w = 0; w < kTokWaves; ++w) {
      kmin = min(kmin, range[w]);
      kmax = max(kmax, range[kTokWaves + w]);
    }
    auto lget = [&](int i) { return ckey[i]; };
    auto lidx = [&](int i) { return cidx[i]; };
    radix_kth_regs<kTokThreads, GPT>(u, total, (uint32_t)kk, hist, bc, T, need, 4, kmin, kmax);
    ordered_take<kTokThreads>(lget, lidx, total, T, need, out, scan_scratch);
    return;
  }
  if constexpr (DENSE) {   // exact fallback over the dense keys
    const float *kr = dkey + (size_t)unit * dstride;
    auto dget = [&](int t) -> uint32_t { return f32_order_key(kr[t]); };
    auto didx = [](int i) { return i; };
    radix_kth<kTokThreads>(dget, n, (uint32_t)kk, hist, bc, T, need);
    ordered_take<kTokThreads>(dget, didx, n, T, need, out, scan_scratch);
    return;
  }
  // exact fallback: recompute every key of the unit
  const uint16_t *kproj = *reinterpret_cast<const uint16_t *const *>(cand + lay.hdr);
  const int R = *reinterpret_cast<const int32_t *>(cand + lay.hdr + 8);
  const double *qq = reinterpret_cast<const double *>(cand + lay.qt) + (size_t)(b * c.Hq + g * G) * R;
  auto gget = [&](int t) -> uint32_t {
    const int phys = c.bt[(size_t)b * c.maxP + t / c.S];
    const uint4 *row = reinterpret_cast<const uint4 *>(kproj + (((size_t)phys * c.Hkv + g) * c.S + t % c.S) * R);
    double acc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) acc[h] = 0.0;
    for (int i0 = 0; i0 < R / 8; ++i0) {
      const uint4 w = row[i0];
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
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
    return f32_order_key((float)best);
  };
  auto gidx = [](int i) { return i; };
  radix_kth<kTokThreads>(gget, n, (uint32_t)kk, hist, bc, T, need);
  ordered_take<kTokThreads>(gget, gidx, n, T, need, out, scan_scratch);
}

// Every page (or token) of the sequence.
__global__ void select_all_kernel(CacheView c, int tokens, int32_t *__restrict__ sel_idx,
                                  int32_t *__restrict__ sel_count, int cap) {
  const int unit = blockIdx.y, b = unit / c.Hkv;
  const int L = seq_len(c, b);
  const int n = tokens ? L : num_pages(c, L);
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i == 0) sel_count[unit] = n;
  if (i < n) sel_idx[(size_t)unit * cap + i] = i;
}

// ---------------------------------------------------------------- Gaussian-aware threshold

// Standard normal cdf Phi(a) and density phi(a) from one exponential e = exp(-a^2 / 2): the tail
// Phi(-|a|) = e erfcx(z) / 2 with z = |a| / sqrt(2) and erfcx(z) = exp(z^2) erfc(z), which is
// smooth in t = 1 / (1 + z / 2) on (0, 1]: erfcx(z) = t P(2t - 1), P of degree 10 fitted to
// erfcx / t at Chebyshev nodes of t (relative error 1.2e-8 exactly, under 3e-7 evaluated in
// float32). phi(a) = e / sqrt(2 pi).
__device__ __forceinline__ void normal_cdf_pdf(float a, float &Phi, float &phi) {
  const float e = __builtin_amdgcn_exp2f(-0.72134752044448170f * a * a);   // exp(-a^2 / 2)
  const float t = __builtin_amdgcn_rcpf(1.0f + 0.35355339059327376f * fabsf(a));
  const float u = 2.0f * t - 1.0f;
  float p = 4.216376417e-05f;
  p = fmaf(p, u, -3.660316048e-05f);
  p = fmaf(p, u, -2.993884877e-04f);
  p = fmaf(p, u, 4.306730555e-04f);
  p = fmaf(p, u, 1.529161653e-03f);
  p = fmaf(p, u, -3.243453603e-03f);
  p = fmaf(p, u, -1.075162759e-02f);
  p = fmaf(p, u, 1.822166983e-02f);
  p = fmaf(p, u, 1.397357337e-01f);
  p = fmaf(p, u, 3.435803187e-01f);
  p = fmaf(p, u, 5.107913569e-01f);
  const float tail = 0.5f * e * t * p;
  Phi = a >= 0.0f ? 1.0f - tail : tail;
  phi = 0.39894228040143268f * e;
}

// E[(X - tau)_+^(1/(alpha-1))] and its first two tau-derivatives for X ~ N(mu_x, sd^2), alpha in
// {1.5, 2}:
//   alpha = 2:   E = mu Phi(a) + sd phi(a),                 E' = -Phi(a),                      E'' = phi(a) / sd
//   alpha = 1.5: E = (mu^2 + sd^2) Phi(a) + mu sd phi(a),   E' = -2 (mu Phi(a) + sd phi(a)),   E'' = 2 Phi(a)
// with mu = mu_x - tau, a = mu / sd (isd = 1 / sd); a zero sd gives the point-mass values.
__device__ __forceinline__ void gauss_moment(float mu, float sd, float isd, bool sparsemax, float &E, float &dE,
                                             float &d2E) {
  if (sd <= 0.0f) {
    const float pos = fmaxf(mu, 0.0f);
    E = sparsemax ? pos : pos * pos;
    dE = sparsemax ? -(mu > 0.0f ? 1.0f : 0.0f) : -2.0f * pos;
    d2E = sparsemax ? 0.0f : (mu > 0.0f ? 2.0f : 0.0f);
    return;
  }
  float Phi, phi;
  normal_cdf_pdf(mu * isd, Phi, phi);
  const float first = mu * Phi + sd * phi;
  if (sparsemax) {
    E = first;
    dE = -Phi;
    d2E = phi * isd;
  } else {
    E = (mu * mu + sd * sd) * Phi + mu * sd * phi;
    dE = -2.0f * first;
    d2E = 2.0f * Phi;
  }
}

// E[(X - tau)_+^k] for any power k = 1/(alpha-1) >= 1 and its tau-derivative -k E[(X - tau)_+^(k-1)],
// X ~ N(mu + tau, sd^2) (mu = mean - tau): sd^k I_k(a) and -k sd^(k-1) I_(k-1)(a) with a = mu / sd and
// I_j(a) = integral over u >= 0 of u^j phi(u - a) du. Gauss-Legendre, 8 nodes per panel of width at
// most 2 over [max(0, a - 9), max(0, a) + 9] (phi is below 3e-18 of its peak outside); the panel
// that starts at 0 is integrated in v with u = h v^2, which smooths the u^k endpoint. a < -9:
// both are below float resolution and taken as 0.
__device__ __forceinline__ void gauss_moment_general(float mu, float sd, float k, float &E, float &dE) {
  if (sd <= 0.0f) {
    const float pos = fmaxf(mu, 0.0f);
    E = pos > 0.0f ? powf(pos, k) : 0.0f;
    dE = pos > 0.0f ? -k * powf(pos, k - 1.0f) : 0.0f;
    return;
  }
  const float a = mu / sd;
  if (a < -9.0f) {
    E = 0.0f;
    dE = 0.0f;
    return;
  }
  // Gauss-Legendre abscissae and weights of order 8 on [-1, 1] (positive half)
  const float gx[4] = {0.18343464249564980f, 0.52553240991632899f, 0.79666647741362674f, 0.96028985649753623f};
  const float gw[4] = {0.36268378337836198f, 0.31370664587788729f, 0.22238103445337447f, 0.10122853629037626f};
  const float lo = fmaxf(a - 9.0f, 0.0f), hi = fmaxf(a, 0.0f) + 9.0f;
  const int np = (int)ceilf(0.5f * (hi - lo));
  const float h = (hi - lo) / np;
  float ik = 0.0f, ik1 = 0.0f;
  for (int pn = 0; pn < np; ++pn) {
    const float l = lo + pn * h;
    const bool at0 = l == 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x = i < 4 ? -gx[3 - i] : gx[i - 4];
      const float w = i < 4 ? gw[3 - i] : gw[i - 4];
      const float t = 0.5f * (1.0f + x);
      float u, wt;
      if (at0) {   // u = h t^2, du = 2 h t dt
        u = h * t * t;
        wt = w * 0.5f * 2.0f * h * t;
      } else {
        u = l + h * t;
        wt = w * 0.5f * h;
      }
      const float d = u - a;
      const float e = expf(-0.5f * d * d) * wt;
      const float p1 = powf(u, k - 1.0f);
      ik1 += p1 * e;
      ik += p1 * u * e;
    }
  }
  const float c = 0.39894228040143268f;   // 1 / sqrt(2 pi)
  E = powf(sd, k) * ik * c;
  dE = -k * powf(sd, k - 1.0f) * ik1 * c;
}

// The same moments from a table: log I_k and log I_(k-1) at a = -9 + i / 32, i = 0 .. 800
// (a in [-9, 16]), filled once per workgroup by the quadrature above (at sd = 1), then evaluated by
// Catmull-Rom cubics in a. I_k is an infinitely smooth function of a (a convolution with phi) and
// its logarithm is nearly quadratic, so the cubic's error is far below float resolution of F's
// terms. The two end cells, a >= 16 and non-finite table values use the quadrature directly.
constexpr int kItabN = 801;
constexpr float kItabLo = -9.0f, kItabStep = 32.0f;   // grid origin and points per unit of a

__device__ void itab_fill(float k, float *__restrict__ lk, float *__restrict__ lk1) {
  for (int i = threadIdx.x; i < kItabN; i += blockDim.x) {
    float E, dE;
    gauss_moment_general(kItabLo + (float)i / kItabStep, 1.0f, k, E, dE);
    lk[i] = logf(E);
    lk1[i] = logf(-dE / k);
  }
}

__device__ __forceinline__ float catmull_rom(const float *t, int i, float u) {
  const float p0 = t[i - 1], p1 = t[i], p2 = t[i + 1], p3 = t[i + 2];
  return p1 + 0.5f * u * (p2 - p0 + u * (2.0f * p0 - 5.0f * p1 + 4.0f * p2 - p3 + u * (3.0f * (p1 - p2) + p3 - p0)));
}

__device__ __forceinline__ void gauss_moment_tab(float mu, float sd, float k, const float *lk, const float *lk1,
                                                 float &E, float &dE) {
  if (sd > 0.0f) {
    const float a = mu / sd;
    if (a < -9.0f) {
      E = 0.0f;
      dE = 0.0f;
      return;
    }
    const float x = (a - kItabLo) * kItabStep;
    const int i = (int)x;
    if (i >= 1 && i <= kItabN - 3) {
      const float u = x - (float)i;
      const float vk = catmull_rom(lk, i, u), vk1 = catmull_rom(lk1, i, u);
      if (isfinite(vk) && isfinite(vk1)) {   // sd^k I_k and k sd^(k-1) I_(k-1), in the log domain
        const float ls = logf(sd);
        E = expf(fmaf(k, ls, vk));
        dE = -k * expf(fmaf(k - 1.0f, ls, vk1));
        return;
      }
    }
  }
  gauss_moment_general(mu, sd, k, E, dE);
}

// tau_hat per (sequence, query head): root of F(tau) = sum_p n_p E_p(tau) - 1, which is convex
// and non-increasing. Start at tau0 = (alpha-1) max_p m_p - 1, where F >= 0. Far from the root F
// falls off like a Gaussian tail, where plain Newton steps are short; the steps are instead taken
// on g = log S, S = F + 1, which tends to the plain step as S -> 1. With the closed forms (alpha
// 1.5 or 2) F'' comes with F and F' from the same Phi and phi, and the step is Halley's on g
// (tau - 2 g g' / (2 g'^2 - g g''), g' = F'/S, g'' = (F'' S - F'^2) / S^2): about four evaluations
// per head where Newton's on g takes six. With the tabulated moments (other alpha) it is Newton's
// on g (-log(S) S / F'), halved while log S > 2 (there the full step passes the root by about
// half). A bracket [lo, hi] (F(lo) >= 0 > F(hi)) safeguards either: a
// proposal outside falls back to the plain Newton step from the left (at or left of the root, F
// being convex), else to bisection. Per-page terms in float32, sums in float64, one block
// reduction per step. Stops when the bracket is below 2^-20 max(1, |tau|), when the plain step
// -F/F' from either side is that small (then taken: F is at its float noise level), when tau (a
// float) no longer moves, or after 64 steps. The
// scaled page terms stay in LDS across the steps (pages beyond kTauLds are read each step).
constexpr int kTauThreads = 1024;
constexpr int kTauLds = 4096;
// KIND: 0 alpha = 1.5, 1 alpha = 2 (closed forms), 2 any other alpha in (1, 2) (tabulated quadrature)
template <int KIND>
__global__ __launch_bounds__(kTauThreads) void tau_hat_kernel(CacheView c, const float *__restrict__ m,
                                                              const float *__restrict__ s, float alpha,
                                                              float *__restrict__ tau_out) {
  __shared__ float t_mu[kTauLds], t_sd[kTauLds], t_isd[kTauLds];
  __shared__ double red3[3 * (kTauThreads / kWave)];
  __shared__ int s_step[2];   // tau (bits) and whether the iteration is over, from wave 0
  __shared__ float redf[kTauThreads / kWave];
  __shared__ float t_lk[KIND == 2 ? kItabN : 1], t_lk1[KIND == 2 ? kItabN : 1];
  const int bh = blockIdx.x, b = bh / c.Hq;
  const int L = seq_len(c, b);
  const int P = num_pages(c, L);
  const float *mr = m + (size_t)bh * c.maxP, *sr = s + (size_t)bh * c.maxP;
  if (P == 0) {
    if (threadIdx.x == 0) tau_out[bh] = NAN;
    return;
  }
  const float am1 = alpha - 1.0f;
  const float kpow = 1.0f / am1;
  if (KIND == 2) itab_fill(kpow, t_lk, t_lk1);   // published by the barrier of block_max below
  float mx = -INFINITY;
  for (int p = threadIdx.x; p < P; p += kTauThreads) {
    const float mv = mr[p];
    mx = fmaxf(mx, mv);
    if (p < kTauLds) {
      const float sd = am1 * sr[p];
      t_mu[p] = am1 * mv;
      t_sd[p] = sd;
      t_isd[p] = sd > 0.0f ? 1.0f / sd : 0.0f;
    }
  }
  mx = block_max<kTauThreads>(mx, redf);   // its barrier also publishes the LDS terms
  float tau = am1 * mx - 1.0f, lo = tau, hi = INFINITY;
  for (int it = 0; it < 64; ++it) {
    double F = 0.0, dF = 0.0, d2F = 0.0;
    for (int p = threadIdx.x; p < P; p += kTauThreads) {
      float mu, sd, isd;
      if (p < kTauLds) {
        mu = t_mu[p];
        sd = t_sd[p];
        isd = t_isd[p];
      } else {
        mu = am1 * mr[p];
        sd = am1 * sr[p];
        isd = sd > 0.0f ? 1.0f / sd : 0.0f;
      }
      const float n = (float)min(c.S, L - p * c.S);
      float E, dE, d2E = 0.0f;
      if (KIND == 2)
        gauss_moment_tab(mu - tau, sd, kpow, t_lk, t_lk1, E, dE);
      else
        gauss_moment(mu - tau, sd, isd, KIND == 1, E, dE, d2E);
      F += (double)(n * E);
      dF += (double)(n * dE);
      if (KIND != 2) d2F += (double)(n * d2E);
    }
    // the waves' sums go to wave 0, which alone takes the step (the sums in the same order as a
    // block reduction) and hands tau, and whether the iteration is over, to the others in LDS
    F = wave_sum_dpp(F);
    dF = wave_sum_dpp(dF);
    d2F = wave_sum_dpp(d2F);
    constexpr int NW = kTauThreads / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) {
      const int w = threadIdx.x / kWave;
      red3[w] = F;
      red3[NW + w] = dF;
      red3[2 * NW + w] = d2F;
    }
    __syncthreads();
    if (threadIdx.x < kWave) {
      F = 0.0;
      dF = 0.0;
      d2F = 0.0;
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        F += red3[i];
        dF += red3[NW + i];
        d2F += red3[2 * NW + i];
      }
      bool done = false;
      F -= 1.0;
      if (!(F != 0.0)) {   // on the root, or not a number
        done = true;
      } else {
        if (F > 0.0) lo = tau; else hi = tau;
        const double tol = 0x1p-20 * fmax(1.0, fabs((double)tau));
        const double S = F + 1.0;
        const bool left_ok = F > 0.0 && dF < 0.0;
        if ((double)hi - (double)lo <= tol) {
          done = true;
        } else if (dF < 0.0 && fabs(F / dF) <= tol) {   // within the float noise of F: one plain step
          tau = (float)((double)tau - F / dF);
          done = true;
        } else {
          float next = NAN;
          if (dF < 0.0 && S > 0.0) {
            const double ls = log(S);
            if (KIND != 2) {
              const double g1 = dF / S, g2 = (d2F * S - dF * dF) / (S * S), den = 2.0 * g1 * g1 - ls * g2;
              if (den > 0.0) next = (float)((double)tau - 2.0 * ls * g1 / den);
            } else {
              next = (float)((double)tau - (ls > 2.0 ? 0.5 : 1.0) * ls * S / dF);   // halved far out, where it overshoots
            }
          }
          if (!(next > lo && next < hi) && left_ok) next = (float)((double)tau - F / dF);
          if (!(next > lo && next < hi)) next = hi < INFINITY ? 0.5f * (lo + hi) : lo + 2.0f * (tau - lo + 1.0f);
          if (next == tau) done = true; else tau = next;
        }
      }
      if (threadIdx.x == 0) {
        s_step[0] = __float_as_int(tau);
        s_step[1] = done ? 1 : 0;
      }
    }
    __syncthreads();
    tau = __int_as_float(s_step[0]);
    if (s_step[1]) break;
  }
  if (threadIdx.x == 0) tau_out[bh] = tau;
}

// Keep page p of unit (b, g) iff some head h of g has (alpha-1) shat_h(p) > tau_h - delta;
// ordered compaction. Each thread takes kThreshPPT consecutive pages of a tile, with the loads of
// all of them (and of every head) issued before the tests, so a tile costs one round of loads and
// one block scan.
constexpr int kThreshThreads = 1024;
constexpr int kThreshPPT = 4;
__global__ __launch_bounds__(kThreshThreads) void select_thresh_kernel(CacheView c, const float *__restrict__ shat,
                                                                       const float *__restrict__ tau, float alpha,
                                                                       float delta, int32_t *__restrict__ sel_idx,
                                                                       int32_t *__restrict__ sel_count, int cap) {
  __shared__ int scan_scratch[kThreshThreads / kWave + 1];
  const int unit = blockIdx.x, b = unit / c.Hkv, g = unit - b * c.Hkv;
  const int P = num_pages(c, seq_len(c, b));
  const float am1 = alpha - 1.0f;
  int32_t *out = sel_idx + (size_t)unit * cap;
  int base = 0;
  for (int t0 = 0; t0 < P; t0 += kThreshThreads * kThreshPPT) {
    const int p0 = t0 + threadIdx.x * kThreshPPT;
    bool keep[kThreshPPT];
#pragma unroll
    for (int u = 0; u < kThreshPPT; ++u) keep[u] = false;
    for (int h = 0; h < c.G; ++h) {
      const int bh = b * c.Hq + g * c.G + h;
      const float bar = tau[bh] - delta;
      const float *sr = shat + (size_t)bh * c.maxP;
      float x[kThreshPPT];
#pragma unroll
      for (int u = 0; u < kThreshPPT; ++u) x[u] = p0 + u < P ? sr[p0 + u] : -INFINITY;
#pragma unroll
      for (int u = 0; u < kThreshPPT; ++u) keep[u] = keep[u] || am1 * x[u] > bar;
    }
    int n = 0;
#pragma unroll
    for (int u = 0; u < kThreshPPT; ++u) n += keep[u] ? 1 : 0;
    int tot;
    int pos = base + block_excl_scan<kThreshThreads>(n, scan_scratch, &tot);
#pragma unroll
    for (int u = 0; u < kThreshPPT; ++u)
      if (keep[u]) out[pos++] = p0 + u;
    base += tot;
  }
  if (threadIdx.x == 0) sel_count[unit] = base;
}

// The threshold policy with the box bound as the page's estimated maximum ("EntmaxKV" summary
// s2.A's deterministic bound in s2.B's threshold test): keep page p of unit (b, g) iff
// (alpha-1) scale key[p] > min_h tau_h - delta over the G heads of g, key = the unit's box key
// (max over its heads of the unscaled bound). Every page the per-head box test would keep is kept.
__global__ __launch_bounds__(kThreshThreads) void select_thresh_box_kernel(CacheView c, const float *__restrict__ key,
                                                                           const float *__restrict__ tau, float alpha,
                                                                           float scale, float delta,
                                                                           int32_t *__restrict__ sel_idx,
                                                                           int32_t *__restrict__ sel_count, int cap) {
  __shared__ int scan_scratch[kThreshThreads / kWave + 1];
  const int unit = blockIdx.x, b = unit / c.Hkv, g = unit - b * c.Hkv;
  const int P = num_pages(c, seq_len(c, b));
  float tmin = INFINITY;
  for (int h = 0; h < c.G; ++h) tmin = fminf(tmin, tau[b * c.Hq + g * c.G + h]);
  const float bar = tmin - delta, f = (alpha - 1.0f) * scale;
  const float *kr = key + (size_t)unit * c.maxP;
  int32_t *out = sel_idx + (size_t)unit * cap;
  int base = 0;
  for (int t0 = 0; t0 < P; t0 += kThreshThreads * kThreshPPT) {
    const int p0 = t0 + threadIdx.x * kThreshPPT;
    float x[kThreshPPT];
#pragma unroll
    for (int u = 0; u < kThreshPPT; ++u) x[u] = p0 + u < P ? kr[p0 + u] : -INFINITY;
    bool keep[kThreshPPT];
    int n = 0;
#pragma unroll
    for (int u = 0; u < kThreshPPT; ++u) {
      keep[u] = p0 + u < P && f * x[u] > bar;
      n += keep[u] ? 1 : 0;
    }
    int tot;
    int pos = base + block_excl_scan<kThreshThreads>(n, scan_scratch, &tot);
#pragma unroll
    for (int u = 0; u < kThreshPPT; ++u)
      if (keep[u]) out[pos++] = p0 + u;
    base += tot;
  }
  if (threadIdx.x == 0) sel_count[unit] = base;
}

hipError_t launch_select_topk(const CacheView &c, const float *key, int key_stride, int policy, int k, int pct,
                              int32_t *sel_idx, int32_t *sel_count, int cap, hipStream_t st) {
  if (policy == 3)
    select_topk_large_kernel<<<c.B * c.Hkv, kTokThreads, 0, st>>>(c, key, key_stride, k, sel_idx, sel_count, cap);
  else
    select_topk_kernel<<<c.B * c.Hkv, kSelThreads, 0, st>>>(c, key, key_stride, policy, k, pct, sel_idx, sel_count,
                                                            cap);
  return hipGetLastError();
}

template <typename T, int D, int R>
static hipError_t token_bound_r(const CacheView &c, const void *q, int k, const float *proj, const uint16_t *kproj,
                                char *cand, const CandLayout &lay, hipStream_t st) {
  switch (c.G) {
    case 1: token_bound_kernel<T, D, R, 1><<<c.B * c.Hkv, kBoundThreads, 0, st>>>(c, static_cast<const T *>(q), k, proj, kproj, cand, lay); break;
    case 2: token_bound_kernel<T, D, R, 2><<<c.B * c.Hkv, kBoundThreads, 0, st>>>(c, static_cast<const T *>(q), k, proj, kproj, cand, lay); break;
    case 4: token_bound_kernel<T, D, R, 4><<<c.B * c.Hkv, kBoundThreads, 0, st>>>(c, static_cast<const T *>(q), k, proj, kproj, cand, lay); break;
    case 8: token_bound_kernel<T, D, R, 8><<<c.B * c.Hkv, kBoundThreads, 0, st>>>(c, static_cast<const T *>(q), k, proj, kproj, cand, lay); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t token_bound_d(const CacheView &c, const void *q, int k, int r, const float *proj,
                                const uint16_t *kproj, char *cand, const CandLayout &lay, hipStream_t st) {
  switch (r) {
    case 16: return token_bound_r<T, D, 16>(c, q, k, proj, kproj, cand, lay, st);
    case 32: return token_bound_r<T, D, 32>(c, q, k, proj, kproj, cand, lay, st);
    case 64: return token_bound_r<T, D, 64>(c, q, k, proj, kproj, cand, lay, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_token_bound(const CacheView &c, int dtype, const void *q, int k, int r, const float *proj,
                              const uint16_t *kproj, char *cand, hipStream_t st) {
  const CandLayout lay(c.B, c.Hq, c.Hkv, c.maxP * c.S, 64);   // layout independent of the rank
  if (dtype == 0)
    return c.D == 64 ? token_bound_d<float, 64>(c, q, k, r, proj, kproj, cand, lay, st)
                     : token_bound_d<float, 128>(c, q, k, r, proj, kproj, cand, lay, st);
  return c.D == 64 ? token_bound_d<uint16_t, 64>(c, q, k, r, proj, kproj, cand, lay, st)
                   : token_bound_d<uint16_t, 128>(c, q, k, r, proj, kproj, cand, lay, st);
}

hipError_t launch_select_token_cand(const CacheView &c, int k, int r, const char *cand, int32_t *sel_idx,
                                    int32_t *sel_count, int cap, hipStream_t st) {
  const CandLayout lay(c.B, c.Hq, c.Hkv, c.maxP * c.S, 64);   // layout independent of the rank
  const dim3 grid(c.B * c.Hkv);
  switch (c.G) {
#define SKV_TOKCAND(GG)                                                                                         \
  case GG:                                                                                                      \
    select_token_cand_kernel<GG, false><<<grid, kTokThreads, 0, st>>>(c, k, cand, lay, nullptr, 0, sel_idx, \
                                                                      sel_count, cap);                      \
    break;
    SKV_TOKCAND(1) SKV_TOKCAND(2) SKV_TOKCAND(4) SKV_TOKCAND(8)
#undef SKV_TOKCAND
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_select_token_dense(const CacheView &c, const float *key, int key_stride, int k, char *ws,
                                     int32_t *sel_idx, int32_t *sel_count, int cap, hipStream_t st) {
  const CandLayout lay(c.B, c.Hq, c.Hkv, c.maxP * c.S, 64);
  uint32_t *bound = reinterpret_cast<uint32_t *>(ws + lay.bound);
  int32_t *count = reinterpret_cast<int32_t *>(ws + lay.count);
  float2 *segs = reinterpret_cast<float2 *>(ws + lay.seg);
  const int U = c.B * c.Hkv;
  dense_bound_kernel<<<U, kTokThreads, 0, st>>>(c, key, key_stride, k, bound);
  const int vec = (key_stride % 4 == 0) && (reinterpret_cast<uintptr_t>(key) % 16 == 0);
  dense_filter_kernel<<<dim3((lay.nb + 3) / 4, U), 256, 0, st>>>(c, key, key_stride, vec, bound, count, segs, lay.nb);
  select_token_cand_kernel<1, true><<<U, kTokThreads, 0, st>>>(c, k, ws, lay, key, key_stride, sel_idx, sel_count,
                                                                cap);
  return hipGetLastError();
}

hipError_t launch_select_all(const CacheView &c, int tokens, int32_t *sel_idx, int32_t *sel_count, int cap,
                             hipStream_t st) {
  const int n = tokens ? c.maxP * c.S : c.maxP;
  select_all_kernel<<<dim3((n + 255) / 256, c.B * c.Hkv), 256, 0, st>>>(c, tokens, sel_idx, sel_count, cap);
  return hipGetLastError();
}

hipError_t launch_tau_hat(const CacheView &c, const float *m, const float *s, float alpha, float *tau,
                          hipStream_t st) {
  const dim3 grid(c.B * c.Hq);
  if (alpha == 1.5f)
    tau_hat_kernel<0><<<grid, kTauThreads, 0, st>>>(c, m, s, alpha, tau);
  else if (alpha == 2.0f)
    tau_hat_kernel<1><<<grid, kTauThreads, 0, st>>>(c, m, s, alpha, tau);
  else
    tau_hat_kernel<2><<<grid, kTauThreads, 0, st>>>(c, m, s, alpha, tau);
  return hipGetLastError();
}

hipError_t launch_select_thresh_box(const CacheView &c, const float *m, const float *s, const float *key, float alpha,
                                    float scale, float delta, float *tau, int32_t *sel_idx, int32_t *sel_count,
                                    int cap, hipStream_t st) {
  hipError_t e = launch_tau_hat(c, m, s, alpha, tau, st);
  if (e != hipSuccess) return e;
  select_thresh_box_kernel<<<c.B * c.Hkv, kThreshThreads, 0, st>>>(c, key, tau, alpha, scale, delta, sel_idx,
                                                                   sel_count, cap);
  return hipGetLastError();
}

hipError_t launch_select_thresh(const CacheView &c, const float *m, const float *s, const float *shat, float alpha,
                                float delta, float *tau, int32_t *sel_idx, int32_t *sel_count, int cap, hipStream_t st) {
  hipError_t e = launch_tau_hat(c, m, s, alpha, tau, st);
  if (e != hipSuccess) return e;
  select_thresh_kernel<<<c.B * c.Hkv, kThreshThreads, 0, st>>>(c, shat, tau, alpha, delta, sel_idx, sel_count, cap);
  return hipGetLastError();
}

}  // namespace skv
