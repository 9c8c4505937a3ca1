/*
 * skv_oracle.c -- plain, slow, float64 CPU oracle for query-aware sparse decode attention
 * over a paged grouped-query (GQA) KV cache.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the package smoke check and the benchmark's
 * CPU-baseline leg may load this library. The GPU library never links, loads or calls it, and
 * the two share no source: this file decodes bf16 itself, sorts with the C library's qsort,
 * and runs every sum in float64 in plain index order (j = 0, 1, ..., d-1; t ascending).
 *
 * Sources, by page title and section (the pages are summaries of the papers):
 *   [EKV]    "EntmaxKV - Decodificacao Consciente de Suporte para Atencao Entmax"
 *            (gist.science/pt/paper/2605.21649): s1 problem, s2.A query-aware page scoring,
 *            s2.B candidate selection policies, s2.C sparse entmax attention, s3 theory.
 *   [JSSA]   "Joint Subspace Sparse Attention per una decodifica efficiente con contesti
 *            lunghi" (ai.info, 2610.19026), authors' abstract: token-level scoring in a shared
 *            low-dimensional q/k subspace, distinct selection per KV head, GQA paged layout.
 *   [SOCKET] "SOCKET - Estimador de Kernel de Colisao Suave para Atencao Esparsa"
 *            (gist.science/pt/paper/2602.06283), Methodology, soft LSH steps 1-4: hashing of
 *            keys into L tables with cached value norms, soft bucket assignment of the query,
 *            per-key soft-collision scores, deterministic top-k and exact attention.
 *   [NOSA]   "NOSA: Atencao Esparsa Nativa e Descarregavel" (gist.science/pt/paper/2510.13602),
 *            Algorithm: mean pooling over sub-blocks, then max pooling, as a block score.
 *   alpha-entmax itself is not printed on the pages; it is taken from its published
 *   definition (Peters, Niculae & Martins, 2019): p = [(alpha-1) z - tau]_+^(1/(alpha-1)),
 *   sum p = 1; alpha -> 1 is softmax, alpha = 2 is sparsemax (Martins & Astudillo, 2016).
 *
 * Layouts (row-major, element strides):
 *   k, v        [Nphys, Hkv, S, d]   dtype f32 or bf16 (raw 16-bit patterns)
 *   q           [B, Hq, d]           same dtype as k
 *   block_table [B, maxP] int32      logical page -> physical page
 *   seq_lens    [B] int32            clamped to [0, maxP*S]
 *   query head h belongs to KV head g = h / G, G = Hq / Hkv.
 * Page p of sequence b holds tokens [p*S, min(p*S+S, L_b)); n_p is that count.
 * A physical page is assumed to be referenced by at most one (sequence, logical page).
 *
 * Every function is single-threaded and reentrant; callers may run units in parallel threads.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_BF16 = 1 };

typedef struct {
  int32_t B, Hq, Hkv, d, S, maxP, Nphys, dtype;
  const void *k, *v, *q;
  const int32_t *block_table, *seq_lens;
} orc_cache;

/* ------------------------------------------------------------------ helpers */

/* bf16 is the top half of an IEEE binary32: widen the 16-bit pattern by 16 zero bits. */
static double orc_decode(const void *base, size_t i, int dtype) {
  if (dtype == ORC_F32) return (double)((const float *)base)[i];
  uint32_t u = (uint32_t)((const uint16_t *)base)[i] << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static int64_t orc_len(const orc_cache *c, int32_t b) {
  int64_t L = c->seq_lens[b];
  int64_t cap = (int64_t)c->maxP * c->S;
  if (L < 0) L = 0;
  if (L > cap) L = cap;
  return L;
}

static int32_t orc_pages(const orc_cache *c, int32_t b) {
  return (int32_t)((orc_len(c, b) + c->S - 1) / c->S);
}

static int32_t orc_page_tokens(const orc_cache *c, int32_t b, int32_t p) {
  int64_t rest = orc_len(c, b) - (int64_t)p * c->S;
  return (int32_t)(rest < c->S ? rest : c->S);
}

static int32_t orc_phys(const orc_cache *c, int32_t b, int32_t p) {
  return c->block_table[(size_t)b * c->maxP + p];
}

static size_t orc_kv_at(const orc_cache *c, int32_t phys, int32_t g, int32_t t, int32_t j) {
  return (((size_t)phys * c->Hkv + g) * c->S + t) * c->d + j;
}

static double orc_q(const orc_cache *c, int32_t b, int32_t h, int32_t j) {
  return orc_decode(c->q, ((size_t)b * c->Hq + h) * c->d + j, c->dtype);
}

/* Round a double to the nearest bf16 value, ties to even, by scaling its significand to
 * 8 bits and rounding with nearbyint (the default rounding mode is round-to-nearest-even).
 * Below 2^-126 bf16 is subnormal with a fixed quantum of 2^-133. Returns the 16-bit pattern. */
uint16_t orc_round_bf16(double x) {
  if (isnan(x)) return 0x7fc0;
  double y;
  if (x == 0.0) {
    y = x;
  } else if (fabs(x) < 0x1p-126) {
    y = nearbyint(x * 0x1p133) * 0x1p-133;
  } else {
    int e;
    frexp(x, &e); /* x = f * 2^e, 0.5 <= |f| < 1 */
    y = ldexp(nearbyint(ldexp(x, 8 - e)), e - 8);
  }
  float f = (float)y; /* exact: y has at most 8 significant bits; overflow gives inf */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------ page metadata */

/* [EKV] s2.A, bounding-box bullet: coordinate-wise minimum and maximum of the keys of a page.
 * Computed over the page's valid tokens. Output [Nphys, Hkv, d]; pages no sequence uses are
 * left untouched. */
void orc_meta_box(const orc_cache *c, double *kmin, double *kmax) {
  for (int32_t b = 0; b < c->B; ++b)
    for (int32_t p = 0; p < orc_pages(c, b); ++p) {
      int32_t phys = orc_phys(c, b, p), n = orc_page_tokens(c, b, p);
      for (int32_t g = 0; g < c->Hkv; ++g)
        for (int32_t j = 0; j < c->d; ++j) {
          double lo = INFINITY, hi = -INFINITY;
          for (int32_t t = 0; t < n; ++t) {
            double x = orc_decode(c->k, orc_kv_at(c, phys, g, t, j), c->dtype);
            if (x < lo) lo = x;
            if (x > hi) hi = x;
          }
          size_t o = ((size_t)phys * c->Hkv + g) * c->d + j;
          kmin[o] = lo;
          kmax[o] = hi;
        }
    }
}

/* [EKV] s2.A, Gaussian-statistics bullet: first and second moments of the keys of a page.
 * Reading: per coordinate (diagonal), population variance (divide by n_p), valid tokens only,
 * two passes (mean first, then the mean squared deviation). Output [Nphys, Hkv, d]. */
void orc_meta_gauss(const orc_cache *c, double *mean, double *var) {
  for (int32_t b = 0; b < c->B; ++b)
    for (int32_t p = 0; p < orc_pages(c, b); ++p) {
      int32_t phys = orc_phys(c, b, p), n = orc_page_tokens(c, b, p);
      for (int32_t g = 0; g < c->Hkv; ++g)
        for (int32_t j = 0; j < c->d; ++j) {
          double sum = 0.0;
          for (int32_t t = 0; t < n; ++t) sum += orc_decode(c->k, orc_kv_at(c, phys, g, t, j), c->dtype);
          double mu = sum / n;
          double ss = 0.0;
          for (int32_t t = 0; t < n; ++t) {
            double dv = orc_decode(c->k, orc_kv_at(c, phys, g, t, j), c->dtype) - mu;
            ss += dv * dv;
          }
          size_t o = ((size_t)phys * c->Hkv + g) * c->d + j;
          mean[o] = mu;
          var[o] = ss / n;
        }
    }
}

/* [NOSA] section 1, block-level selection scores: mean pooling within sub-blocks, then max
 * pooling over the block. Reading: a page is the block; its sub-blocks are the runs of
 * pb consecutive token slots [j pb, j pb + pb) (pb divides S); the metadata of sub-block j is
 * RN_f32 of the float64 mean (sum over its valid tokens t ascending, then divided by their number)
 * of the keys, stored [Nphys, Hkv, S / pb, d]; sub-blocks without a valid token are not written.
 * The mean of the scores q . k_t over a sub-block equals q . (its mean key), so pooling scores and
 * pooling keys agree. */
void orc_meta_pool(const orc_cache *c, int32_t pb, float *pool) {
  int32_t nsb = c->S / pb;
  for (int32_t b = 0; b < c->B; ++b)
    for (int32_t p = 0; p < orc_pages(c, b); ++p) {
      int32_t phys = orc_phys(c, b, p), n = orc_page_tokens(c, b, p);
      for (int32_t g = 0; g < c->Hkv; ++g)
        for (int32_t sb = 0; sb < nsb; ++sb) {
          int32_t t0 = sb * pb, t1 = t0 + pb < n ? t0 + pb : n;
          if (t0 >= t1) continue;
          for (int32_t j = 0; j < c->d; ++j) {
            double sum = 0.0;
            for (int32_t t = t0; t < t1; ++t) sum += orc_decode(c->k, orc_kv_at(c, phys, g, t, j), c->dtype);
            pool[(((size_t)phys * c->Hkv + g) * nsb + sb) * c->d + j] = (float)(sum / (t1 - t0));
          }
        }
    }
}

/* [JSSA] abstract: keys are scored in a shared low-dimensional subspace. Reading: one
 * projection P [r, d] (float32) shared by queries and keys of every head; the projected key
 * k~_t[i] = RN_bf16(sum_j P[i][j] k_t[j]), summed in float64 over j ascending, is cached per
 * token. Output kproj [Nphys, Hkv, S, r] as bf16 patterns; rows of invalid tokens untouched. */
void orc_meta_proj(const orc_cache *c, int32_t r, const float *P, uint16_t *kproj) {
  for (int32_t b = 0; b < c->B; ++b)
    for (int32_t p = 0; p < orc_pages(c, b); ++p) {
      int32_t phys = orc_phys(c, b, p), n = orc_page_tokens(c, b, p);
      for (int32_t g = 0; g < c->Hkv; ++g)
        for (int32_t t = 0; t < n; ++t)
          for (int32_t i = 0; i < r; ++i) {
            double acc = 0.0;
            for (int32_t j = 0; j < c->d; ++j)
              acc += (double)P[(size_t)i * c->d + j] * orc_decode(c->k, orc_kv_at(c, phys, g, t, j), c->dtype);
            kproj[(((size_t)phys * c->Hkv + g) * c->S + t) * r + i] = orc_round_bf16(acc);
          }
    }
}

/* [SOCKET] Methodology, soft LSH step 1 (prefill): each key is hashed into L tables by random
 * projections, one bucket id per table, and the norm of its value vector is kept. Reading (the
 * page names neither the hash family nor the table width): table l has P hyperplanes
 * w_{l,0..P-1} (float32 rows of planes [L, P, d], given); bit i of the key's bucket id is set iff
 * w_{l,i}.k > 0, the dot a float64 sum over j ascending (f32 x bf16 and f32 x f32 products are
 * exact in float64), so ids lie in [0, 2^P). The value norm is RN_f32(sqrt(sum_j v_j^2)), the sum
 * in float64. Outputs bucket [Nphys, Hkv, S, L] uint8 and vnorm [Nphys, Hkv, S] float32; rows of
 * invalid tokens are left untouched. */
void orc_meta_lsh(const orc_cache *c, int32_t L, int32_t P, const float *planes, uint8_t *bucket, float *vnorm) {
  for (int32_t b = 0; b < c->B; ++b)
    for (int32_t p = 0; p < orc_pages(c, b); ++p) {
      int32_t phys = orc_phys(c, b, p), n = orc_page_tokens(c, b, p);
      for (int32_t g = 0; g < c->Hkv; ++g)
        for (int32_t t = 0; t < n; ++t) {
          size_t row = ((size_t)phys * c->Hkv + g) * c->S + t;
          for (int32_t l = 0; l < L; ++l) {
            uint32_t id = 0;
            for (int32_t i = 0; i < P; ++i) {
              const float *w = planes + ((size_t)l * P + i) * c->d;
              double dot = 0.0;
              for (int32_t j = 0; j < c->d; ++j) dot += (double)w[j] * orc_decode(c->k, orc_kv_at(c, phys, g, t, j), c->dtype);
              if (dot > 0.0) id |= 1u << i;
            }
            bucket[row * L + l] = (uint8_t)id;
          }
          double ss = 0.0;
          for (int32_t j = 0; j < c->d; ++j) {
            double x = orc_decode(c->v, orc_kv_at(c, phys, g, t, j), c->dtype);
            ss += x * x;
          }
          vnorm[row] = (float)sqrt(ss);
        }
    }
}

/* ------------------------------------------------------------------ page / token scores */

/* [EKV] s2.A, bounding box: the largest q.k over all keys in the box [kmin, kmax] is
 * U_h(p) = sum_j max(q_j kmin_j, q_j kmax_j), an upper bound on the page's true maximum.
 * Reading for GQA (one selection per KV head, [JSSA]): the KV head's key is the maximum
 * over its G query heads. The key is left unscaled (a positive scale does not change the
 * ranking) and rounded once to float32. Products of f32/bf16 values are exact in float64.
 * Output key [B, Hkv, maxP]; pages at or beyond P_b get -inf. */
void orc_score_box(const orc_cache *c, const double *kmin, const double *kmax, float *key) {
  int32_t G = c->Hq / c->Hkv;
  for (int32_t b = 0; b < c->B; ++b)
    for (int32_t g = 0; g < c->Hkv; ++g)
      for (int32_t p = 0; p < c->maxP; ++p) {
        float *out = &key[((size_t)b * c->Hkv + g) * c->maxP + p];
        if (p >= orc_pages(c, b)) {
          *out = -INFINITY;
          continue;
        }
        const double *lo = &kmin[((size_t)orc_phys(c, b, p) * c->Hkv + g) * c->d];
        const double *hi = &kmax[((size_t)orc_phys(c, b, p) * c->Hkv + g) * c->d];
        double best = -INFINITY;
        for (int32_t h = g * G; h < g * G + G; ++h) {
          double U = 0.0;
          for (int32_t j = 0; j < c->d; ++j) {
            double qj = orc_q(c, b, h, j);
            double a = qj * lo[j], e = qj * hi[j];
            U += (a > e ? a : e);
          }
          if (U > best) best = U;
        }
        *out = (float)best;
      }
}

/* [EKV] s2.A, Gaussian statistics: model the scaled scores z = scale * q.k of a page's tokens
 * as a Gaussian. With the diagonal moments, m = scale * sum_j q_j mu_j and
 * s = scale * sqrt(sum_j q_j^2 var_j). The "estimated maximum score" of s2.B is read as
 * shat = m + s * sqrt(2 ln n_p), the standard bound on the expected maximum of n_p Gaussians
 * (shat = m when n_p = 1). Outputs [B, Hq, maxP]; invalid pages get NaN. */
static double orc_Phi(double a);

/* Phi^-1(p) for 0 < p < 1: bisection on Phi over [-40, 40] down to adjacent doubles. */
double orc_Phi_inv(double p) {
  double lo = -40.0, hi = 40.0;
  for (int it = 0; it < 200 && hi - lo > 0.0; ++it) {
    double mid = 0.5 * (lo + hi);
    if (mid <= lo || mid >= hi) break;
    if (orc_Phi(mid) < p) lo = mid; else hi = mid;
  }
  return 0.5 * (lo + hi);
}

/* Phi^-1(1 - q) for 0 < q < 1, accurate in the upper tail: bisection on the upper tail
 * Q(x) = erfc(x / sqrt 2) / 2 = q (1 - q itself would lose the digits of a small q). */
double orc_Phi_inv_upper(double q) {
  double lo = -40.0, hi = 40.0;
  for (int it = 0; it < 200 && hi - lo > 0.0; ++it) {
    double mid = 0.5 * (lo + hi);
    if (mid <= lo || mid >= hi) break;
    if (0.5 * erfc(mid / sqrt(2.0)) > q) lo = mid; else hi = mid;
  }
  return 0.5 * (lo + hi);
}

void orc_score_gauss(const orc_cache *c, const double *mean, const double *var, double scale, int32_t quantile,
                     double *m, double *s, double *shat) {
  int32_t G = c->Hq / c->Hkv;
  /* the estimated-maximum factor per page size n: sqrt(2 ln n), or Phi^-1(1 - 1/n) (quantile) */
  double *fac = (double *)malloc(sizeof(double) * (size_t)(c->S + 1));
  for (int32_t n = 1; n <= c->S; ++n)
    fac[n] = n == 1 ? 0.0 : (quantile ? orc_Phi_inv_upper(1.0 / n) : sqrt(2.0 * log((double)n)));
  for (int32_t b = 0; b < c->B; ++b)
    for (int32_t h = 0; h < c->Hq; ++h)
      for (int32_t p = 0; p < c->maxP; ++p) {
        size_t o = ((size_t)b * c->Hq + h) * c->maxP + p;
        if (p >= orc_pages(c, b)) {
          m[o] = s[o] = shat[o] = NAN;
          continue;
        }
        size_t mo = ((size_t)orc_phys(c, b, p) * c->Hkv + h / G) * c->d;
        double sm = 0.0, sv = 0.0;
        for (int32_t j = 0; j < c->d; ++j) {
          double qj = orc_q(c, b, h, j);
          sm += qj * mean[mo + j];
          sv += qj * qj * var[mo + j];
        }
        int32_t n = orc_page_tokens(c, b, p);
        m[o] = scale * sm;
        s[o] = scale * sqrt(sv);
        shat[o] = m[o] + s[o] * fac[n];
      }
  free(fac);
}

/* [NOSA] section 1, pooled page key: key[b][g][p] = RN_f32(max over the G query heads h of g and
 * over the sub-blocks j holding a valid token of sum_i q_hi pool_j[i]), the sum in float64 over i
 * ascending (products of the bf16 or float32 query with float32 means are exact in float64);
 * -inf past the sequence. */
void orc_score_pool(const orc_cache *c, int32_t pb, const float *pool, float *key) {
  int32_t G = c->Hq / c->Hkv, nsb = c->S / pb;
  for (int32_t b = 0; b < c->B; ++b)
    for (int32_t g = 0; g < c->Hkv; ++g)
      for (int32_t p = 0; p < c->maxP; ++p) {
        size_t o = ((size_t)b * c->Hkv + g) * c->maxP + p;
        if (p >= orc_pages(c, b)) {
          key[o] = -INFINITY;
          continue;
        }
        int32_t phys = orc_phys(c, b, p), n = orc_page_tokens(c, b, p);
        double best = -INFINITY;
        for (int32_t sb = 0; sb < nsb && sb * pb < n; ++sb)
          for (int32_t hh = 0; hh < G; ++hh) {
            const float *mv = pool + (((size_t)phys * c->Hkv + g) * nsb + sb) * c->d;
            double u = 0.0;
            for (int32_t i = 0; i < c->d; ++i) u += orc_q(c, b, g * G + hh, i) * (double)mv[i];
            if (u > best) best = u;
          }
        key[o] = (float)best;
      }
}

/* [JSSA] abstract, token-level scoring in the shared subspace: q~_h = RN_f32(P q_h) (float64
 * sum over j), u_h(t) = sum_i q~_h[i] k~_t[i] (float64 sum over i; the f32 x bf16 products
 * are exact), and the KV head's key is RN_f32(max over its G query heads). Output key
 * [B, Hkv, maxP*S] indexed by token position; tokens at or beyond L_b get -inf. */
void orc_score_proj(const orc_cache *c, int32_t r, const float *P, const uint16_t *kproj, float *key) {
  int32_t G = c->Hq / c->Hkv;
  size_t Lmax = (size_t)c->maxP * c->S;
  float *qt = (float *)malloc(sizeof(float) * (size_t)G * r);
  for (int32_t b = 0; b < c->B; ++b)
    for (int32_t g = 0; g < c->Hkv; ++g) {
      for (int32_t hh = 0; hh < G; ++hh)
        for (int32_t i = 0; i < r; ++i) {
          double acc = 0.0;
          for (int32_t j = 0; j < c->d; ++j) acc += (double)P[(size_t)i * c->d + j] * orc_q(c, b, g * G + hh, j);
          qt[hh * r + i] = (float)acc;
        }
      int64_t L = orc_len(c, b);
      for (size_t t = 0; t < Lmax; ++t) {
        float *out = &key[((size_t)b * c->Hkv + g) * Lmax + t];
        if ((int64_t)t >= L) {
          *out = -INFINITY;
          continue;
        }
        int32_t phys = orc_phys(c, b, (int32_t)(t / c->S));
        const uint16_t *kr = &kproj[(((size_t)phys * c->Hkv + g) * c->S + t % c->S) * r];
        double best = -INFINITY;
        for (int32_t hh = 0; hh < G; ++hh) {
          double u = 0.0;
          for (int32_t i = 0; i < r; ++i) u += (double)qt[hh * r + i] * orc_decode(kr, (size_t)i, ORC_BF16);
          if (u > best) best = u;
        }
        *out = (float)best;
      }
    }
  free(qt);
}

/* [SOCKET] Methodology, soft LSH step 2 (decode): the query does not take one bucket per table but
 * a probability distribution over all of them, a softmax with temperature tau of a soft hash
 * score built from its projections on the table's hyperplanes. Reading: z_i = w_{l,i}.q / ||q||
 * (float64 sums over j ascending; z = 0 when q = 0), and bucket beta, with sign vector s
 * (s_i = +1 where bit i of beta is set, else -1), gets
 *   p_l(beta) = exp(<s, z>/tau) / sum over the 2^P sign vectors s' of exp(<s', z>/tau).
 * The normaliser factorises over the bits, so p_l(beta) = prod_i sigma(2 s_i z_i / tau) with
 * sigma(x) = 1 / (1 + exp(-x)); that product form is what is computed (bits ascending, the
 * argument formed as (+-2 z_i) / tau). The mass is kept in fixed point, T = p * 2^24 rounded to
 * the nearest integer (ties to even), so that the sums of step 3 are exact. tau is used as given.
 * Output tab [B, Hq, L, 2^P] uint32. */
void orc_lsh_tables(const orc_cache *c, int32_t L, int32_t P, const float *planes, double tau, uint32_t *tab) {
  int32_t nb = 1 << P;
  double *sp = (double *)malloc(sizeof(double) * (size_t)P), *sn = (double *)malloc(sizeof(double) * (size_t)P);
  for (int32_t b = 0; b < c->B; ++b)
    for (int32_t h = 0; h < c->Hq; ++h) {
      double ss = 0.0;
      for (int32_t j = 0; j < c->d; ++j) ss += orc_q(c, b, h, j) * orc_q(c, b, h, j);
      double nq = sqrt(ss);
      for (int32_t l = 0; l < L; ++l) {
        for (int32_t i = 0; i < P; ++i) {
          const float *w = planes + ((size_t)l * P + i) * c->d;
          double dot = 0.0;
          for (int32_t j = 0; j < c->d; ++j) dot += (double)w[j] * orc_q(c, b, h, j);
          double z = nq > 0.0 ? dot / nq : 0.0;
          sp[i] = 1.0 / (1.0 + exp(-((2.0 * z) / tau)));
          sn[i] = 1.0 / (1.0 + exp(-((-2.0 * z) / tau)));
        }
        uint32_t *out = tab + (((size_t)b * c->Hq + h) * L + l) * nb;
        for (int32_t beta = 0; beta < nb; ++beta) {
          double pr = 1.0;
          for (int32_t i = 0; i < P; ++i) pr *= (beta >> i) & 1 ? sp[i] : sn[i];
          out[beta] = (uint32_t)rint(ldexp(pr, 24));
        }
      }
    }
  free(sp);
  free(sn);
}

/* [SOCKET] Methodology, soft LSH step 3: a key's score gathers the probability mass the query puts
 * on the key's own bucket over all L tables, weighted by the norm of the key's value vector.
 * Reading for GQA (one selection per KV head): the largest of the G query heads' sums.
 *   key(t) = RN_f32(||v_t|| * (max_h sum_l T_{h,l}[bucket_l(t)]) * 2^-24),
 * the integer sums exact, the product one float64 multiplication. Output key [B, Hkv, maxP*S];
 * tokens at or beyond L_b get -inf. */
void orc_score_lsh(const orc_cache *c, int32_t L, int32_t P, const uint8_t *bucket, const float *vnorm,
                   const uint32_t *tab, float *key) {
  int32_t G = c->Hq / c->Hkv, nb = 1 << P;
  size_t Lmax = (size_t)c->maxP * c->S;
  for (int32_t b = 0; b < c->B; ++b)
    for (int32_t g = 0; g < c->Hkv; ++g) {
      int64_t len = orc_len(c, b);
      for (size_t t = 0; t < Lmax; ++t) {
        float *out = &key[((size_t)b * c->Hkv + g) * Lmax + t];
        if ((int64_t)t >= len) {
          *out = -INFINITY;
          continue;
        }
        int32_t phys = orc_phys(c, b, (int32_t)(t / c->S));
        size_t row = ((size_t)phys * c->Hkv + g) * c->S + t % c->S;
        uint64_t best = 0;
        for (int32_t hh = 0; hh < G; ++hh) {
          const uint32_t *th = tab + ((size_t)b * c->Hq + g * G + hh) * L * nb;
          uint64_t sum = 0;
          for (int32_t l = 0; l < L; ++l) sum += th[(size_t)l * nb + bucket[row * L + l]];
          if (sum > best) best = sum;
        }
        *out = (float)((double)vnorm[row] * ldexp((double)best, -24));
      }
    }
}

/* ------------------------------------------------------------------ selection */

typedef struct {
  float key;
  int32_t idx;
} orc_ki;

/* order: key descending, then index ascending (ties go to the lower index) */
static int orc_cmp_desc(const void *a, const void *b) {
  const orc_ki *x = (const orc_ki *)a, *y = (const orc_ki *)b;
  if (x->key > y->key) return -1;
  if (x->key < y->key) return 1;
  return (x->idx > y->idx) - (x->idx < y->idx);
}

static int orc_cmp_i32(const void *a, const void *b) {
  int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
  return (x > y) - (x < y);
}

/* [EKV] s2.B policy 1 (fixed budget: the k pages with the largest bound) and [SOCKET]
 * Methodology step 4 / [JSSA] (top-k tokens per KV head): brute force. Sort all n candidates
 * by (key desc, index asc), keep the first min(k, n) and emit them in ascending index order.
 * Returns the number emitted. */
int32_t orc_select_topk(const float *key, int32_t n, int32_t k, int32_t *out) {
  if (n <= 0 || k <= 0) return 0;
  orc_ki *a = (orc_ki *)malloc(sizeof(orc_ki) * (size_t)n);
  for (int32_t i = 0; i < n; ++i) {
    a[i].key = key[i];
    a[i].idx = i;
  }
  qsort(a, (size_t)n, sizeof(orc_ki), orc_cmp_desc);
  int32_t cnt = k < n ? k : n;
  for (int32_t i = 0; i < cnt; ++i) out[i] = a[i].idx;
  qsort(out, (size_t)cnt, sizeof(int32_t), orc_cmp_i32);
  free(a);
  return cnt;
}

/* Budget policy: keep ceil(pct * P_b / 100) pages (at least one page when P_b > 0). */
int32_t orc_budget_k(int32_t P_b, int32_t pct) {
  if (P_b <= 0) return 0;
  int64_t k = ((int64_t)pct * P_b + 99) / 100;
  return (int32_t)(k < 1 ? 1 : k);
}

/* Standard normal cdf and pdf from libm's erfc and exp. */
static double orc_Phi(double a) { return 0.5 * erfc(-a / sqrt(2.0)); }
static double orc_phi(double a) { return exp(-0.5 * a * a) / sqrt(2.0 * acos(-1.0)); }

/* I_k(a) = integral over u >= 0 of u^k phi(u - a) du, the k-th truncated power moment of a unit
 * Gaussian shifted by a: E[(Z + a)_+^k] for Z ~ N(0, 1). The integrand is below 1e-40 of its peak
 * outside [max(0, a - 14), max(a, 0) + 14] (u^k grows with u), and that interval is integrated by
 * the tanh-sinh (double-exponential) rule of Takahasi and Mori (1974): u = c + w tanh(x) with
 * x = (pi/2) sinh t, du = w (pi/2) cosh t / cosh^2 x dt, and the trapezoid rule in t over
 * [-4, 4] (beyond, the weights are below 1e-60 of the interval), its step halved until two
 * successive levels agree to 1e-15 relative (at least five levels). The change of variable
 * clusters the nodes at both ends, which absorbs the u^k behaviour at u = 0 for fractional k.
 * Points near an end are placed by their distance to it, 2 w / (1 + e^(2|x|)), which keeps them
 * accurate where tanh(x) rounds to +-1. */
static double orc_ts_term(double a, double k, double l, double r, double t) {
  const double hw = 0.5 * (r - l), x = 0.5 * acos(-1.0) * sinh(t);
  if (fabs(x) > 350.0) return 0.0;
  const double d = 2.0 * hw / (1.0 + exp(2.0 * fabs(x)));   /* distance from the nearer end */
  const double u = x > 0.0 ? r - d : l + d;
  const double ch = cosh(x);
  const double wt = hw * 0.5 * acos(-1.0) * cosh(t) / (ch * ch);
  return wt * pow(u, k) * exp(-0.5 * (u - a) * (u - a));
}

static double orc_tanh_sinh(double a, double k, double l, double r) {
  const double T = 4.0;
  double h = 0.5, sum = orc_ts_term(a, k, l, r, 0.0);
  for (double t = h; t <= T; t += h) sum += orc_ts_term(a, k, l, r, t) + orc_ts_term(a, k, l, r, -t);
  double prev = h * sum;
  for (int level = 1; level <= 14; ++level) {
    h *= 0.5;   /* the new nodes are the odd multiples of the halved step */
    for (double t = h; t <= T; t += 2.0 * h) sum += orc_ts_term(a, k, l, r, t) + orc_ts_term(a, k, l, r, -t);
    const double cur = h * sum;
    if (level >= 5 && fabs(cur - prev) <= 1e-15 * fabs(cur)) return cur;
    prev = cur;
  }
  return prev;
}

double orc_trunc_power_moment(double a, double k) {
  if (a < -40.0) return 0.0;
  const double L0 = a > 14.0 ? a - 14.0 : 0.0, U = (a > 0.0 ? a : 0.0) + 14.0;
  return orc_tanh_sinh(a, k, L0, U) / sqrt(2.0 * acos(-1.0));
}

/* E[(X - tau)_+^(1/(alpha-1))] for X ~ N(mu_x, sd_x^2). With mu = mu_x - tau and a = mu / sd:
 * alpha = 2 (first partial moment) gives mu Phi(a) + sd phi(a); alpha = 1.5 (second) gives
 * (mu^2 + sd^2) Phi(a) + mu sd phi(a); any other alpha in (1, 2) gives sd^k I_k(a) with
 * k = 1/(alpha-1) by quadrature (orc_trunc_power_moment). A zero sd gives the point-mass value
 * mu_+^k. orc_gauss_partial_moment_quad always takes the quadrature (used to pin it). */
double orc_gauss_partial_moment_quad(double mu_x, double sd_x, double tau, double alpha) {
  double mu = mu_x - tau, k = 1.0 / (alpha - 1.0);
  if (sd_x == 0.0) return mu > 0 ? pow(mu, k) : 0.0;
  return pow(sd_x, k) * orc_trunc_power_moment(mu / sd_x, k);
}

double orc_gauss_partial_moment(double mu_x, double sd_x, double tau, double alpha) {
  double mu = mu_x - tau;
  if (alpha != 2.0 && alpha != 1.5) return orc_gauss_partial_moment_quad(mu_x, sd_x, tau, alpha);
  if (sd_x == 0.0) {
    double pos = mu > 0 ? mu : 0.0;
    return alpha == 2.0 ? pos : pos * pos;
  }
  double a = mu / sd_x;
  if (alpha == 2.0) return mu * orc_Phi(a) + sd_x * orc_phi(a);
  return (mu * mu + sd_x * sd_x) * orc_Phi(a) + mu * sd_x * orc_phi(a);
}

/* [EKV] s2.B policy 2, the "approximate normalization equation". Reading: each page's token
 * scores are n_p draws of Z ~ N(m_p, s_p^2); the entmax normalizer sum_t p_t = 1 is replaced by
 * its expectation, F(tau) = sum_p n_p E[((alpha-1) Z - tau)_+^(1/(alpha-1))] - 1 = 0, and
 * tau_hat is its root. F is continuous and non-increasing in tau. Bracket: lo =
 * (alpha-1) max_p m_p - 1 gives F(lo) >= 0 (Jensen: E[f(X)] >= f(E X) for the convex
 * f(x) = (x - tau)_+^(1/(alpha-1)), and the top page alone contributes >= 1); hi is pushed
 * right by doubling until F(hi) < 0; then bisection until hi - lo <= 2^-40 max(1, |lo|).
 * Only pages with n_p > 0 enter; alpha in (1, 2]. Returns tau_hat (NaN if P = 0). */
static double orc_F(const double *m, const double *s, const int32_t *n, int32_t P, double alpha, double tau) {
  double f = -1.0;
  for (int32_t p = 0; p < P; ++p)
    if (n[p] > 0) f += n[p] * orc_gauss_partial_moment((alpha - 1.0) * m[p], (alpha - 1.0) * s[p], tau, alpha);
  return f;
}

double orc_tau_hat(const double *m, const double *s, const int32_t *n, int32_t P, double alpha) {
  double mmax = -INFINITY;
  for (int32_t p = 0; p < P; ++p)
    if (n[p] > 0 && m[p] > mmax) mmax = m[p];
  if (mmax == -INFINITY) return NAN;
  double lo = (alpha - 1.0) * mmax - 1.0, hi = lo + 1.0;
  while (orc_F(m, s, n, P, alpha, hi) >= 0.0) hi = lo + 2.0 * (hi - lo);
  while (hi - lo > 0x1p-40 * fmax(1.0, fabs(lo))) {
    double mid = 0.5 * (lo + hi);
    if (orc_F(m, s, n, P, alpha, mid) >= 0.0)
      lo = mid;
    else
      hi = mid;
  }
  return 0.5 * (lo + hi);
}

/* [EKV] s2.B policy 2, selection: keep page p for KV head g iff some query head h of g has
 * (alpha-1) shat_h(p) > tau_hat_h - delta (reading: delta is in tau units and lowers the bar,
 * strict >). shat and tau_hat are given for the G heads: shat[G][P], tau_hat[G].
 * Emits ascending page indices; returns the count. */
int32_t orc_select_thresh(const double *shat, const double *tau_hat, int32_t G, int32_t P, double alpha,
                          double delta, int32_t *out) {
  int32_t cnt = 0;
  for (int32_t p = 0; p < P; ++p) {
    int keep = 0;
    for (int32_t hh = 0; hh < G; ++hh)
      if ((alpha - 1.0) * shat[(size_t)hh * P + p] > tau_hat[hh] - delta) keep = 1;
    if (keep) out[cnt++] = p;
  }
  return cnt;
}

/* The threshold policy with the box bound as the page's estimated maximum (reading: the box
 * key of a KV head is max over its G query heads of the unscaled bound U_h(p), so the test
 * compares it with the lowest threshold of the group): keep page p iff
 * (alpha-1) scale key[p] > min_h tau_hat_h - delta. Any page the per-head test
 * (alpha-1) scale U_h(p) > tau_hat_h - delta keeps is kept. Emits ascending indices. */
int32_t orc_select_thresh_box(const double *key, const double *tau_hat, int32_t G, int32_t P, double scale,
                              double alpha, double delta, int32_t *out) {
  double tmin = INFINITY;
  for (int32_t hh = 0; hh < G; ++hh)
    if (tau_hat[hh] < tmin) tmin = tau_hat[hh];
  int32_t cnt = 0;
  for (int32_t p = 0; p < P; ++p)
    if ((alpha - 1.0) * scale * key[p] > tmin - delta) out[cnt++] = p;
  return cnt;
}

/* ------------------------------------------------------------------ entmax */

/* softmax: p_t = exp(z_t - max z) / sum_u exp(z_u - max z). */
void orc_softmax(const double *z, int32_t n, double *p) {
  double mx = -INFINITY, sum = 0.0;
  for (int32_t t = 0; t < n; ++t)
    if (z[t] > mx) mx = z[t];
  for (int32_t t = 0; t < n; ++t) sum += exp(z[t] - mx);
  for (int32_t t = 0; t < n; ++t) p[t] = exp(z[t] - mx) / sum;
}

static int orc_cmp_dbl_desc(const void *a, const void *b) {
  double x = *(const double *)a, y = *(const double *)b;
  return (x < y) - (x > y);
}

/* sparsemax (alpha = 2), sort-based (Martins & Astudillo 2016): with z sorted descending,
 * k* = max{k : 1 + k z_(k) > sum_{i<=k} z_(i)}, tau = (sum_{i<=k*} z_(i) - 1) / k*,
 * p = (z - tau)_+. Returns tau. */
double orc_sparsemax(const double *z, int32_t n, double *p) {
  double *zs = (double *)malloc(sizeof(double) * (size_t)n);
  memcpy(zs, z, sizeof(double) * (size_t)n);
  qsort(zs, (size_t)n, sizeof(double), orc_cmp_dbl_desc);
  double cum = 0.0, tau = 0.0;
  for (int32_t k = 1; k <= n; ++k) {
    cum += zs[k - 1];
    if (1.0 + k * zs[k - 1] > cum) tau = (cum - 1.0) / k;
  }
  for (int32_t t = 0; t < n; ++t) p[t] = z[t] > tau ? z[t] - tau : 0.0;
  free(zs);
  return tau;
}

/* 1.5-entmax, exact sort-based (Peters, Niculae & Martins 2019): with z' = z / 2 sorted
 * descending, for each k: M_k = mean of the top k, Q_k = mean of their squares,
 * delta_k = (1 - k (Q_k - M_k^2)) / k, tau_k = M_k - sqrt(delta_k) (when delta_k >= 0);
 * k* = the largest k with z'_(k) > tau_k; p = (z' - tau_k*)_+^2. Returns tau in the units of
 * (alpha-1) z, i.e. z' units. */
double orc_entmax15(const double *z, int32_t n, double *p) {
  double *zs = (double *)malloc(sizeof(double) * (size_t)n);
  for (int32_t t = 0; t < n; ++t) zs[t] = 0.5 * z[t];
  qsort(zs, (size_t)n, sizeof(double), orc_cmp_dbl_desc);
  double s1 = 0.0, s2 = 0.0, tau = zs[0] - 1.0;
  for (int32_t k = 1; k <= n; ++k) {
    s1 += zs[k - 1];
    s2 += zs[k - 1] * zs[k - 1];
    double M = s1 / k, Q = s2 / k;
    double dk = (1.0 - k * (Q - M * M)) / k;
    if (dk < 0.0) continue;
    double tk = M - sqrt(dk);
    if (zs[k - 1] > tk) tau = tk;
  }
  for (int32_t t = 0; t < n; ++t) {
    double x = 0.5 * z[t] - tau;
    p[t] = x > 0 ? x * x : 0.0;
  }
  free(zs);
  return tau;
}

/* alpha-entmax for any alpha in (1, 2] by bisection on tau in
 * [(alpha-1) max z - 1, (alpha-1) max z - n^(1-alpha)] (at the left end the top entry alone
 * has mass 1; at the right end every entry has mass <= 1/n), until the interval stops
 * shrinking. p = [(alpha-1) z - tau]_+^(1/(alpha-1)), not renormalized. Returns tau. */
double orc_entmax_bisect(const double *z, int32_t n, double alpha, double *p) {
  double am1 = alpha - 1.0, mx = -INFINITY;
  for (int32_t t = 0; t < n; ++t)
    if (z[t] > mx) mx = z[t];
  double lo = am1 * mx - 1.0, hi = am1 * mx - pow((double)n, -am1);
  for (int it = 0; it < 2000; ++it) {
    double mid = 0.5 * (lo + hi);
    if (mid <= lo || mid >= hi) break;
    double sum = 0.0;
    for (int32_t t = 0; t < n; ++t) {
      double x = am1 * z[t] - mid;
      if (x > 0) sum += pow(x, 1.0 / am1);
    }
    if (sum >= 1.0)
      lo = mid;
    else
      hi = mid;
  }
  double tau = 0.5 * (lo + hi);
  for (int32_t t = 0; t < n; ++t) {
    double x = am1 * z[t] - tau;
    p[t] = x > 0 ? pow(x, 1.0 / am1) : 0.0;
  }
  return tau;
}

/* [EKV] s2.C: alpha = 1 is softmax, alpha = 2 sparsemax, alpha = 1.5 the exact sort-based
 * 1.5-entmax, any other alpha in (1, 2) bisection. */
double orc_entmax(const double *z, int32_t n, double alpha, double *p) {
  if (n <= 0) return NAN;
  if (alpha == 1.0) {
    orc_softmax(z, n, p);
    return NAN;
  }
  if (alpha == 2.0) return orc_sparsemax(z, n, p);
  if (alpha == 1.5) return orc_entmax15(z, n, p);
  return orc_entmax_bisect(z, n, alpha, p);
}

/* ------------------------------------------------------------------ attention */

/* Token positions of a unit's selection: granularity 0 means sel holds logical page indices
 * (each expands to its valid tokens, ascending); granularity 1 means sel holds token
 * positions. Entries outside the sequence are skipped. Returns the token count written. */
static int64_t orc_tokens(const orc_cache *c, int32_t b, const int32_t *sel, int32_t count, int32_t gran,
                          int64_t *tok) {
  int64_t n = 0, L = orc_len(c, b);
  for (int32_t i = 0; i < count; ++i) {
    if (gran == 1) {
      if (sel[i] >= 0 && sel[i] < L) tok[n++] = sel[i];
    } else if (sel[i] >= 0 && sel[i] < orc_pages(c, b)) {
      int32_t np = orc_page_tokens(c, b, sel[i]);
      for (int32_t t = 0; t < np; ++t) tok[n++] = (int64_t)sel[i] * c->S + t;
    }
  }
  return n;
}

/* Decode row t (token position) of KV head g of sequence b from base (k or v) into row[d]. */
static void orc_row(const orc_cache *c, const void *base, int32_t b, int32_t g, int64_t t, double *row) {
  size_t at = orc_kv_at(c, orc_phys(c, b, (int32_t)(t / c->S)), g, (int32_t)(t % c->S), 0);
  for (int32_t j = 0; j < c->d; ++j) row[j] = orc_decode(base, at + (size_t)j, c->dtype);
}

/* [EKV] s2.C: attention weights over the selected KV only, for query head h:
 * z_t = scale * sum_j q_hj k_tj (float64, j ascending), p = entmax_alpha(z),
 * out = sum_t p_t v_t (t ascending). p_out (optional, length = token count) receives the
 * weights, tok_out (optional) the token positions. An empty selection gives a zero output.
 * Returns the token count. */
int64_t orc_attend_head(const orc_cache *c, int32_t b, int32_t h, const int32_t *sel, int32_t count,
                        int32_t gran, double alpha, double scale, double *out, double *p_out, int64_t *tok_out) {
  int32_t g = h / (c->Hq / c->Hkv);
  int64_t cap = gran == 1 ? (int64_t)count : (int64_t)count * c->S;
  int64_t *tok = (int64_t *)malloc(sizeof(int64_t) * (size_t)(cap > 0 ? cap : 1));
  int64_t n = orc_tokens(c, b, sel, count, gran, tok);
  double *qh = (double *)malloc(sizeof(double) * (size_t)c->d);
  double *row = (double *)malloc(sizeof(double) * (size_t)c->d);
  for (int32_t j = 0; j < c->d; ++j) {
    qh[j] = orc_q(c, b, h, j);
    out[j] = 0.0;
  }
  if (n > 0) {
    double *z = (double *)malloc(sizeof(double) * (size_t)n);
    double *p = (double *)malloc(sizeof(double) * (size_t)n);
    for (int64_t i = 0; i < n; ++i) {
      orc_row(c, c->k, b, g, tok[i], row);
      double acc = 0.0;
      for (int32_t j = 0; j < c->d; ++j) acc += qh[j] * row[j];
      z[i] = scale * acc;
    }
    orc_entmax(z, (int32_t)n, alpha, p);
    for (int64_t i = 0; i < n; ++i)
      if (p[i] != 0.0) {
        orc_row(c, c->v, b, g, tok[i], row);
        for (int32_t j = 0; j < c->d; ++j) out[j] += p[i] * row[j];
      }
    if (p_out) memcpy(p_out, p, sizeof(double) * (size_t)n);
    free(z);
    free(p);
  }
  if (tok_out) memcpy(tok_out, tok, sizeof(int64_t) * (size_t)n);
  free(qh);
  free(row);
  free(tok);
  return n;
}

/* Full-cache reference: the same computation over every valid token of sequence b. */
int64_t orc_attend_full_head(const orc_cache *c, int32_t b, int32_t h, double alpha, double scale, double *out,
                             double *p_out) {
  int64_t L = orc_len(c, b);
  int32_t *all = (int32_t *)malloc(sizeof(int32_t) * (size_t)(L > 0 ? L : 1));
  for (int64_t t = 0; t < L; ++t) all[t] = (int32_t)t;
  int64_t n = orc_attend_head(c, b, h, all, (int32_t)L, 1, alpha, scale, out, p_out, NULL);
  free(all);
  return n;
}
