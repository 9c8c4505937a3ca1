// C ABI of libskv: synchronous host-side validation, workspace planning and kernel dispatch.
// Nothing is enqueued unless every argument checks out. See include/skv.h for the contract.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstdint>
#include <cstring>
#include <vector>

#include "launch.hpp"
#include "skv.h"

namespace {

using skv::CacheView;

constexpr size_t kAlign = 256;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

skv_status check_cache(const skv_cache *c) {
  if (!c || !c->k || !c->v || !c->block_table || !c->seq_lens) return SKV_ERR_INVALID_ARG;
  if (c->batch < 1 || c->num_q_heads < 1 || c->num_kv_heads < 1 || c->head_dim < 1 || c->page_size < 1 ||
      c->max_pages < 1 || c->num_phys_pages < 1)
    return SKV_ERR_INVALID_ARG;
  if (c->num_q_heads % c->num_kv_heads) return SKV_ERR_INVALID_ARG;
  if (c->dtype != SKV_DTYPE_F32 && c->dtype != SKV_DTYPE_BF16) return SKV_ERR_INVALID_ARG;
  const int G = c->num_q_heads / c->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return SKV_ERR_UNSUPPORTED;
  if (c->head_dim != 64 && c->head_dim != 128) return SKV_ERR_UNSUPPORTED;
  if (c->page_size > 1024) return SKV_ERR_UNSUPPORTED;
  if ((int64_t)c->max_pages * c->page_size > INT32_MAX) return SKV_ERR_UNSUPPORTED;
  if ((int64_t)c->batch * c->num_kv_heads > 65535 || c->batch > 65535) return SKV_ERR_UNSUPPORTED;
  if (!aligned(c->k, 16) || !aligned(c->v, 16)) return SKV_ERR_INVALID_ARG;
  return SKV_OK;
}

CacheView view(const skv_cache *c) {
  CacheView v;
  v.B = c->batch;
  v.Hq = c->num_q_heads;
  v.Hkv = c->num_kv_heads;
  v.D = c->head_dim;
  v.S = c->page_size;
  v.maxP = c->max_pages;
  v.Nphys = c->num_phys_pages;
  v.G = c->num_q_heads / c->num_kv_heads;
  v.k = c->k;
  v.v = c->v;
  v.bt = c->block_table;
  v.lens = c->seq_lens;
  return v;
}

skv_status hip_status(hipError_t e) { return e == hipSuccess ? SKV_OK : SKV_ERR_HIP; }

skv::KernelEvents events(void *begin, void *end) {
  skv::KernelEvents e;
  e.begin = static_cast<hipEvent_t>(begin);
  e.end = static_cast<hipEvent_t>(end);
  return e;
}

bool rank_ok(int r) { return r == 16 || r == 32 || r == 64; }

bool lsh_ok(int L, int P) { return (L == 16 || L == 32 || L == 48 || L == 64) && P >= 1 && P <= 8; }

// Workspace of a scoring call. LSH: the bucket masses of every unit, G * L * 2^P uint32 each
// (`lsh_entries` per unit; the size query, which does not see L and P, assumes the maximum).
size_t score_ws(const skv_cache *c, int kind, int r, size_t lsh_entries = skv::kLshMaxEntries) {
  if (kind == SKV_SCORE_GAUSS || kind == SKV_SCORE_GAUSS_Q || kind == SKV_SCORE_POOL) return 0;   // q staged by the scorer
  if (kind == SKV_SCORE_BOX && c->num_q_heads <= 4 * c->num_kv_heads) return 0;                    // likewise at G <= 4
  if (kind == SKV_SCORE_PROJ) return round_up(sizeof(double) * (size_t)c->batch * c->num_q_heads * r);
  if (kind == SKV_SCORE_LSH) return round_up(sizeof(uint32_t) * (size_t)c->batch * c->num_kv_heads * lsh_entries);
  return round_up(sizeof(double) * 2 * (size_t)c->batch * c->num_q_heads * c->head_dim);
}

// Split-K plan of the attention call.
struct AttnPlan {
  int spi = 1, nsplit = 1, rps = 1;
  size_t part = 0, cand = 0, cnt = 0, mx = 0, total = 0;
};

skv_status attn_plan(const skv_cache *c, const skv_attn_params *p, int cap, AttnPlan *out) {
  const int G = c->num_q_heads / c->num_kv_heads;
  const int rows_per_item = p->granularity ? 1 : c->page_size;
  const bool entmax = p->alpha != 1.0f;
  const int64_t U = (int64_t)c->batch * c->num_kv_heads;
  const int rmax = 1024;   // rows per partition (entmax: at most 40 KiB of logits and offsets at G = 8)
  int64_t spi = p->split;
  if (spi <= 0) {
    spi = ((int64_t)cap * U + 1023) / 1024;   // about 1024 partitions in total
    spi = std::max<int64_t>(1, std::min<int64_t>(spi, std::max(1, rmax / rows_per_item)));
  }
  spi = std::min<int64_t>(spi, cap);
  spi = std::max<int64_t>(spi, (cap + 2047) / 2048);   // at most 2048 partitions per unit
  const int64_t nsplit = (cap + spi - 1) / spi;
  const int64_t rps = spi * rows_per_item;
  // LDS of a partition: logits (entmax) and row offsets
  if (entmax && (int64_t)G * 4 * ((rps + 3) / 4) * 4 + rps * 8 + 8 > 65536) return SKV_ERR_UNSUPPORTED;
  if (!entmax && rps * 8 > 32768) return SKV_ERR_UNSUPPORTED;
  out->spi = (int)spi;
  out->nsplit = (int)nsplit;
  out->rps = (int)rps;
  if (!entmax) {
    out->part = nsplit > 1 ? round_up(sizeof(float) * (size_t)U * nsplit * G * (c->head_dim + 2)) : 0;
  } else {
    out->cand = round_up(sizeof(float) * 2 * (size_t)U * G * nsplit * rps);
    out->cnt = round_up(sizeof(int32_t) * (size_t)U * G * nsplit);
    out->mx = round_up(sizeof(float) * (size_t)U * G * nsplit);
  }
  out->total = out->part + out->cand + out->cnt + out->mx;
  return SKV_OK;
}

skv_status check_attn_params(const skv_attn_params *p) {
  if (!p) return SKV_ERR_INVALID_ARG;
  if (!std::isfinite(p->alpha) || !(p->alpha == 1.0f || (p->alpha > 1.0f && p->alpha <= 2.0f)))
    return SKV_ERR_INVALID_ARG;
  if (!std::isfinite(p->sm_scale) || !(p->sm_scale > 0.0f)) return SKV_ERR_INVALID_ARG;
  if (p->granularity != 0 && p->granularity != 1) return SKV_ERR_INVALID_ARG;
  if (p->split < 0) return SKV_ERR_INVALID_ARG;
  return SKV_OK;
}

// ---------------------------------------------------------------- SKV_DEBUG checks
// With SKV_DEBUG set (to anything but "0"), a call first synchronises its stream, copies the
// device-side inputs it indexes with to the host and checks them; an out-of-range entry returns
// SKV_ERR_INVALID_ARG before anything is launched. Off by default: it costs a synchronisation and
// host copies per call.
bool debug_on() {
  const char *e = std::getenv("SKV_DEBUG");
  return e && *e && std::strcmp(e, "0") != 0;
}

skv_status debug_fetch(const int32_t *src, size_t n, std::vector<int32_t> &dst, hipStream_t s) {
  dst.resize(n);
  if (n == 0) return SKV_OK;
  if (hipStreamSynchronize(s) != hipSuccess ||
      hipMemcpy(dst.data(), src, n * sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess) {
    (void)hipGetLastError();
    return SKV_ERR_HIP;
  }
  return SKV_OK;
}

// seq_lens clamped as the kernels clamp them; block_table entries of the pages in use within
// [0, num_phys_pages). Writes the clamped lengths.
skv_status debug_check_cache(const skv_cache *c, hipStream_t s, std::vector<int64_t> &lens) {
  std::vector<int32_t> raw, bt;
  skv_status st = debug_fetch(c->seq_lens, (size_t)c->batch, raw, s);
  if (st == SKV_OK) st = debug_fetch(c->block_table, (size_t)c->batch * c->max_pages, bt, s);
  if (st != SKV_OK) return st;
  const int64_t cap = (int64_t)c->max_pages * c->page_size;
  lens.resize(c->batch);
  for (int b = 0; b < c->batch; ++b) {
    lens[b] = std::min<int64_t>(std::max<int64_t>(raw[b], 0), cap);
    const int64_t P = (lens[b] + c->page_size - 1) / c->page_size;
    for (int64_t p = 0; p < P; ++p) {
      const int32_t x = bt[(size_t)b * c->max_pages + p];
      if (x < 0 || x >= c->num_phys_pages) return SKV_ERR_INVALID_ARG;
    }
  }
  return SKV_OK;
}

skv_status debug_check_cache(const skv_cache *c, hipStream_t s) {
  std::vector<int64_t> lens;
  return debug_check_cache(c, s, lens);
}

// A selection as skv_select_pages writes it: counts within [0, cap], entries inside the sequence
// (logical pages below P_b, or tokens below L_b) and strictly ascending.
skv_status debug_check_selection(const skv_cache *c, const int32_t *sel_idx, const int32_t *sel_count, int cap,
                                 int gran, hipStream_t s) {
  std::vector<int64_t> lens;
  skv_status st = debug_check_cache(c, s, lens);
  if (st != SKV_OK) return st;
  const size_t U = (size_t)c->batch * c->num_kv_heads;
  std::vector<int32_t> cnt, idx;
  if ((st = debug_fetch(sel_count, U, cnt, s)) != SKV_OK || (st = debug_fetch(sel_idx, U * cap, idx, s)) != SKV_OK)
    return st;
  for (size_t u = 0; u < U; ++u) {
    const int64_t L = lens[u / c->num_kv_heads];
    const int64_t limit = gran ? L : (L + c->page_size - 1) / c->page_size;
    if (cnt[u] < 0 || cnt[u] > cap) return SKV_ERR_INVALID_ARG;
    for (int i = 0; i < cnt[u]; ++i) {
      const int32_t e = idx[u * cap + i];
      if (e < 0 || e >= limit || (i > 0 && e <= idx[u * cap + i - 1])) return SKV_ERR_INVALID_ARG;
    }
  }
  return SKV_OK;
}

int budget_cap(int maxP, int pct) {
  const int64_t k = ((int64_t)pct * maxP + 99) / 100;
  return (int)std::max<int64_t>(1, k);
}

}  // namespace

extern "C" {

const char *skv_status_str(skv_status s) {
  // A C caller may pass any int; in C++ loading it as the enum type would be undefined, so the
  // argument's representation is read as an integer.
  int v;
  static_assert(sizeof v == sizeof s, "skv_status is int-sized");
  std::memcpy(&v, &s, sizeof v);
  switch (v) {
    case SKV_OK: return "SKV_OK";
    case SKV_ERR_INVALID_ARG: return "SKV_ERR_INVALID_ARG";
    case SKV_ERR_UNSUPPORTED: return "SKV_ERR_UNSUPPORTED";
    case SKV_ERR_CAPACITY: return "SKV_ERR_CAPACITY";
    case SKV_ERR_WORKSPACE: return "SKV_ERR_WORKSPACE";
    case SKV_ERR_HIP: return "SKV_ERR_HIP";
  }
  return "SKV_ERR_UNKNOWN";
}

skv_status skv_workspace_bytes(const skv_cache *c, int32_t op, const void *params, int32_t cap, size_t *bytes) {
  if (!bytes || !params) return SKV_ERR_INVALID_ARG;
  skv_status st = check_cache(c);
  if (st != SKV_OK) return st;
  if (op == SKV_OP_SCORE) {
    const int kind = *static_cast<const int32_t *>(params);
    if (kind < SKV_SCORE_BOX || kind > SKV_SCORE_LSH) return SKV_ERR_INVALID_ARG;
    *bytes = score_ws(c, kind, 64);
    return SKV_OK;
  }
  if (op == SKV_OP_SELECT) {   // token top-k over dense keys: the candidate segments of the many-block path
    const skv_select_params *p = static_cast<const skv_select_params *>(params);
    *bytes = 0;
    if (p->policy == SKV_SEL_TOKEN_TOPK) {
      const skv::CandLayout lay(c->batch, c->num_q_heads, c->num_kv_heads, c->max_pages * c->page_size, 64);
      if (lay.nb <= 8192) *bytes = lay.total;
    }
    return SKV_OK;
  }
  if (op == SKV_OP_CANDIDATES) {
    if (*static_cast<const int32_t *>(params) < 1) return SKV_ERR_INVALID_ARG;
    const skv::CandLayout lay(c->batch, c->num_q_heads, c->num_kv_heads, c->max_pages * c->page_size, 64);
    if (lay.nb > 8192) return SKV_ERR_UNSUPPORTED;
    *bytes = lay.total;
    return SKV_OK;
  }
  if (op == SKV_OP_ATTN) {
    const skv_attn_params *p = static_cast<const skv_attn_params *>(params);
    if ((st = check_attn_params(p)) != SKV_OK) return st;
    if (cap < 1) return SKV_ERR_INVALID_ARG;
    AttnPlan plan;
    if ((st = attn_plan(c, p, cap, &plan)) != SKV_OK) return st;
    *bytes = plan.total;
    return SKV_OK;
  }
  return SKV_ERR_INVALID_ARG;
}

// Shared by the build and the append: metadata kinds, outputs and the projection's LDS fit.
static skv_status meta_args(const skv_cache *c, const skv_meta *m) {
  skv_status st = check_cache(c);
  if (st != SKV_OK) return st;
  if (!m || m->kinds == 0 ||
      (m->kinds & ~(uint32_t)(SKV_META_BOX | SKV_META_GAUSS | SKV_META_PROJ | SKV_META_POOL | SKV_META_LSH)))
    return SKV_ERR_INVALID_ARG;
  const bool box = m->kinds & SKV_META_BOX, gauss = m->kinds & SKV_META_GAUSS, proj = m->kinds & SKV_META_PROJ;
  if ((box && !m->box) || (gauss && !m->gauss)) return SKV_ERR_INVALID_ARG;
  if (m->kinds & SKV_META_POOL) {
    if (!m->pool || !aligned(m->pool, 16) || m->pool_block < 1 || c->page_size % m->pool_block != 0)
      return SKV_ERR_INVALID_ARG;
  }
  if (m->kinds & SKV_META_LSH) {
    if (!m->lsh_planes || !m->lsh_bucket || !m->vnorm || !aligned(m->lsh_bucket, 16) || !aligned(m->lsh_planes, 16) ||
        !aligned(m->vnorm, 4))
      return SKV_ERR_INVALID_ARG;
    if (!lsh_ok(m->lsh_tables, m->lsh_bits)) return SKV_ERR_UNSUPPORTED;
  }
  if (box && !aligned(m->box, 16)) return SKV_ERR_INVALID_ARG;
  if (gauss && !aligned(m->gauss, 16)) return SKV_ERR_INVALID_ARG;
  if (proj) {
    if (!m->proj || !m->kproj || !aligned(m->kproj, 16)) return SKV_ERR_INVALID_ARG;
    if (!rank_ok(m->proj_rank)) return SKV_ERR_UNSUPPORTED;
  }
  // the row-dot kernels of the projected keys and soft-LSH buckets index token rows in 32 bits
  // (more rows than that would not fit next to K anyway)
  if ((proj || (m->kinds & SKV_META_LSH)) &&
      (uint64_t)c->num_phys_pages * c->num_kv_heads * c->page_size > 0xffffffffull)
    return SKV_ERR_UNSUPPORTED;
  return SKV_OK;
}

static skv_status meta_launch(const skv_cache *c, const skv_meta *m, int tail, void *stream) {
  if (debug_on()) {
    const skv_status st = debug_check_cache(c, static_cast<hipStream_t>(stream));
    if (st != SKV_OK) return st;
  }
  const bool box = m->kinds & SKV_META_BOX, gauss = m->kinds & SKV_META_GAUSS, proj = m->kinds & SKV_META_PROJ;
  const bool pool = m->kinds & SKV_META_POOL;
  (void)hipGetLastError();
  hipError_t e = skv::launch_build_meta(view(c), c->dtype, tail, box ? m->box : nullptr, gauss ? m->gauss : nullptr,
                                        m->proj_rank, proj ? m->proj : nullptr, proj ? m->kproj : nullptr,
                                        m->pool_block, pool ? m->pool : nullptr, static_cast<hipStream_t>(stream));
  if (e == hipSuccess && (m->kinds & SKV_META_LSH))
    e = skv::launch_build_lsh(view(c), c->dtype, tail, m->lsh_tables, m->lsh_bits, m->lsh_planes, m->lsh_bucket,
                              m->vnorm, static_cast<hipStream_t>(stream));
  return hip_status(e);
}

skv_status skv_build_page_meta(const skv_cache *c, const skv_meta *m, void *stream) {
  const skv_status st = meta_args(c, m);
  return st != SKV_OK ? st : meta_launch(c, m, 0, stream);
}

skv_status skv_append_page_meta(const skv_cache *c, const skv_meta *m, int32_t n_new, void *stream) {
  const skv_status st = meta_args(c, m);
  if (st != SKV_OK) return st;
  if (n_new < 1) return SKV_ERR_INVALID_ARG;
  return meta_launch(c, m, n_new, stream);
}

skv_status skv_score_pages(const skv_cache *c, const skv_meta *m, const void *q, int32_t kind, float sm_scale,
                           const skv_scores *out, void *workspace, size_t workspace_bytes, void *stream) {
  skv_status st = check_cache(c);
  if (st != SKV_OK) return st;
  if (!m || !q || !out) return SKV_ERR_INVALID_ARG;
  if (!aligned(q, 16)) return SKV_ERR_INVALID_ARG;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (debug_on() && (st = debug_check_cache(c, s)) != SKV_OK) return st;
  const CacheView v = view(c);
  const skv::KernelEvents ev = events(out->ev_begin, out->ev_end);
  if (kind == SKV_SCORE_BOX) {
    if (!(m->kinds & SKV_META_BOX) || !m->box || !out->key || !aligned(m->box, 16)) return SKV_ERR_INVALID_ARG;
  } else if (kind == SKV_SCORE_POOL) {
    if (!(m->kinds & SKV_META_POOL) || !m->pool || !out->key || !aligned(m->pool, 16) || m->pool_block < 1 ||
        c->page_size % m->pool_block != 0)
      return SKV_ERR_INVALID_ARG;
  } else if (kind == SKV_SCORE_LSH) {
    if (!(m->kinds & SKV_META_LSH) || !m->lsh_planes || !m->lsh_bucket || !m->vnorm || !out->key ||
        !aligned(m->lsh_bucket, 16) || !aligned(m->lsh_planes, 16) || !aligned(m->vnorm, 4))
      return SKV_ERR_INVALID_ARG;
    if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f)) return SKV_ERR_INVALID_ARG;   // the temperature
    if (!lsh_ok(m->lsh_tables, m->lsh_bits) ||
        ((size_t)c->num_q_heads / c->num_kv_heads) * ((size_t)m->lsh_tables << m->lsh_bits) > skv::kLshMaxEntries)
      return SKV_ERR_UNSUPPORTED;
  } else if (kind == SKV_SCORE_GAUSS || kind == SKV_SCORE_GAUSS_Q) {
    if (!(m->kinds & SKV_META_GAUSS) || !m->gauss || !out->m || !out->s || !out->shat || !aligned(m->gauss, 16))
      return SKV_ERR_INVALID_ARG;
    if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f)) return SKV_ERR_INVALID_ARG;
  } else if (kind == SKV_SCORE_PROJ) {
    if (!(m->kinds & SKV_META_PROJ) || !m->kproj || !m->proj) return SKV_ERR_INVALID_ARG;
    if (!rank_ok(m->proj_rank)) return SKV_ERR_UNSUPPORTED;
    if (!aligned(m->kproj, 16) || !aligned(m->proj, 16)) return SKV_ERR_INVALID_ARG;
    if (out->token_k < 0) return SKV_ERR_INVALID_ARG;
    if (out->token_k > 0) {
      if (!out->cand || !aligned(out->cand, 256)) return SKV_ERR_INVALID_ARG;
      const skv::CandLayout lay(c->batch, c->num_q_heads, c->num_kv_heads, c->max_pages * c->page_size, 64);
      if (lay.nb > 8192) return SKV_ERR_UNSUPPORTED;
      const int32_t ph = out->token_phase;
      if (ph != SKV_TOKEN_PHASE_ALL && ph != SKV_TOKEN_PHASE_BOUND && ph != SKV_TOKEN_PHASE_FILTER)
        return SKV_ERR_INVALID_ARG;
      (void)hipGetLastError();
      hipError_t e = hipSuccess;
      if (ph != SKV_TOKEN_PHASE_FILTER)
        e = skv::launch_token_bound(v, c->dtype, q, out->token_k, m->proj_rank, m->proj, m->kproj,
                                    static_cast<char *>(out->cand), s);
      if (e == hipSuccess && ph != SKV_TOKEN_PHASE_BOUND)
        e = skv::launch_score_proj_cand(v, m->proj_rank, m->kproj, static_cast<char *>(out->cand), s, ev);
      return hip_status(e);
    }
    if (!out->key) return SKV_ERR_INVALID_ARG;
  } else {
    return SKV_ERR_INVALID_ARG;
  }
  const size_t need =
      score_ws(c, kind, m->proj_rank,
               kind == SKV_SCORE_LSH ? ((size_t)c->num_q_heads / c->num_kv_heads) * ((size_t)m->lsh_tables << m->lsh_bits)
                                     : 0);
  if (need && (!workspace || workspace_bytes < need || !aligned(workspace, 8))) return SKV_ERR_WORKSPACE;
  double *ws = static_cast<double *>(workspace);
  (void)hipGetLastError();
  hipError_t e;
  if (kind == SKV_SCORE_BOX)
    e = skv::launch_score_box(v, c->dtype, q, m->box, out->key, ws, s, ev);
  else if (kind == SKV_SCORE_POOL)
    e = skv::launch_score_pool(v, c->dtype, q, m->pool_block, m->pool, out->key, s, ev);
  else if (kind == SKV_SCORE_LSH)
    e = skv::launch_score_lsh(v, c->dtype, q, m->lsh_tables, m->lsh_bits, m->lsh_planes, sm_scale, m->lsh_bucket,
                              m->vnorm, out->key, workspace, s, ev);
  else if (kind == SKV_SCORE_GAUSS || kind == SKV_SCORE_GAUSS_Q)
    e = skv::launch_score_gauss(v, c->dtype, q, m->gauss, sm_scale, kind == SKV_SCORE_GAUSS_Q, out->m, out->s,
                                out->shat, s, ev);
  else
    e = skv::launch_score_proj(v, c->dtype, q, m->proj_rank, m->proj, m->kproj, out->key, ws, s, ev);
  return hip_status(e);
}

skv_status skv_select_pages(const skv_cache *c, const skv_scores *sc, const skv_select_params *p, int32_t *sel_idx,
                            int32_t *sel_count, int32_t cap, float *tau_hat, void *workspace, size_t workspace_bytes,
                            void *stream) {
  skv_status st = check_cache(c);
  if (st != SKV_OK) return st;
  if (!sc || !p || !sel_idx || !sel_count || cap < 1) return SKV_ERR_INVALID_ARG;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (debug_on() && (st = debug_check_cache(c, s)) != SKV_OK) return st;
  const CacheView v = view(c);
  const int maxP = c->max_pages, Lmax = c->max_pages * c->page_size;
  (void)hipGetLastError();
  switch (p->policy) {
    case SKV_SEL_TOPK:
    case SKV_SEL_TOKEN_TOPK: {
      if (p->policy == SKV_SEL_TOKEN_TOPK && sc->token_k > 0) {   // candidate set of a fused scoring
        if (p->k != sc->token_k || !sc->cand || !aligned(sc->cand, 256)) return SKV_ERR_INVALID_ARG;
        if (cap < p->k) return SKV_ERR_CAPACITY;
        const skv::CandLayout lay(c->batch, c->num_q_heads, c->num_kv_heads, c->max_pages * c->page_size, 64);
        if (lay.nb > 8192) return SKV_ERR_UNSUPPORTED;
        return hip_status(skv::launch_select_token_cand(v, p->k, 64, static_cast<const char *>(sc->cand), sel_idx,
                                                        sel_count, cap, s));
      }
      if (p->k < 1 || !sc->key) return SKV_ERR_INVALID_ARG;
      if (cap < p->k) return SKV_ERR_CAPACITY;
      if (p->policy == SKV_SEL_TOKEN_TOPK && workspace && aligned(workspace, 256)) {
        const skv::CandLayout lay(c->batch, c->num_q_heads, c->num_kv_heads, Lmax, 64);
        if (lay.nb <= 8192 && workspace_bytes >= lay.total)
          return hip_status(skv::launch_select_token_dense(v, sc->key, Lmax, p->k, static_cast<char *>(workspace),
                                                           sel_idx, sel_count, cap, s));
      }
      const int stride = p->policy == SKV_SEL_TOPK ? maxP : Lmax;
      return hip_status(skv::launch_select_topk(v, sc->key, stride, p->policy, p->k, 0, sel_idx, sel_count, cap, s));
    }
    case SKV_SEL_BUDGET: {
      if (p->budget_pct < 1 || p->budget_pct > 100 || !sc->key) return SKV_ERR_INVALID_ARG;
      if (cap < budget_cap(maxP, p->budget_pct)) return SKV_ERR_CAPACITY;
      return hip_status(
          skv::launch_select_topk(v, sc->key, maxP, p->policy, 0, p->budget_pct, sel_idx, sel_count, cap, s));
    }
    case SKV_SEL_THRESH_GAUSS:
    case SKV_SEL_THRESH_BOX: {
      const bool box = p->policy == SKV_SEL_THRESH_BOX;
      if (!sc->m || !sc->s || !tau_hat || (box ? !sc->key : !sc->shat)) return SKV_ERR_INVALID_ARG;
      if (!std::isfinite(p->delta) || p->delta < 0.0f) return SKV_ERR_INVALID_ARG;
      if (!std::isfinite(p->alpha) || !(p->alpha > 1.0f && p->alpha <= 2.0f)) return SKV_ERR_INVALID_ARG;
      if (box && (!std::isfinite(p->scale) || !(p->scale > 0.0f))) return SKV_ERR_INVALID_ARG;
      if (cap < maxP) return SKV_ERR_CAPACITY;
      if (box)
        return hip_status(skv::launch_select_thresh_box(v, sc->m, sc->s, sc->key, p->alpha, p->scale, p->delta, tau_hat,
                                                        sel_idx, sel_count, cap, s));
      return hip_status(skv::launch_select_thresh(v, sc->m, sc->s, sc->shat, p->alpha, p->delta, tau_hat, sel_idx,
                                                  sel_count, cap, s));
    }
    case SKV_SEL_ALL: {
      if (p->tokens != 0 && p->tokens != 1) return SKV_ERR_INVALID_ARG;
      if (cap < (p->tokens ? Lmax : maxP)) return SKV_ERR_CAPACITY;
      return hip_status(skv::launch_select_all(v, p->tokens, sel_idx, sel_count, cap, s));
    }
    default:
      return SKV_ERR_INVALID_ARG;
  }
}

// Validation and split-K plan shared by both attention entry points.
static skv_status attn_check(const skv_cache *c, const void *q, const int32_t *sel_idx, const int32_t *sel_count,
                             int32_t cap, const skv_attn_params *p, float *out, AttnPlan *plan) {
  skv_status st = check_cache(c);
  if (st != SKV_OK) return st;
  if (!q || !sel_idx || !sel_count || !out || cap < 1) return SKV_ERR_INVALID_ARG;
  if (!aligned(q, 16)) return SKV_ERR_INVALID_ARG;
  if ((st = check_attn_params(p)) != SKV_OK) return st;
  // the entmax logits kernel of bf16 caches keeps 32-bit row indices (any cache that fits in
  // device memory has fewer than 2^32 - 1 rows)
  if (p->alpha != 1.0f && c->dtype == SKV_DTYPE_BF16 &&
      (uint64_t)c->num_phys_pages * c->num_kv_heads * c->page_size >= 0xffffffffull)
    return SKV_ERR_UNSUPPORTED;
  return attn_plan(c, p, cap, plan);
}

static skv_status attn_launch(const skv_cache *c, const void *q, const int32_t *sel_idx, const int32_t *sel_count,
                              int32_t cap, const skv_attn_params *p, float *out, char *ws, const AttnPlan &plan,
                              void *stream) {
  if (debug_on()) {
    const skv_status st =
        debug_check_selection(c, sel_idx, sel_count, cap, p->granularity, static_cast<hipStream_t>(stream));
    if (st != SKV_OK) return st;
  }
  skv::AttnArgs a;
  a.c = view(c);
  a.dtype = c->dtype;
  a.q = q;
  a.sel_idx = sel_idx;
  a.sel_count = sel_count;
  a.cap = cap;
  a.gran = p->granularity;
  a.spi = plan.spi;
  a.nsplit = plan.nsplit;
  a.alpha = p->alpha;
  a.sm_scale = p->sm_scale;
  a.out = out;
  a.part = plan.part ? reinterpret_cast<float *>(ws) : nullptr;
  a.cand = plan.cand ? reinterpret_cast<float2 *>(ws) : nullptr;
  a.cand_cnt = plan.cnt ? reinterpret_cast<int32_t *>(ws + plan.cand) : nullptr;
  a.cand_max = plan.mx ? reinterpret_cast<float *>(ws + plan.cand + plan.cnt) : nullptr;
  a.ev = events(p->ev_begin, p->ev_end);
  (void)hipGetLastError();
  return hip_status(skv::launch_attn(a, static_cast<hipStream_t>(stream)));
}

skv_status skv_sparse_decode_attn(const skv_cache *c, const void *q, const int32_t *sel_idx, const int32_t *sel_count,
                                  int32_t cap, const skv_attn_params *p, float *out, void *workspace,
                                  size_t workspace_bytes, void *stream) {
  AttnPlan plan;
  skv_status st = attn_check(c, q, sel_idx, sel_count, cap, p, out, &plan);
  if (st != SKV_OK) return st;
  if (plan.total && (!workspace || workspace_bytes < plan.total || !aligned(workspace, 16))) return SKV_ERR_WORKSPACE;
  return attn_launch(c, q, sel_idx, sel_count, cap, p, out, static_cast<char *>(workspace), plan, stream);
}

skv_status skv_sparse_decode_attn_noalloc(const skv_cache *c, const void *q, const int32_t *sel_idx,
                                          const int32_t *sel_count, int32_t cap, const skv_attn_params *p,
                                          float *out, void *stream) {
  AttnPlan plan;
  skv_status st = attn_check(c, q, sel_idx, sel_count, cap, p, out, &plan);
  if (st != SKV_OK) return st;
  if (plan.total > skv::kScratchBytes) return SKV_ERR_WORKSPACE;
  void *ws = nullptr;
  if (plan.total && skv::scratch_address(&ws) != hipSuccess) {
    (void)hipGetLastError();
    return SKV_ERR_HIP;
  }
  return attn_launch(c, q, sel_idx, sel_count, cap, p, out, static_cast<char *>(ws), plan, stream);
}

}  // extern "C"
