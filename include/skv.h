/*
 * skv.h -- C ABI of libskv.so: query-aware sparse decode attention over a paged
 * grouped-query (GQA) KV cache, for AMD Instinct MI355X (gfx950).
 *
 * The calls follow the pipeline the pages describe for one decode step:
 *   skv_build_page_meta    per-page metadata, once per page at prefill time
 *   skv_append_page_meta   the same metadata kept current for the pages that new tokens reach
 *                          ("EntmaxKV" summary, s2.A: box bounds k_min/k_max and Gaussian
 *                          moments stored per page; "Joint Subspace Sparse Attention" abstract:
 *                          keys cached in a shared low-dimensional subspace)
 *   skv_score_pages        query-aware page (or token) scores from the metadata ("EntmaxKV" s2.A)
 *   skv_select_pages       candidate selection: top-k pages, a page budget, the Gaussian-aware
 *                          entmax threshold tau_hat with margin Delta ("EntmaxKV" s2.B), or
 *                          top-k tokens per KV head ("Joint Subspace Sparse Attention" abstract;
 *                          "SOCKET" summary, Methodology step 4)
 *   skv_sparse_decode_attn softmax or alpha-entmax attention over the selected KV only
 *                          ("EntmaxKV" s2.C; softmax is the comparator of s1 and s3)
 *
 * Conventions shared by every call
 *   - Memory: every pointer in a struct or argument is a device pointer unless stated
 *     otherwise; the caller owns all memory, including workspaces (size them with
 *     skv_workspace_bytes). The library never allocates or frees memory, creates no HIP objects
 *     and keeps no mutable state between calls.
 *   - Streams: `stream` is a hipStream_t (NULL = the null stream). Every call only enqueues
 *     work on it and returns; nothing is synchronised. Results are valid once the stream
 *     reaches the enqueued work.
 *   - Errors: arguments are validated on the host before anything is enqueued; on any error
 *     nothing is enqueued and a non-zero skv_status is returned. A launch failure reported by
 *     the HIP runtime returns SKV_ERR_HIP. Device-side data (seq_lens, block_table, counts)
 *     cannot be validated on the host: seq_lens are clamped to [0, max_pages * page_size],
 *     block_table entries of pages below the clamped length must lie in [0, num_phys_pages),
 *     sel_count entries are clamped to [0, cap]. With the environment variable SKV_DEBUG set
 *     (to anything but "0"), every call first synchronises its stream and checks these on the
 *     host: block_table entries of the pages in use in [0, num_phys_pages), and for the
 *     attention also sel_count in [0, cap] and selections strictly ascending inside the
 *     sequence; a violation returns SKV_ERR_INVALID_ARG and nothing is launched.
 *   - Threading: calls are reentrant; concurrent calls must not share output or workspace
 *     buffers.
 *   - Determinism: for a fixed input, launch configuration and device, outputs are bitwise
 *     reproducible (no floating-point atomics).
 *
 * Cache layout ("Joint Subspace Sparse Attention" abstract: the standard GQA paged layout)
 *   k, v        [num_phys_pages, num_kv_heads, page_size, head_dim], dtype `dtype`
 *   block_table [batch, max_pages] int32: logical page p of sequence b -> physical page
 *   seq_lens    [batch] int32
 *   q           [batch, num_q_heads, head_dim], dtype `dtype`
 *   Query head h reads KV head h / G, G = num_q_heads / num_kv_heads. Page p of sequence b holds
 *   tokens [p*S, min(p*S + S, L_b)). A physical page is referenced by at most one
 *   (sequence, logical page).
 * Supported: head_dim 64 or 128; page_size 1..1024; G in {1, 2, 4, 8}; dtype f32 or bf16.
 */
#ifndef SKV_H
#define SKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum skv_status {
  SKV_OK = 0,
  SKV_ERR_INVALID_ARG = 1, /* null pointer, bad size, inconsistent dimensions */
  SKV_ERR_UNSUPPORTED = 2, /* valid but outside the supported set above */
  SKV_ERR_CAPACITY = 3,    /* an output capacity (cap) is too small for the policy */
  SKV_ERR_WORKSPACE = 4,   /* workspace missing or smaller than skv_workspace_bytes */
  SKV_ERR_HIP = 5          /* the HIP runtime reported an error */
} skv_status;

enum { SKV_DTYPE_F32 = 0, SKV_DTYPE_BF16 = 1 };

typedef struct skv_cache {
  int32_t batch;          /* B */
  int32_t num_q_heads;    /* Hq */
  int32_t num_kv_heads;   /* Hkv; Hq must be a multiple */
  int32_t head_dim;       /* d */
  int32_t page_size;      /* S (tokens per page) */
  int32_t max_pages;      /* columns of block_table */
  int32_t num_phys_pages; /* rows of k and v */
  int32_t dtype;          /* SKV_DTYPE_* of k, v, q and the box metadata */
  const void *k;
  const void *v;
  const int32_t *block_table;
  const int32_t *seq_lens;
} skv_cache;

/* ------------------------------------------------------------------ page metadata */

enum { SKV_META_BOX = 1, SKV_META_GAUSS = 2, SKV_META_PROJ = 4, SKV_META_POOL = 8, SKV_META_LSH = 16 };

typedef struct skv_meta {
  uint32_t kinds;     /* OR of SKV_META_* to build (build_page_meta) / available (score) */
  void *box;          /* BOX:   [Nphys, Hkv, d/C, 2, C] cache dtype, C = 64 bytes of elements
                         (32 bf16, 16 float32): 64-byte blocks of k_min and of k_max alternate */
  float *gauss;       /* GAUSS: [Nphys, Hkv, d/16, 2, 16] float32: 64-byte blocks of the mean and
                         of the variance row alternate (16 coordinates each) */
  int32_t proj_rank;  /* PROJ:  r: 16, 32 or 64 */
  const float *proj;  /* PROJ:  [r, d] float32 projection shared by queries and keys */
  uint16_t *kproj;    /* PROJ:  [Nphys, Hkv, S, r] bf16 bit patterns (16-byte aligned) */
  int32_t pool_block; /* POOL:  tokens per sub-block, dividing S */
  float *pool;        /* POOL:  [Nphys, Hkv, S / pool_block, d] float32 sub-block mean keys */
  int32_t lsh_tables; /* LSH:   number of hash tables L: 16, 32, 48 or 64 */
  int32_t lsh_bits;   /* LSH:   hyperplanes per table P, 1..8 (2^P buckets) */
  const float *lsh_planes; /* LSH: [L, P, d] float32 hyperplanes (read only, 16-byte aligned) */
  uint8_t *lsh_bucket; /* LSH:  [Nphys, Hkv, S, L] bucket id of every token in every table */
  float *vnorm;       /* LSH:   [Nphys, Hkv, S] float32 norm of every token's value vector */
} skv_meta;

/* Builds the requested metadata of every page in use (p < ceil(L_b / S)) from the valid tokens
 * of the page ("EntmaxKV" s2.A; "Joint Subspace Sparse Attention" abstract).
 *   BOX:   coordinate-wise min and max of the keys (exact, stored in the cache dtype).
 *   GAUSS: per-coordinate mean and population variance, computed in float64 (mean first, then
 *          mean squared deviation) and rounded once to float32.
 *   PROJ:  k~_t[i] = RN_bf16(sum_j proj[i][j] k_t[j]), the sum in float64 over j ascending.
 *   POOL:  per sub-block of pool_block token slots, RN_f32 of the float64 mean of its valid keys
 *          (sum over t ascending, divided by their number) ("NOSA" summary s1: mean pooling
 *          within sub-blocks).
 *   LSH:   per token and table l, the bucket id whose bit i is set iff lsh_planes[l][i] . k_t > 0
 *          (float64 sum over j ascending, exact products), and vnorm = RN_f32(sqrt(sum_j v_j^2))
 *          (float64 sum) ("SOCKET" summary, Methodology, soft LSH step 1: keys hashed into L
 *          tables by random projections at prefill, value norms cached).
 * Not written: metadata of unused physical pages, kproj and LSH rows of tokens past L_b, and pool
 * rows of sub-blocks without a valid token.
 * Errors: SKV_ERR_INVALID_ARG for null or inconsistent arguments or a missing output of a
 * requested kind; SKV_ERR_UNSUPPORTED outside the supported set (also: PROJ or LSH over a cache
 * of more than 2^32 - 1 KV rows, num_phys_pages * num_kv_heads * page_size, more than device
 * memory holds). */
skv_status skv_build_page_meta(const skv_cache *c, const skv_meta *m, void *stream);

/* Keeps the metadata current while decoding. The metadata is stored per page and maintained as
 * the cache grows ("EntmaxKV" s2.A). The caller has written the last n_new tokens of every
 * sequence into k (seq_lens already counts them; a sequence shorter than n_new counts all its
 * tokens as new). For every page holding one of those tokens, BOX, GAUSS and POOL are
 * recomputed over all valid tokens of the page, and PROJ and LSH rows are written for the new
 * tokens only. Afterwards the metadata of those pages equals what skv_build_page_meta writes for
 * them (bit for bit, same arithmetic); every other page and row is left untouched. A page holds at most S tokens, so
 * the work per sequence and KV head is O(S d), whatever the context length.
 * Errors: as skv_build_page_meta, and SKV_ERR_INVALID_ARG for n_new < 1. */
skv_status skv_append_page_meta(const skv_cache *c, const skv_meta *m, int32_t n_new, void *stream);

/* ------------------------------------------------------------------ scores */

enum {
  SKV_SCORE_BOX = 0,
  SKV_SCORE_GAUSS = 1,
  SKV_SCORE_PROJ = 2,
  SKV_SCORE_GAUSS_Q = 3,
  SKV_SCORE_POOL = 4,
  SKV_SCORE_LSH = 5
};

typedef struct skv_scores {
  float *key;   /* BOX, POOL: [B, Hkv, max_pages]; PROJ, LSH: [B, Hkv, max_pages * S] */
  float *m;     /* GAUSS, GAUSS_Q: [B, Hq, max_pages] Gaussian mean of the scaled scores of the page */
  float *s;     /* GAUSS: [B, Hq, max_pages] its standard deviation */
  float *shat;  /* GAUSS: [B, Hq, max_pages] estimated maximum m + s sqrt(2 ln n_p) */
  int32_t token_k; /* PROJ only. 0: write every key into `key`. k > 0: write only the token candidates
                      a top-k selection can need into `cand` (key is unused); select them with
                      SKV_SEL_TOKEN_TOPK and the same k */
  void *cand;      /* PROJ with token_k > 0: opaque candidate set, skv_workspace_bytes(c,
                      SKV_OP_CANDIDATES, &token_k, 0) bytes, 256-byte aligned. The selection that
                      consumes it also reads the projected keys (meta->kproj), which must still hold
                      the same values */
  int32_t token_phase; /* PROJ with token_k > 0: which part of the candidate scoring a call runs.
                          SKV_TOKEN_PHASE_ALL (0) both; SKV_TOKEN_PHASE_BOUND (1) only the sampled
                          bound (projected queries and T_lo into cand); SKV_TOKEN_PHASE_FILTER (2)
                          only the filtered scoring of every token, which needs a BOUND call with
                          the same q and cand before it on the same stream. Ignored otherwise */
  void *ev_begin;  /* optional hipEvent_t pair owned by the caller (a measurement aid): when both are */
  void *ev_end;    /* non-null, skv_score_pages records ev_begin on the stream right before the scoring
                      kernel proper (after any query-preparation kernel; for the candidate scoring of a
                      token top-k, the filtered pass) and ev_end right after it, so that their elapsed
                      time is that kernel alone. Not recorded while the stream is being captured into a
                      graph. A failed record returns SKV_ERR_HIP. Ignored by skv_select_pages */
} skv_scores;

enum { SKV_TOKEN_PHASE_ALL = 0, SKV_TOKEN_PHASE_BOUND = 1, SKV_TOKEN_PHASE_FILTER = 2 };

/* Query-aware scores ("EntmaxKV" s2.A; "Joint Subspace Sparse Attention" abstract).
 *   BOX:   key[b][g][p] = RN_f32(max over the G query heads h of g of
 *          U_h(p) = sum_j max(q_hj k_min_j, q_hj k_max_j)), the upper bound of q_h . k over the
 *          page's box; float64 sum over j ascending (products are exact), unscaled.
 *   GAUSS: per query head, m = sm_scale sum_j q_j mean_j, s = sm_scale sqrt(sum_j q_j^2 var_j),
 *          shat = m + s sqrt(2 ln n_p) (n_p valid tokens of the page; shat = m for n_p = 1). The
 *          sums run in float32 (the scores only feed the threshold estimate): each is within
 *          about 2 d 2^-24 of the sum of the absolute terms of the float64 value.
 *   GAUSS_Q: the same m and s (GAUSS metadata, GAUSS outputs), with the estimated maximum
 *          shat = m + s Phi^-1(1 - 1/n_p), the normal quantile exceeded by one of n_p draws on
 *          average ("EntmaxKV" s2.B leaves the estimate open).
 *   PROJ:  q~_h = RN_f32(proj q_h) (float64 sum), u_h(t) = sum_i q~_h[i] k~_t[i] (float64 sum,
 *          i ascending), key[b][g][t] = RN_f32(max over the G heads of g of u_h(t)).
 *   POOL:  key[b][g][p] = RN_f32(max over the G heads h of g and the sub-blocks j of the page
 *          holding a valid token of sum_i q_hi pool_j[i]) (float64 sum, i ascending; products
 *          exact), unscaled: mean pooling of the scores within sub-blocks, then max pooling over
 *          the page ("NOSA" summary s1). TOPK and BUDGET select on it like on the BOX key.
 *   LSH:   soft-collision token scores ("SOCKET" summary, Methodology, soft LSH steps 2-3). Per
 *          query head and table l, z_i = lsh_planes[l][i] . q / ||q|| (float64; 0 for q = 0) and
 *          bucket beta gets the softmax mass p_l(beta) = prod_i sigma(2 s_i z_i / tau), s_i = +1
 *          where bit i of beta is set and -1 elsewhere, sigma(x) = 1 / (1 + exp(-x)) (the exact
 *          factorisation of a softmax over all 2^P sign vectors of <s, z> / tau), held as the
 *          integer T = p * 2^24 rounded to nearest even. key[b][g][t] = RN_f32(vnorm_t *
 *          (max over the G heads of sum_l T_l[bucket_l(t)]) * 2^-24), one float64 product. The
 *          temperature tau > 0 is passed in `sm_scale`. Needs G * L * 2^P <= 16384. Select with
 *          SKV_SEL_TOKEN_TOPK (tokens = 1).
 * Entries past the sequence (p >= ceil(L_b / S), or t >= L_b) are -inf (BOX, PROJ) or NaN
 * (GAUSS). `q` is [B, Hq, d] in the cache dtype. `workspace` must hold
 * skv_workspace_bytes(c, SKV_OP_SCORE, &kind, 0) bytes (256-byte aligned; GAUSS, GAUSS_Q, POOL and
 * BOX with at most 4 query heads per KV head need none and may pass NULL).
 * Errors: SKV_ERR_INVALID_ARG (null pointers, kind not in m->kinds, bad sm_scale or temperature),
 * SKV_ERR_WORKSPACE, SKV_ERR_UNSUPPORTED, SKV_ERR_HIP. */
skv_status skv_score_pages(const skv_cache *c, const skv_meta *m, const void *q, int32_t kind, float sm_scale,
                           const skv_scores *out, void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------ selection */

enum {
  SKV_SEL_TOPK = 0,         /* the k pages with the largest BOX key */
  SKV_SEL_BUDGET = 1,       /* the ceil(budget_pct * P_b / 100) pages (at least 1) with the largest BOX key */
  SKV_SEL_THRESH_GAUSS = 2, /* Gaussian-aware entmax threshold (GAUSS scores) */
  SKV_SEL_TOKEN_TOPK = 3,   /* the k tokens with the largest PROJ or LSH key */
  SKV_SEL_ALL = 4,          /* every page (tokens == 0) or every token (tokens == 1): full cache */
  SKV_SEL_THRESH_BOX = 5    /* the entmax threshold of THRESH_GAUSS tested against the BOX key */
};

typedef struct skv_select_params {
  int32_t policy;     /* SKV_SEL_* */
  int32_t k;          /* TOPK, TOKEN_TOPK: k >= 1 */
  int32_t budget_pct; /* BUDGET: 1..100 */
  float alpha;        /* THRESH_GAUSS, THRESH_BOX: 1 < alpha <= 2 */
  float delta;        /* THRESH_GAUSS, THRESH_BOX: safety margin Delta >= 0, in units of tau */
  int32_t tokens;     /* ALL: 0 pages, 1 tokens */
  float scale;        /* THRESH_BOX: the logit scale c (z = c q . k) the GAUSS scores were taken with */
} skv_select_params;

/* Candidate selection, one selection per (sequence, KV head) shared by its G query heads
 * ("Joint Subspace Sparse Attention" abstract: distinct selection per KV head).
 *   TOPK / BUDGET / TOKEN_TOPK: order candidates by (key descending, index ascending) and keep
 *     the first min(k, n); ties go to the lower index ("EntmaxKV" s2.B policy 1).
 *   THRESH_GAUSS ("EntmaxKV" s2.B policy 2): per query head, tau_hat solves
 *     sum_p n_p E[((alpha-1) Z_p - tau)_+^(1/(alpha-1))] = 1 with Z_p ~ N(m_p, s_p^2); a page is
 *     kept iff some head h of the group has (alpha-1) shat_h(p) > tau_hat_h - delta.
 *     tau_hat [B, Hq] float32 receives the thresholds (unused pointer otherwise). alpha = 1.5
 *     and 2 use the closed forms of the expectation; any other alpha in (1, 2) evaluates it from a
 *     table of the needed Gaussian integrals, filled once per solve by Gauss-Legendre quadrature.
 *   THRESH_BOX: tau_hat as THRESH_GAUSS (from the GAUSS m, s); the page's estimated maximum is
 *     the deterministic box bound ("EntmaxKV" s2.A): keep iff (alpha-1) scale key[p] >
 *     min_h tau_hat_h - delta, key = the BOX key (max over the group's heads of the unscaled
 *     bound). No page the per-head box test would keep is dropped. Needs the BOX key and the
 *     GAUSS m, s in the same skv_scores.
 * Output: sel_idx [B, Hkv, cap] int32 holds the kept logical page (or token) indices in
 * ascending order, sel_count [B, Hkv] int32 their number; entries past the count are not
 * written. cap must be >= k (TOPK, TOKEN_TOPK), >= max_pages (BUDGET, THRESH_*, ALL pages)
 * or >= max_pages * S (ALL tokens), else SKV_ERR_CAPACITY. The scores are those written by
 * skv_score_pages for the same cache.
 * workspace: optional. skv_workspace_bytes(c, SKV_OP_SELECT, p, cap) is non-zero only for
 * TOKEN_TOPK over dense keys (token_k = 0): given at least that many bytes, 256-byte aligned, the
 * selection runs on many workgroups per (sequence, KV head) (a sampled bound, a filtered pass and
 * an exact selection among the candidates); with less it runs on one workgroup per (sequence, KV
 * head). Both give the same indices. */
skv_status skv_select_pages(const skv_cache *c, const skv_scores *sc, const skv_select_params *p,
                            int32_t *sel_idx, int32_t *sel_count, int32_t cap, float *tau_hat, void *workspace,
                            size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------ attention */

typedef struct skv_attn_params {
  float alpha;         /* 1 = softmax; 1 < alpha <= 2 = alpha-entmax (2 = sparsemax) */
  float sm_scale;      /* logit scale c: z_t = c q_h . k_t (c > 0, finite) */
  int32_t granularity; /* 0: sel_idx holds logical pages; 1: sel_idx holds token positions */
  int32_t split;       /* selected items (pages or tokens) per split-K partition; 0 = automatic */
  void *ev_begin;      /* optional caller-owned hipEvent_t pair, recorded right before and right after */
  void *ev_end;        /* the first attention kernel (the softmax split kernel or the entmax logits
                          kernel); as in skv_scores. NULL: not recorded */
} skv_attn_params;

/* Attention of every query head over the KV rows its KV head selected ("EntmaxKV" s2.C; the
 * token-granular form reads the rows in place through block_table with no gathered copy,
 * "Joint Subspace Sparse Attention" abstract).
 *   z_t = sm_scale q_h . k_t (float32 accumulation), p = softmax(z) (alpha = 1) or
 *   p = [(alpha-1) z - tau]_+^(1/(alpha-1)) with sum p = 1 (entmax), out_h = sum_t p_t v_t.
 * Softmax runs as a split-K flash-decode (online max/sum per partition, fixed-order
 * log-sum-exp combine). Entmax runs in two passes: logits of each partition are filtered to
 * those within reach of the threshold ((alpha-1) z > (alpha-1) max z - 1), tau is solved per
 * head over the survivors (bisection, then the closed form on the support for alpha 1.5 and
 * 2), and V is read only for rows with p > 0.
 * sel_idx / sel_count / cap are as written by skv_select_pages (indices ascending, within the
 * sequence; others are skipped). out [B, Hq, d] float32; an empty selection gives zeros.
 * workspace: skv_workspace_bytes(c, SKV_OP_ATTN, p, cap). Errors: SKV_ERR_INVALID_ARG,
 * SKV_ERR_UNSUPPORTED (also: entmax over a bf16 cache of 2^32 - 1 or more KV rows,
 * num_phys_pages * num_kv_heads * page_size, more than device memory holds), SKV_ERR_WORKSPACE,
 * SKV_ERR_HIP. */
skv_status skv_sparse_decode_attn(const skv_cache *c, const void *q, const int32_t *sel_idx,
                                  const int32_t *sel_count, int32_t cap, const skv_attn_params *p, float *out,
                                  void *workspace, size_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): skv_sparse_decode_attn without a workspace argument. Its
 * workspace is a fixed device array inside the library, SKV_NOALLOC_SCRATCH_BYTES (64 MiB) on every
 * GPU the library runs on, held until the process ends; the first call on a device looks up that
 * device's copy. The call allocates nothing; the caller still passes every input and the output.
 * Results equal skv_sparse_decode_attn's bit for bit (same kernels, same plan).
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU (concurrent streams
 * or threads) race and must not be issued. Nothing needs clearing between calls.
 * Errors: as skv_sparse_decode_attn, and SKV_ERR_WORKSPACE when the call needs more workspace than
 * SKV_NOALLOC_SCRATCH_BYTES (skv_workspace_bytes(c, SKV_OP_ATTN, p, cap) says how much: large
 * entmax selections, whose candidate lists are sized for every selected row, can exceed it). */
#define SKV_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
skv_status skv_sparse_decode_attn_noalloc(const skv_cache *c, const void *q, const int32_t *sel_idx,
                                          const int32_t *sel_count, int32_t cap, const skv_attn_params *p,
                                          float *out, void *stream);

/* ------------------------------------------------------------------ utilities */

enum { SKV_OP_SCORE = 0, SKV_OP_SELECT = 1, SKV_OP_ATTN = 2, SKV_OP_CANDIDATES = 3 };

/* Workspace bytes the call `op` needs for this cache: params points to an int32_t score kind
 * (SCORE), a skv_select_params (SELECT), a skv_attn_params (ATTN) or the int32_t token_k of a
 * candidate set (CANDIDATES: the size of skv_scores.cand); cap as passed to that call.
 * Host-only; enqueues nothing. Writes *bytes; SKV_ERR_INVALID_ARG on bad arguments. */
skv_status skv_workspace_bytes(const skv_cache *c, int32_t op, const void *params, int32_t cap, size_t *bytes);

/* Static, human-readable name of a status code. Never NULL. */
const char *skv_status_str(skv_status s);

#ifdef __cplusplus
}
#endif

#endif /* SKV_H */
