// Internal launchers of libskv (host functions defined next to their kernels).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace skv {

// Optional caller-owned HIP events, recorded on the launch stream right before and right after one
// kernel launch, so that their elapsed time is that kernel alone (a measurement aid). Nothing is
// recorded when either event is null or the stream is being captured into a graph. The library keeps
// no state of its own for them.
struct KernelEvents {
  hipEvent_t begin = nullptr, end = nullptr;
  bool active(hipStream_t st) const {
    if (!begin || !end) return false;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess) {
      (void)hipGetLastError();
      return false;
    }
    return cs == hipStreamCaptureStatusNone;
  }
  hipError_t before(hipStream_t st) const { return active(st) ? hipEventRecord(begin, st) : hipSuccess; }
  // the launch status of the kernel just launched, then the closing record
  hipError_t after(hipStream_t st) const {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return active(st) ? hipEventRecord(end, st) : hipSuccess;
  }
};

struct AttnArgs {
  CacheView c;
  int dtype;
  const void *q;
  const int32_t *sel_idx;
  const int32_t *sel_count;
  int cap, gran, spi, nsplit;
  float alpha, sm_scale;
  float *out;
  float *part;       // softmax split partials [U, nsplit, G, D + 2]
  float2 *cand;      // entmax (z', slot) pairs [U, G, nsplit, rps]
  int32_t *cand_cnt; // [U, G, nsplit]
  float *cand_max;   // [U, G, nsplit]
  KernelEvents ev;   // around the first attention kernel
};

hipError_t launch_build_meta(const CacheView &c, int dtype, int tail, void *box, float *gauss, int r,
                             const float *proj, uint16_t *kproj, int pb, float *pool, hipStream_t st);
hipError_t launch_build_lsh(const CacheView &c, int dtype, int tail, int L, int P, const float *planes,
                            uint8_t *bucket, float *vnorm, hipStream_t st);
hipError_t launch_score_box(const CacheView &c, int dtype, const void *q, const void *box, float *key, double *ws,
                            hipStream_t st, const KernelEvents &ev);
hipError_t launch_score_lsh(const CacheView &c, int dtype, const void *q, int L, int P, const float *planes,
                            float tau, const uint8_t *bucket, const float *vnorm, float *key, void *ws,
                            hipStream_t st, const KernelEvents &ev);
hipError_t launch_score_gauss(const CacheView &c, int dtype, const void *q, const float *gauss, float scale,
                              int quantile, float *m, float *s, float *shat, hipStream_t st, const KernelEvents &ev);
hipError_t launch_score_pool(const CacheView &c, int dtype, const void *q, int pb, const float *pool, float *key,
                             hipStream_t st, const KernelEvents &ev);
hipError_t launch_score_proj(const CacheView &c, int dtype, const void *q, int r, const float *proj,
                             const uint16_t *kproj, float *key, double *ws, hipStream_t st,
                             const KernelEvents &ev);
hipError_t launch_score_proj_cand(const CacheView &c, int r, const uint16_t *kproj, char *cand, hipStream_t st,
                                  const KernelEvents &ev);
hipError_t launch_token_bound(const CacheView &c, int dtype, const void *q, int k, int r, const float *proj,
                              const uint16_t *kproj, char *cand, hipStream_t st);
hipError_t launch_select_token_cand(const CacheView &c, int k, int r, const char *cand, int32_t *sel_idx,
                                    int32_t *sel_count, int cap, hipStream_t st);
hipError_t launch_select_token_dense(const CacheView &c, const float *key, int key_stride, int k, char *ws,
                                     int32_t *sel_idx, int32_t *sel_count, int cap, hipStream_t st);
hipError_t launch_select_topk(const CacheView &c, const float *key, int key_stride, int policy, int k, int pct,
                              int32_t *sel_idx, int32_t *sel_count, int cap, hipStream_t st);
hipError_t launch_select_all(const CacheView &c, int tokens, int32_t *sel_idx, int32_t *sel_count, int cap,
                             hipStream_t st);
hipError_t launch_tau_hat(const CacheView &c, const float *m, const float *s, float alpha, float *tau,
                          hipStream_t st);
hipError_t launch_select_thresh_box(const CacheView &c, const float *m, const float *s, const float *key, float alpha,
                                    float scale, float delta, float *tau, int32_t *sel_idx, int32_t *sel_count,
                                    int cap, hipStream_t st);
hipError_t launch_select_thresh(const CacheView &c, const float *m, const float *s, const float *shat, float alpha,
                                float delta, float *tau, int32_t *sel_idx, int32_t *sel_count, int cap, hipStream_t st);
hipError_t launch_attn(const AttnArgs &a, hipStream_t st);

// The fixed device scratch of skv_sparse_decode_attn_noalloc (noalloc.hip): kScratchBytes on each
// device; scratch_address gives its device address on the current device.
constexpr size_t kScratchBytes = size_t(64) << 20;
hipError_t scratch_address(void **ptr);

}  // namespace skv
