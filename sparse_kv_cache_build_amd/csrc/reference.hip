// Reference kernels for the benchmark's bandwidth ceilings (libskv_ref.so, loaded by bench.py only;
// not part of the decode path): what this GPU delivers for a plain one-pass streaming read, and
// for a gather of scattered fixed-size rows as the attention reads K and V. Each kernel folds what
// it reads into one word per thread block, so that no load can be dropped.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

constexpr int kThreads = 256;
constexpr int kInFlight = 4;   // 16-byte loads per lane issued before any is used

__device__ __forceinline__ uint32_t fold(uint4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// A 16-byte load, marked non-temporal when NT (the line is not kept for reuse).
template <bool NT>
__device__ __forceinline__ uint4 ld(const uint4 *p) {
  if (!NT) return *p;
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void block_out(uint32_t acc, uint32_t *out) {
  __shared__ uint32_t red[kThreads / 64];
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x / 64] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int i = 0; i < kThreads / 64; ++i) r ^= red[i];
    out[blockIdx.x] = r;
  }
}

// Streaming read of n 16-byte words: a grid-stride loop, kInFlight consecutive strides per step.
template <bool NT>
__global__ __launch_bounds__(kThreads) void ref_stream_read_kernel(const uint4 *__restrict__ src, size_t n,
                                                                   uint32_t *__restrict__ out) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kInFlight - 1) * stride < n; i += kInFlight * stride) {
    uint4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) v[u] = ld<NT>(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) acc ^= fold(v[u]);
  }
  for (; i < n; i += stride) acc ^= fold(ld<NT>(src + i));
  block_out(acc, out);
}

// Gather of n_rows rows of row_words 16-byte words each, row r starting at word offset off[r]: a
// group of row_words lanes reads one row (16 bytes per lane), each group two rows per step with
// both in flight, as the attention's lane groups read K and V rows.
template <bool NT>
__global__ __launch_bounds__(kThreads) void ref_gather_rows_kernel(const uint4 *__restrict__ base,
                                                                   const int64_t *__restrict__ off, int n_rows,
                                                                   int row_words, uint32_t *__restrict__ out) {
  const int groups_per_block = kThreads / row_words;
  const int lane_in_row = threadIdx.x % row_words, grp = threadIdx.x / row_words;
  const int total_groups = gridDim.x * groups_per_block;
  uint32_t acc = 0;
  if (grp < groups_per_block) {
    int r = blockIdx.x * groups_per_block + grp;
    for (; r + total_groups < n_rows; r += 2 * total_groups) {
      const uint4 a = ld<NT>(base + off[r] + lane_in_row);
      const uint4 b = ld<NT>(base + off[r + total_groups] + lane_in_row);
      acc ^= fold(a) ^ fold(b);
    }
    if (r < n_rows) acc ^= fold(ld<NT>(base + off[r] + lane_in_row));
  }
  block_out(acc, out);
}

}  // namespace

extern "C" {

// n16: 16-byte words at src (16-byte aligned); out: one uint32 per block (blocks entries);
// nontemporal: mark the loads non-temporal. Returns a hipError_t value.
int skv_ref_stream_read(const void *src, size_t n16, uint32_t *out, int blocks, int nontemporal, void *stream) {
  if (!src || !out || blocks < 1) return (int)hipErrorInvalidValue;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (nontemporal)
    ref_stream_read_kernel<true><<<blocks, kThreads, 0, st>>>(static_cast<const uint4 *>(src), n16, out);
  else
    ref_stream_read_kernel<false><<<blocks, kThreads, 0, st>>>(static_cast<const uint4 *>(src), n16, out);
  return (int)hipGetLastError();
}

// off: n_rows int64 word offsets (device); row_words divides 256 (row bytes / 16).
int skv_ref_gather_rows(const void *base, const int64_t *off, int n_rows, int row_words, uint32_t *out, int blocks,
                        int nontemporal, void *stream) {
  if (!base || !off || !out || blocks < 1 || row_words < 1 || kThreads % row_words) return (int)hipErrorInvalidValue;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (nontemporal)
    ref_gather_rows_kernel<true><<<blocks, kThreads, 0, st>>>(static_cast<const uint4 *>(base), off, n_rows,
                                                               row_words, out);
  else
    ref_gather_rows_kernel<false><<<blocks, kThreads, 0, st>>>(static_cast<const uint4 *>(base), off, n_rows,
                                                                row_words, out);
  return (int)hipGetLastError();
}

}  // extern "C"
