// Fixed device scratch for callers that cannot allocate (code under graph capture, tight serving
// loops): a file-scope device array that serves as the attention workspace of
// skv_sparse_decode_attn_noalloc. Every GPU the library runs on holds its own copy, at its own
// address, until the process ends. Calls on one GPU share that copy, so calls that overlap on one
// GPU race. The attention kernels write every workspace entry they later read, so nothing needs
// clearing between calls.
#include <hip/hip_runtime.h>

#include <atomic>

#include "launch.hpp"

namespace skv {

namespace {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
// Device address of `scratch` per device, looked up once on the first call there (with that device
// current) and only read afterwards. In host code the array's own name is a host-side stand-in, not a
// device address, so it is never passed to a kernel or a copy.
std::atomic<void *> g_scratch_addr[kMaxDevices];

}  // namespace

hipError_t scratch_address(void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void *p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_addr[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace skv
