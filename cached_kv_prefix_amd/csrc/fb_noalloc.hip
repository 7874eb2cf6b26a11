// fb_step for callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc): the step's split-KV partial
// results live in a static device array of the library instead of a caller workspace.
//
// The array is a module global: every GPU the library runs on holds one copy of
// FB_NOALLOC_SCRATCH_BYTES until the process ends.  Its device address is looked up once
// per device (hipGetSymbolAddress, with that device current) on the first call made on
// it, and kept; the host-side name of the array is never handed to a kernel or a copy.
// Nothing in it needs to start at zero: the attention launch writes every partial that
// the combine reads.  Calls that overlap on one GPU (different streams, or another thread)
// share the array and race; such callers must serialise them.
#include <hip/hip_runtime.h>

#include <mutex>

#include "flashblock.h"

namespace {

constexpr size_t kScratchBytes = FB_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of the current device's copy of `scratch` (looked up on first use).
fb_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FB_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FB_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FB_OK;
}

}  // namespace

extern "C" fb_status fb_step_noalloc(const fb_shape* s, const void* q, const void* k, const void* v,
                                     const void* k_blk, const void* v_blk, const uint8_t* reuse_mask,
                                     float* cache_a, float* cache_l, void* a_full, float* l_full,
                                     hipStream_t stream) {
  const size_t need = fb_workspace_size(s);
  if (need == 0)   // an invalid shape: fb_step returns its error before touching a workspace
    return fb_step(s, q, k, v, k_blk, v_blk, reuse_mask, cache_a, cache_l, a_full, l_full, nullptr, 0, nullptr,
                   stream);
  if (need > kScratchBytes) return FB_ERR_WORKSPACE;
  void* ws = nullptr;
  const fb_status st = scratch_of_current_device(&ws);
  if (st != FB_OK) return st;
  return fb_step(s, q, k, v, k_blk, v_blk, reuse_mask, cache_a, cache_l, a_full, l_full, ws, need, nullptr,
                 stream);
}
