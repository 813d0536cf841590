// Error word of the bounds-checked build (compiled with MLA_DEBUG_BOUNDS).
//
// The page table is device memory, so the host layer cannot check what it holds: a seq_lens entry
// past max_seq_len or a page id past the pool would make the kernels read (or, for the cache
// append, write) outside the caller's buffers.  In the bounds-checked build every kernel that
// walks the table tests the entries it uses and reports a violation in a per-device word pair:
// word 0 = the union of the violation bits (kBoundsBadSeqLen, kBoundsBadPage), word 1 = a count of
// reports (one per lane that saw a violation).  The word lives in a file-scope device array whose
// device address is looked up once per device and passed to the kernels like any other pointer;
// mla_debug_bounds_read copies it back and optionally clears it.  The table itself is the one of
// the Perplexity post, section "Слой MLA" (paged cache addressed through a page table).
//
// In the other build the kernels carry the same arguments and test nothing, the word does not
// exist and mla_debug_bounds_read reports MLA_ERR_UNSUPPORTED.
#include <hip/hip_runtime.h>

#include <atomic>

#include "../../include/mla_latent.h"
#include "kernels.h"

namespace mla {

#ifdef MLA_DEBUG_BOUNDS
namespace {
static __device__ __align__(16) uint32_t bounds_word[4];
constexpr int kMaxDevices = 64;
std::atomic<uint32_t*> g_word[kMaxDevices];  // device address of bounds_word per device
}  // namespace

uint32_t* bounds_error_word() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  uint32_t* p = g_word[dev].load(std::memory_order_acquire);
  if (p) return p;
  void* q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(bounds_word)) != hipSuccess || !q) return nullptr;
  g_word[dev].store((uint32_t*)q, std::memory_order_release);
  return (uint32_t*)q;
}
#else
uint32_t* bounds_error_word() { return nullptr; }
#endif

}  // namespace mla

extern "C" int32_t mla_debug_bounds_enabled(void) {
#ifdef MLA_DEBUG_BOUNDS
  return 1;
#else
  return 0;
#endif
}

extern "C" mla_status mla_debug_bounds_read(uint32_t* words, int32_t clear) {
#ifdef MLA_DEBUG_BOUNDS
  if (!words) return MLA_ERR_NULL;
  uint32_t* w = mla::bounds_error_word();
  if (!w) return MLA_ERR_DEVICE;
  // every kernel enqueued so far on any stream of the device has reported
  if (hipDeviceSynchronize() != hipSuccess) return MLA_ERR_DEVICE;
  uint32_t h[2] = {0u, 0u};
  if (hipMemcpy(h, w, sizeof h, hipMemcpyDeviceToHost) != hipSuccess) return MLA_ERR_DEVICE;
  words[0] = h[0];
  words[1] = h[1];
  if (clear) {
    const uint32_t z[2] = {0u, 0u};
    if (hipMemcpy(w, z, sizeof z, hipMemcpyHostToDevice) != hipSuccess) return MLA_ERR_DEVICE;
  }
  return MLA_OK;
#else
  (void)words;
  (void)clear;
  return MLA_ERR_UNSUPPORTED;
#endif
}
