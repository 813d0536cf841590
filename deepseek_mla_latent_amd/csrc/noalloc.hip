// mla_decode_attn_out_proj_static: the fused decode attention + out-projection for callers that
// cannot allocate (code under HIP-graph capture, serving loops that forbid allocation).  The split
// partials live in a file-scope device array instead of a caller workspace; each GPU holds its own
// copy for the life of the process.  The array's device address is looked up once per device with
// hipGetSymbolAddress (the array's name in host code is only a stand-in for it) and passed to the
// kernels like a workspace pointer.
#include <hip/hip_runtime.h>

#include <atomic>

#include "../../include/mla_latent.h"

namespace {

static_assert(MLA_STATIC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) char scratch[MLA_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];  // device address of `scratch` per device (null: not looked up)

// The current device's copy of `scratch`, or null if the device cannot be queried.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
  g_scratch[dev].store(p, std::memory_order_release);
  return p;
}

}  // namespace

extern "C" mla_status mla_decode_attn_out_proj_static(const void* q_lat, const void* q_pe, const void* kv_pool,
                                                      const int32_t* block_table, const int32_t* seq_lens,
                                                      const int32_t* tree_parents, const void* w_uv, void* out,
                                                      float* o_lat, float* lse, int32_t num_splits,
                                                      const mla_params* p, void* stream) {
  if (!p) return MLA_ERR_NULL;
  // the size the workspace of mla_decode_attn_out_proj would need (0 for invalid parameters, which
  // that call then reports), checked before anything touches the device
  const size_t need = mla_decode_attn_out_proj_workspace_bytes(p, num_splits);
  if (need > MLA_STATIC_SCRATCH_BYTES) return MLA_ERR_SCRATCH;
  void* ws = need > 0 ? scratch_on_current_device() : nullptr;
  if (need > 0 && !ws) return MLA_ERR_DEVICE;
  return mla_decode_attn_out_proj(q_lat, q_pe, kv_pool, block_table, seq_lens, tree_parents, w_uv, out, o_lat, lse,
                                  ws, need, num_splits, p, stream);
}
