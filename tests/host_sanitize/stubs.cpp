// Host-only stand-ins for the HIP runtime queries and the kernel launchers, linked with the C-ABI
// layer (mla_api.cpp) into an AddressSanitizer / UndefinedBehaviorSanitizer build that runs on a
// machine without a GPU.  Test infrastructure: never part of the product library.
//
// Every "device" pointer the test hands the C-ABI layer is host memory of exactly the documented
// size.  Each launcher stand-in reads the first and the last byte of every range its kernel would
// touch, as computed from the launch arguments alone, so a range the host layer got wrong (a
// workspace carved past its end, an output offset too far) is an out-of-bounds read that the
// sanitizer reports.  Launches are counted by kind.
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include "../../deepseek_mla_latent_amd/csrc/kernels.h"

namespace {

int g_cus = 256;
long g_launches[16];
enum Kind { kAttn, kLseMerge, kAbsorb, kMergeOutProj, kOutProj, kKvUp, kPrefill, kLinear, kQuant, kAbsorbFp8,
            kOutProjFp8, kRope, kMergeOutProjF32, kKinds };

volatile unsigned char g_sink;

void touch(const void* p, size_t bytes) {
  if (!p || bytes == 0) return;
  const volatile unsigned char* c = (const volatile unsigned char*)p;
  g_sink = c[0];
  g_sink = c[bytes - 1];
}

size_t elem(bool bf16) { return bf16 ? 2 : 4; }

}  // namespace

extern "C" {

hipError_t hipGetDevice(int* dev) {
  *dev = 0;
  return hipSuccess;
}

hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t attr, int dev) {
  (void)dev;
  if (attr != hipDeviceAttributeMultiprocessorCount) return hipErrorInvalidValue;
  *value = g_cus;
  return hipSuccess;
}

// compute units the stand-in device reports (split planning depends on it)
void san_set_cus(int n) { g_cus = n; }
long san_launches(int kind) { return kind >= 0 && kind < kKinds ? g_launches[kind] : -1; }
void san_reset() {
  for (long& c : g_launches) c = 0;
}

}  // extern "C"

namespace mla {

uint32_t* bounds_error_word() { return nullptr; }

hipError_t launch_decode_attn(const AttnArgs& a, int rows, hipStream_t) {
  ++g_launches[kAttn];
  const size_t e = elem(a.dtype_bf16);
  const size_t r = (size_t)rows;
  touch(a.q_lat, r * kHeads * kDc * e);
  touch(a.q_pe, r * kHeads * kDr * e);
  touch(a.seq_lens, (size_t)a.B * 4);
  touch(a.block_table, (size_t)a.B * a.max_pages * 4);
  if (a.tree_parents) touch(a.tree_parents, (size_t)a.B * a.S * 4);
  if (a.bounds.num_pages > 0) touch(a.pool, (size_t)a.bounds.num_pages * kPage * kRow * e);
  if (!a.final_out && (size_t)a.range_budget < r * a.num_splits) return hipErrorInvalidValue;
  const size_t out_rows = a.final_out ? r : (size_t)a.range_budget;
  touch(a.o_out, out_rows * kHeads * kDc * (a.final_out ? 4 : e));
  touch(a.lse_out, out_rows * kHeads * 4);
  if (!a.final_out) {  // the range plan: (first slot, count) of every row
    if (!a.row_plan) return hipErrorInvalidValue;
    touch(a.row_plan, 16 + r * 8);
  }
  return hipSuccess;
}

hipError_t launch_lse_merge(const void* o_part, bool part_bf16, const float* lse_part, const int32_t* row_plan,
                            float* o_lat, float* lse, int rows, int num_splits, int slots, hipStream_t) {
  ++g_launches[kLseMerge];
  if (slots < rows * num_splits) return hipErrorInvalidValue;
  const size_t n = (size_t)slots * kHeads;
  if (!row_plan) return hipErrorInvalidValue;
  touch(o_part, n * kDc * elem(part_bf16));
  touch(lse_part, n * 4);
  touch(row_plan, 16 + (size_t)rows * 8);
  touch(o_lat, (size_t)rows * kHeads * kDc * 4);
  touch(lse, (size_t)rows * kHeads * 4);
  return hipSuccess;
}

hipError_t launch_absorb_q(const void* q_nope, const void* w_uk, void* q_lat, int tokens, bool bf16, hipStream_t) {
  ++g_launches[kAbsorb];
  touch(q_nope, (size_t)tokens * kHeads * kDh * elem(bf16));
  touch(w_uk, (size_t)kHeads * kDc * kDh * elem(bf16));
  touch(q_lat, (size_t)tokens * kHeads * kDc * elem(bf16));
  return hipSuccess;
}

constexpr size_t kFp8Bytes = (size_t)kHeads * kDc * kDh + (size_t)kHeads * 4 * 4;

hipError_t launch_merge_out_proj(const void* o_part, const float* lse_part, const int32_t* row_plan, const void* w_uv,
                                 bool w_fp8, void* out, float* o_lat, float* lse, int rows, int num_splits,
                                 int slots, hipStream_t) {
  ++g_launches[kMergeOutProj];
  if (slots < rows * num_splits) return hipErrorInvalidValue;
  const size_t n = (size_t)slots * kHeads;
  if (!row_plan) return hipErrorInvalidValue;
  touch(o_part, n * kDc * 2);
  touch(lse_part, n * 4);
  touch(row_plan, 16 + (size_t)rows * 8);
  touch(w_uv, w_fp8 ? kFp8Bytes : (size_t)kHeads * kDc * kDh * 2);
  touch(out, (size_t)rows * kHeads * kDh * 2);
  touch(o_lat, (size_t)rows * kHeads * kDc * 4);
  touch(lse, (size_t)rows * kHeads * 4);
  return hipSuccess;
}

hipError_t launch_out_proj(const float* o_lat, const void* w_uv, void* out, int tokens, bool bf16, hipStream_t) {
  ++g_launches[kOutProj];
  touch(o_lat, (size_t)tokens * kHeads * kDc * 4);
  touch(w_uv, (size_t)kHeads * kDc * kDh * elem(bf16));
  touch(out, (size_t)tokens * kHeads * kDh * elem(bf16));
  return hipSuccess;
}

hipError_t launch_merge_out_proj_f32(const float* o_part, const float* lse_part, const int32_t* row_plan,
                                     const float* w_uv, float* out, float* o_lat, float* lse, int tokens, int num_splits,
                                     int slots, hipStream_t) {
  ++g_launches[kMergeOutProjF32];
  if (tokens > kGemvMergeTokens || slots < tokens * num_splits || !row_plan) return hipErrorInvalidValue;
  const size_t n = (size_t)slots * kHeads;
  touch(o_part, n * kDc * 4);
  touch(lse_part, n * 4);
  touch(row_plan, 16 + (size_t)tokens * 8);
  touch(w_uv, (size_t)kHeads * kDc * kDh * 4);
  touch(out, (size_t)tokens * kHeads * kDh * 4);
  touch(o_lat, (size_t)tokens * kHeads * kDc * 4);
  touch(lse, (size_t)tokens * kHeads * 4);
  return hipSuccess;
}

hipError_t launch_kv_up_grid(const void* pool, const int32_t* block_table, const int32_t* seq_lens,
                             const void* w_uk, const void* w_uv, void* kv, void* kpe, int batch, int max_pages,
                             int pages_max, const Bounds& bounds, hipStream_t) {
  ++g_launches[kKvUp];
  if (pages_max > max_pages) return hipErrorInvalidValue;  // the walk stays inside a table row
  const size_t Lp = (size_t)max_pages * kPage;
  touch(block_table, (size_t)batch * max_pages * 4);
  touch(seq_lens, (size_t)batch * 4);
  touch(w_uk, (size_t)kHeads * kDc * kDh * 2);
  touch(w_uv, (size_t)kHeads * kDc * kDh * 2);
  touch(kv, (size_t)batch * kHeads * Lp * 2 * kDh * 2);
  touch(kpe, (size_t)batch * Lp * kDr * 2);
  if (bounds.num_pages > 0) touch(pool, (size_t)bounds.num_pages * kPage * kRow * 2);
  return hipSuccess;
}

hipError_t launch_prefill_attn(const PrefillArgs& a, hipStream_t) {
  ++g_launches[kPrefill];
  const size_t t = (size_t)a.B * a.S;
  touch(a.q_nope, t * kHeads * kDh * 2);
  touch(a.q_pe, t * kHeads * kDr * 2);
  touch(a.kv, (size_t)a.B * kHeads * a.Lp * 2 * kDh * 2);
  touch(a.kpe, (size_t)a.B * a.Lp * kDr * 2);
  touch(a.seq_lens, (size_t)a.B * 4);
  touch(a.out, t * kHeads * kDh * 2);
  touch(a.lse, t * kHeads * 4);
  return hipSuccess;
}

hipError_t launch_linear(const void* x, const void* w, void* y, float* partial, int M, int K, int N, int splits,
                         hipStream_t) {
  ++g_launches[kLinear];
  touch(x, (size_t)M * K * 2);
  touch(w, (size_t)K * N * 2);
  touch(y, (size_t)M * N * 2);
  if (splits > 1) touch(partial, (size_t)splits * M * N * 4);
  return hipSuccess;
}

hipError_t launch_quantize_weight_fp8(const void* w, void* packed, bool, hipStream_t) {
  ++g_launches[kQuant];
  touch(w, (size_t)kHeads * kDc * kDh * 2);
  touch(packed, kFp8Bytes);
  return hipSuccess;
}

hipError_t launch_absorb_q_fp8(const void* q_nope, const void* packed, void* q_lat, int tokens, hipStream_t) {
  ++g_launches[kAbsorbFp8];
  touch(q_nope, (size_t)tokens * kHeads * kDh * 2);
  touch(packed, kFp8Bytes);
  touch(q_lat, (size_t)tokens * kHeads * kDc * 2);
  return hipSuccess;
}

hipError_t launch_out_proj_fp8(const float* o_lat, const void* packed, void* out, int tokens, hipStream_t) {
  ++g_launches[kOutProjFp8];
  touch(o_lat, (size_t)tokens * kHeads * kDc * 4);
  touch(packed, kFp8Bytes);
  touch(out, (size_t)tokens * kHeads * kDh * 2);
  return hipSuccess;
}

hipError_t launch_rope_append(void* q_pe, const void* kv_a, int kv_stride, void* pool, const int32_t* block_table,
                              const int32_t* seq_lens, int B, int S, int max_pages, double base,
                              const Bounds& bounds, hipStream_t) {
  ++g_launches[kRope];
  if (!(base > 0.0)) return hipErrorInvalidValue;
  const size_t t = (size_t)B * S;
  touch(q_pe, t * kHeads * kDr * 2);
  if (t) touch(kv_a, ((t - 1) * kv_stride + kRow) * 2);
  touch(block_table, (size_t)B * max_pages * 4);
  touch(seq_lens, (size_t)B * 4);
  if (bounds.num_pages > 0) touch(pool, (size_t)bounds.num_pages * kPage * kRow * 2);
  return hipSuccess;
}

}  // namespace mla
