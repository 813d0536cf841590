// C-ABI host layer: argument checks (all before any launch), key-split planning, workspace
// sizing and kernel dispatch.  Allocates nothing, never synchronises.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>

#include "../../include/mla_latent.h"
#include "attn_schedule.h"
#include "kernels.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];  // 0 = not queried yet (a cache, not state)

int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
  if (dev < kMaxDevices) {
    const int cached = g_cu_count[dev].load(std::memory_order_relaxed);
    if (cached > 0) return cached;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return -1;
  if (dev < kMaxDevices) g_cu_count[dev].store(n, std::memory_order_relaxed);
  return n;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

mla_status check_params(const mla_params* p) {
  if (!p) return MLA_ERR_NULL;
  if (p->dtype != MLA_F32 && p->dtype != MLA_BF16) return MLA_ERR_DTYPE;
  if (p->num_heads != mla::kHeads || p->kv_lora_rank != mla::kDc || p->rope_dim != mla::kDr ||
      p->head_dim != mla::kDh || p->page_size != mla::kPage)
    return MLA_ERR_UNSUPPORTED;
  if (p->batch < 0 || p->q_len < 1 || p->max_seq_len < 0 || p->max_pages_per_seq < 0 || p->num_pages < 0)
    return MLA_ERR_SHAPE;
  if ((int64_t)p->batch * p->q_len > (int64_t)(1 << 24)) return MLA_ERR_SHAPE;
  return MLA_OK;
}

int64_t tokens_of(const mla_params* p) { return (int64_t)p->batch * p->q_len; }

// Pages that max_seq_len tokens occupy (64-bit sum: max_seq_len may be INT32_MAX).
int pages_of(const mla_params* p) { return (int)(((int64_t)p->max_seq_len + mla::kPage - 1) / mla::kPage); }

// The table limits the kernels test in the bounds-checked build (mla::Bounds); that build needs
// the device's error word, the other one passes the limits along unused.
mla_status table_bounds(const mla_params* p, mla::Bounds* b) {
  b->err = mla::bounds_error_word();
  b->max_seq_len = p->max_seq_len;
  b->num_pages = p->num_pages;
#ifdef MLA_DEBUG_BOUNDS
  if (!b->err) return MLA_ERR_DEVICE;
#endif
  return MLA_OK;
}

// K splits of mla_linear: the fewest that give at least 7/8 of a workgroup per compute unit (more
// splits only add partial traffic and a second workgroup per unit, which measured slower); every
// split keeps >= 4 chunks of 64.
int linear_splits(int M, int K, int N, int cus) {
  const int mb = M >= 512 ? 4 : 1;
  const int tiles = ((M + 32 * mb - 1) / (32 * mb)) * (N / 64);
  int s = 1;
  while (8 * tiles * s < 7 * cus && (K / (s * 2)) % 64 == 0 && K / (s * 2) >= 256) s *= 2;
  return s;
}

// Split planning: one workgroup per (b, i, split); aim for about one workgroup per compute unit
// (each holds a CU: 128 heads of accumulators and two 72 KiB LDS tiles) with page-aligned,
// equal page ranges and no trailing empty split.
struct SplitPlan {
  int splits, pages_per_split;
  int64_t slots;  // key ranges the device plan may use = partial slots = attention workgroups (bf16)
};

SplitPlan plan_splits(const mla_params* p, int requested, int cus) {
  const int max_pages = pages_of(p);
  const int64_t rows = tokens_of(p);
  int s = requested;
  if (s <= 0) {
    if (max_pages <= 1 || rows <= 0) {
      s = 1;
    } else {
      const int64_t want = (cus + rows - 1) / rows;
      s = (int)(want < max_pages ? want : max_pages);
      if (s < 1) s = 1;
    }
  }
  if (max_pages == 0) return {1, 1, rows};
  if (s > max_pages) s = max_pages;
  // a workgroup stages its range's page ids in LDS: at most kMaxSplitPages pages per split
  const int min_splits = (max_pages + mla::kMaxSplitPages - 1) / mla::kMaxSplitPages;
  if (s < min_splits) s = min_splits;
  const int pps = (max_pages + s - 1) / s;
  s = (max_pages + pps - 1) / pps;
  // With the library's choice of splits, bf16, and 33..kPlanRows query rows, rows of unequal length
  // may take up to 9/8 of a key range per compute unit, dispatched longest first: the eighth past
  // the first wave fills the units whose first range was short (decode_attn.hip, plan_ranges).
  // More, shorter ranges measured slower (each pays a workgroup's fixed cost).  Rows of equal
  // length still use rows * s of them (the rest exit); 32 rows or fewer keep exactly rows * s
  // workgroups.
  int64_t slots = rows * s;
  if (requested <= 0 && p->dtype == MLA_BF16 && s > 1 && rows > 32 && rows <= mla::kPlanRows) {
    const int64_t want = (9 * (int64_t)cus + 7) / 8;
    if (slots < want) slots = want;
  }
  return {s, pps, slots};
}

// Split partials: o (rows, splits, H, d_c) in the input dtype (bf16 partials carry 8 mantissa bits,
// far inside the bf16 tolerance; they halve the bytes written and merged), then lse (rows, splits, H)
// fp32.  The o block is a multiple of 16 bytes, so lse stays aligned.
size_t part_elem_bytes(const mla_params* p) { return p->dtype == MLA_BF16 ? 2 : 4; }

// After them the key-range plan: a 16-byte header (word 0: every row has the fixed slots), then
// (first slot, number of ranges) per row, padded to 16 bytes.
size_t row_plan_bytes(const mla_params* p) { return 16 + ((size_t)tokens_of(p) * 8 + 15) / 16 * 16; }

size_t workspace_for(const mla_params* p, const SplitPlan& plan) {
  if (plan.splits <= 1) return 0;
  const size_t n = (size_t)plan.slots * mla::kHeads;
  return n * mla::kDc * part_elem_bytes(p) + n * sizeof(float) + row_plan_bytes(p);
}

// mla_decode_attn_out_proj: with at least one 16-row block of query rows and more than one split,
// the merge runs inside the W_UV kernel, which reads the bf16 partials.  With fewer rows most of
// that kernel's lanes would idle while each walks every split, and with one split there is no
// merge to save (the attention writes o_lat itself), so the call then takes the separate kernels,
// with o_lat in the workspace after any partials when the caller wants none.  In fp32, with at most
// kGemvMergeTokens query rows and more than one split, the merge runs inside the out-projection
// GEMV (fp32 partials), which saves the separate merge launch.
bool merge_in_out_proj(const mla_params* p, int splits) {
  return p->dtype == MLA_BF16 && tokens_of(p) >= 16 && splits > 1;
}
bool merge_in_gemv(const mla_params* p, int splits) {
  return p->dtype == MLA_F32 && tokens_of(p) <= mla::kGemvMergeTokens && splits > 1;
}

size_t fused_workspace_for(const mla_params* p, const SplitPlan& plan) {
  if (merge_in_out_proj(p, plan.splits)) {
    const size_t n = (size_t)plan.slots * mla::kHeads;
    return n * mla::kDc * 2 + n * sizeof(float) + row_plan_bytes(p);
  }
  if (merge_in_gemv(p, plan.splits)) return workspace_for(p, plan);
  return workspace_for(p, plan) + (size_t)tokens_of(p) * mla::kHeads * mla::kDc * sizeof(float);
}

// Prefill buffer: [K_nope | V] (B, H, Lp, 256) then k_pe (B, Lp, 64), bf16, Lp = max_pages * page.
size_t prefill_kv_bytes(const mla_params* p) {
  const size_t Lp = (size_t)p->max_pages_per_seq * mla::kPage;
  return (size_t)p->batch * Lp * ((size_t)mla::kHeads * 2 * mla::kDh + mla::kDr) * 2;
}

mla_status check_prefill(const mla_params* p) {
  mla_status st = check_params(p);
  if (st != MLA_OK) return st;
  if (p->dtype != MLA_BF16) return MLA_ERR_DTYPE;
  const int max_pages = pages_of(p);
  if (p->max_pages_per_seq < max_pages) return MLA_ERR_SHAPE;
  // the kv buffer holds B x (max_pages_per_seq x 64) rows per head: keep its size far from overflow
  if ((int64_t)p->batch * p->max_pages_per_seq > 0x7fffffffLL / mla::kPage) return MLA_ERR_SHAPE;
  return MLA_OK;
}

mla_status check_linear(int32_t m, int32_t k, int32_t n) {
  if (m < 0 || k <= 0 || n <= 0 || k % 64 != 0 || n % 64 != 0) return MLA_ERR_SHAPE;
  if ((int64_t)m * k * 2 >= (int64_t)1 << 32 || (int64_t)k * n * 2 >= (int64_t)1 << 32) return MLA_ERR_SHAPE;
  return MLA_OK;
}

}  // namespace

extern "C" {

const char* mla_status_str(mla_status s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_NULL: return "MLA_ERR_NULL: a required pointer is NULL";
    case MLA_ERR_SHAPE: return "MLA_ERR_SHAPE: a size is out of range";
    case MLA_ERR_DTYPE: return "MLA_ERR_DTYPE: dtype not supported by this call (MLA_F32 or MLA_BF16; prefill and the FP8 calls: MLA_BF16 only)";
    case MLA_ERR_ALIGN: return "MLA_ERR_ALIGN: pointers must be 16-byte aligned";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace too small";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: only H=128, d_c=512, d_R=64, d_h=128, page 64";
    case MLA_ERR_LAUNCH: return "MLA_ERR_LAUNCH: kernel launch failed";
    case MLA_ERR_DEVICE: return "MLA_ERR_DEVICE: no usable HIP device";
    case MLA_ERR_SCRATCH: return "MLA_ERR_SCRATCH: the call needs more than MLA_STATIC_SCRATCH_BYTES of static scratch";
  }
  return "unknown mla_status";
}

mla_status mla_absorb_q(const void* q_nope, const void* w_uk, void* q_lat, const mla_params* p, void* stream) {
  mla_status st = check_params(p);
  if (st != MLA_OK) return st;
  if (tokens_of(p) == 0) return MLA_OK;
  if (!q_nope || !w_uk || !q_lat) return MLA_ERR_NULL;
  if (!aligned16(q_nope) || !aligned16(w_uk) || !aligned16(q_lat)) return MLA_ERR_ALIGN;
  if (mla::launch_absorb_q(q_nope, w_uk, q_lat, (int)tokens_of(p), p->dtype == MLA_BF16, (hipStream_t)stream) !=
      hipSuccess)
    return MLA_ERR_LAUNCH;
  return MLA_OK;
}

int32_t mla_decode_num_splits(const mla_params* p, int32_t num_splits) {
  mla_status st = check_params(p);
  if (st != MLA_OK) return st;
  if (num_splits < 0) return MLA_ERR_SHAPE;
  const int cus = num_splits > 0 ? 1 : cu_count();
  if (cus <= 0) return MLA_ERR_DEVICE;
  return plan_splits(p, num_splits, cus).splits;
}

size_t mla_decode_workspace_bytes(const mla_params* p, int32_t num_splits) {
  const int32_t s = mla_decode_num_splits(p, num_splits);
  // more (row, split) workgroups than a grid holds: the call rejects it (MLA_ERR_SHAPE)
  if (s <= 0 || tokens_of(p) * s > 0x7fffffffLL) return 0;
  return workspace_for(p, plan_splits(p, num_splits, num_splits > 0 ? 1 : cu_count()));
}

}  // extern "C"

namespace {

// mla_decode_attn and mla_decode_attn_tree: `tree_parents` null = the causal / full rule of p.
// With w_uv and out (the fused route): the split partials are merged and projected by W_UV in one
// kernel; o_lat and lse are then optional outputs.
mla_status decode_attn_impl(const void* q_lat, const void* q_pe, const void* kv_pool, const int32_t* block_table,
                            const int32_t* seq_lens, const int32_t* tree_parents, float* o_lat, float* lse,
                            void* workspace, size_t workspace_bytes, int32_t num_splits, const mla_params* p,
                            void* stream, const void* w_uv = nullptr, void* out = nullptr, bool w_fp8 = false) {
  const bool fused = w_uv != nullptr || out != nullptr;
  mla_status st = check_params(p);
  if (st != MLA_OK) return st;
  if (num_splits < 0) return MLA_ERR_SHAPE;
  const int max_pages = pages_of(p);
  if (p->max_pages_per_seq < max_pages) return MLA_ERR_SHAPE;
  if (fused && w_fp8 && p->dtype != MLA_BF16) return MLA_ERR_DTYPE;
  if (tokens_of(p) == 0) return MLA_OK;
  if (!q_lat || !q_pe || !seq_lens || (!fused && !o_lat)) return MLA_ERR_NULL;
  if (fused && (!w_uv || !out)) return MLA_ERR_NULL;
  if (max_pages > 0 && (!kv_pool || !block_table)) return MLA_ERR_NULL;
  if (!aligned16(q_lat) || !aligned16(q_pe) || !aligned16(kv_pool) || !aligned16(o_lat)) return MLA_ERR_ALIGN;
  if (fused && (!aligned16(w_uv) || !aligned16(out))) return MLA_ERR_ALIGN;
  // the kernels take a tile's maximum before scaling: the scale must be positive
  if (!std::isfinite(p->softmax_scale) || !(p->softmax_scale > 0.f)) return MLA_ERR_SHAPE;
  const int cus = num_splits > 0 ? 1 : cu_count();
  if (cus <= 0) return MLA_ERR_DEVICE;
  mla::Bounds bounds;
  st = table_bounds(p, &bounds);
  if (st != MLA_OK) return st;
  const SplitPlan plan = plan_splits(p, num_splits, cus);
  const int64_t grid = tokens_of(p) * plan.splits * (p->dtype == MLA_BF16 ? 1 : mla::kHeads / mla::kF32Heads);
  if (grid > 0x7fffffffLL) return MLA_ERR_SHAPE;
  const size_t need = fused ? fused_workspace_for(p, plan) : workspace_for(p, plan);
  const bool merge_in_proj = fused && merge_in_out_proj(p, plan.splits);
  const bool merge_gemv = fused && merge_in_gemv(p, plan.splits);
  if (need > 0) {
    if (!workspace) return MLA_ERR_NULL;
    if (workspace_bytes < need) return MLA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MLA_ERR_ALIGN;
  }
  if (fused && !merge_in_proj && !merge_gemv) {  // the separate merge and out-projection, o_lat maybe in the workspace
    float* o = o_lat ? o_lat : (float*)((char*)workspace + workspace_for(p, plan));
    st = decode_attn_impl(q_lat, q_pe, kv_pool, block_table, seq_lens, tree_parents, o, lse, workspace,
                          workspace_bytes, num_splits, p, stream);
    if (st != MLA_OK) return st;
    const hipError_t e = w_fp8 ? mla::launch_out_proj_fp8(o, w_uv, out, (int)tokens_of(p), (hipStream_t)stream)
                               : mla::launch_out_proj(o, w_uv, out, (int)tokens_of(p), p->dtype == MLA_BF16,
                                                      (hipStream_t)stream);
    return e == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
  }

  mla::AttnArgs a;
  a.q_lat = q_lat;
  a.q_pe = q_pe;
  a.pool = kv_pool;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.tree_parents = tree_parents;
  a.B = p->batch;
  a.S = p->q_len;
  a.max_pages = p->max_pages_per_seq;
  a.pages_per_split = plan.pages_per_split;
  a.num_splits = plan.splits;
  a.range_budget = (int)plan.slots;
  a.causal = p->causal ? 1 : 0;
  a.dtype_bf16 = p->dtype == MLA_BF16;
  a.scale = p->softmax_scale;
  a.scale_log2 = (float)((double)p->softmax_scale * 1.4426950408889634);
  a.bounds = bounds;
  const int rows = (int)tokens_of(p);
  hipStream_t s = (hipStream_t)stream;
  if (plan.splits == 1 && !merge_in_proj) {
    a.o_out = o_lat;
    a.lse_out = lse;
    a.row_plan = nullptr;
    a.final_out = 1;
    if (mla::launch_decode_attn(a, rows, s) != hipSuccess) return MLA_ERR_LAUNCH;
    return MLA_OK;
  }
  char* o_part = (char*)workspace;
  const size_t nslots = (size_t)plan.slots * mla::kHeads;
  float* lse_part = (float*)(o_part + nslots * mla::kDc * part_elem_bytes(p));
  int32_t* row_plan = (int32_t*)(lse_part + nslots);
  a.o_out = o_part;
  a.lse_out = lse_part;
  a.row_plan = row_plan;
  a.final_out = 0;
  if (mla::launch_decode_attn(a, rows, s) != hipSuccess) return MLA_ERR_LAUNCH;
  if (merge_in_proj) {
    if (mla::launch_merge_out_proj(o_part, lse_part, row_plan, w_uv, w_fp8, out, o_lat, lse, rows, plan.splits,
                                   (int)plan.slots, s) !=
        hipSuccess)
      return MLA_ERR_LAUNCH;
    return MLA_OK;
  }
  if (merge_gemv) {
    if (mla::launch_merge_out_proj_f32((const float*)o_part, lse_part, row_plan, (const float*)w_uv, (float*)out,
                                       o_lat, lse, rows, plan.splits, (int)plan.slots, s) != hipSuccess)
      return MLA_ERR_LAUNCH;
    return MLA_OK;
  }
  if (mla::launch_lse_merge(o_part, p->dtype == MLA_BF16, lse_part, row_plan, o_lat, lse, rows, plan.splits,
                            (int)plan.slots, s) !=
      hipSuccess)
    return MLA_ERR_LAUNCH;
  return MLA_OK;
}

}  // namespace

extern "C" {

mla_status mla_decode_attn(const void* q_lat, const void* q_pe, const void* kv_pool, const int32_t* block_table,
                           const int32_t* seq_lens, float* o_lat, float* lse, void* workspace,
                           size_t workspace_bytes, int32_t num_splits, const mla_params* p, void* stream) {
  return decode_attn_impl(q_lat, q_pe, kv_pool, block_table, seq_lens, nullptr, o_lat, lse, workspace,
                          workspace_bytes, num_splits, p, stream);
}

mla_status mla_decode_attn_tree(const void* q_lat, const void* q_pe, const void* kv_pool,
                                const int32_t* block_table, const int32_t* seq_lens, const int32_t* tree_parents,
                                float* o_lat, float* lse, void* workspace, size_t workspace_bytes,
                                int32_t num_splits, const mla_params* p, void* stream) {
  mla_status st = check_params(p);
  if (st != MLA_OK) return st;
  if (p->q_len > 64) return MLA_ERR_SHAPE;  // one 64-bit visibility mask per query row
  if (tokens_of(p) > 0 && !tree_parents) return MLA_ERR_NULL;
  return decode_attn_impl(q_lat, q_pe, kv_pool, block_table, seq_lens, tree_parents, o_lat, lse, workspace,
                          workspace_bytes, num_splits, p, stream);
}

size_t mla_decode_attn_out_proj_workspace_bytes(const mla_params* p, int32_t num_splits) {
  const int32_t s = mla_decode_num_splits(p, num_splits);
  if (s <= 0 || tokens_of(p) * s > 0x7fffffffLL) return 0;
  return fused_workspace_for(p, plan_splits(p, num_splits, num_splits > 0 ? 1 : cu_count()));
}

mla_status mla_decode_attn_out_proj(const void* q_lat, const void* q_pe, const void* kv_pool,
                                    const int32_t* block_table, const int32_t* seq_lens,
                                    const int32_t* tree_parents, const void* w_uv, void* out, float* o_lat,
                                    float* lse, void* workspace, size_t workspace_bytes, int32_t num_splits,
                                    const mla_params* p, void* stream) {
  mla_status st = check_params(p);
  if (st != MLA_OK) return st;
  if (tree_parents && p->q_len > 64) return MLA_ERR_SHAPE;  // one 64-bit visibility mask per query row
  if (!w_uv || !out) return tokens_of(p) == 0 ? MLA_OK : MLA_ERR_NULL;
  return decode_attn_impl(q_lat, q_pe, kv_pool, block_table, seq_lens, tree_parents, o_lat, lse, workspace,
                          workspace_bytes, num_splits, p, stream, w_uv, out);
}

mla_status mla_decode_attn_out_proj_fp8(const void* q_lat, const void* q_pe, const void* kv_pool,
                                        const int32_t* block_table, const int32_t* seq_lens,
                                        const int32_t* tree_parents, const void* w_uv_fp8, void* out, float* o_lat,
                                        float* lse, void* workspace, size_t workspace_bytes, int32_t num_splits,
                                        const mla_params* p, void* stream) {
  mla_status st = check_params(p);
  if (st != MLA_OK) return st;
  if (tree_parents && p->q_len > 64) return MLA_ERR_SHAPE;
  if (!w_uv_fp8 || !out) return tokens_of(p) == 0 ? MLA_OK : MLA_ERR_NULL;
  return decode_attn_impl(q_lat, q_pe, kv_pool, block_table, seq_lens, tree_parents, o_lat, lse, workspace,
                          workspace_bytes, num_splits, p, stream, w_uv_fp8, out, true);
}

mla_status mla_out_proj(const float* o_lat, const void* w_uv, void* out, const mla_params* p, void* stream) {
  mla_status st = check_params(p);
  if (st != MLA_OK) return st;
  if (tokens_of(p) == 0) return MLA_OK;
  if (!o_lat || !w_uv || !out) return MLA_ERR_NULL;
  if (!aligned16(o_lat) || !aligned16(w_uv) || !aligned16(out)) return MLA_ERR_ALIGN;
  if (mla::launch_out_proj(o_lat, w_uv, out, (int)tokens_of(p), p->dtype == MLA_BF16, (hipStream_t)stream) !=
      hipSuccess)
    return MLA_ERR_LAUNCH;
  return MLA_OK;
}

size_t mla_prefill_kv_bytes(const mla_params* p) {
  if (check_prefill(p) != MLA_OK) return 0;
  return prefill_kv_bytes(p);
}

mla_status mla_prefill_kv_up(const void* kv_pool, const int32_t* block_table, const int32_t* seq_lens,
                             const void* w_uk, const void* w_uv, void* kv, size_t kv_bytes, const mla_params* p,
                             void* stream) {
  mla_status st = check_prefill(p);
  if (st != MLA_OK) return st;
  const int pages = pages_of(p);
  if (p->batch == 0 || pages == 0) return MLA_OK;
  if (!kv_pool || !block_table || !seq_lens || !w_uk || !w_uv || !kv) return MLA_ERR_NULL;
  if (!aligned16(kv_pool) || !aligned16(w_uk) || !aligned16(w_uv) || !aligned16(kv)) return MLA_ERR_ALIGN;
  if (kv_bytes < prefill_kv_bytes(p)) return MLA_ERR_WORKSPACE;
  if ((int64_t)p->batch * pages > 0x7fffffffLL) return MLA_ERR_SHAPE;
  mla::Bounds bounds;
  st = table_bounds(p, &bounds);
  if (st != MLA_OK) return st;
  char* kpe = (char*)kv + (size_t)p->batch * mla::kHeads * p->max_pages_per_seq * mla::kPage * 2 * mla::kDh * 2;
  // the walk covers the pages max_seq_len needs; rows are laid out with the table's page stride
  if (mla::launch_kv_up_grid(kv_pool, block_table, seq_lens, w_uk, w_uv, kv, kpe, p->batch, p->max_pages_per_seq,
                             pages, bounds, (hipStream_t)stream) != hipSuccess)
    return MLA_ERR_LAUNCH;
  return MLA_OK;
}

mla_status mla_prefill_attn(const void* q_nope, const void* q_pe, const void* kv, size_t kv_bytes,
                            const int32_t* seq_lens, void* out, float* lse, const mla_params* p, void* stream) {
  mla_status st = check_prefill(p);
  if (st != MLA_OK) return st;
  if (tokens_of(p) == 0) return MLA_OK;
  if (!q_nope || !q_pe || !seq_lens || !out) return MLA_ERR_NULL;
  if (p->max_seq_len > 0 && !kv) return MLA_ERR_NULL;
  if (!aligned16(q_nope) || !aligned16(q_pe) || !aligned16(kv) || !aligned16(out)) return MLA_ERR_ALIGN;
  if (!std::isfinite(p->softmax_scale) || !(p->softmax_scale > 0.f)) return MLA_ERR_SHAPE;  // as decode
  if (p->max_seq_len > 0 && kv_bytes < prefill_kv_bytes(p)) return MLA_ERR_WORKSPACE;
  const int nqb = (p->q_len + 255) / 256;  // 256 queries per workgroup
  if ((int64_t)p->batch * mla::kHeads * nqb > 0x7fffffffLL) return MLA_ERR_SHAPE;
  mla::PrefillArgs a;
  st = table_bounds(p, &a.bounds);
  if (st != MLA_OK) return st;
  a.q_nope = q_nope;
  a.q_pe = q_pe;
  a.kv = kv;
  a.kpe = kv ? (const char*)kv + (size_t)p->batch * mla::kHeads * p->max_pages_per_seq * mla::kPage * 2 * mla::kDh * 2
             : nullptr;
  a.seq_lens = seq_lens;
  a.out = out;
  a.lse = lse;
  a.B = p->batch;
  a.S = p->q_len;
  a.Lp = p->max_pages_per_seq * mla::kPage;
  a.nqb = nqb;
  a.causal = p->causal ? 1 : 0;
  a.scale_log2 = (float)((double)p->softmax_scale * 1.4426950408889634);
  if (mla::launch_prefill_attn(a, (hipStream_t)stream) != hipSuccess) return MLA_ERR_LAUNCH;
  return MLA_OK;
}

size_t mla_linear_workspace_bytes(int32_t m, int32_t k, int32_t n) {
  if (check_linear(m, k, n) != MLA_OK || m == 0) return 0;
  const int cus = cu_count();
  if (cus <= 0) return 0;
  const int s = linear_splits(m, k, n, cus);
  return s > 1 ? (size_t)s * m * n * sizeof(float) : 0;
}

mla_status mla_linear(const void* x, const void* w, void* y, int32_t m, int32_t k, int32_t n, void* workspace,
                      size_t workspace_bytes, void* stream) {
  mla_status st = check_linear(m, k, n);
  if (st != MLA_OK) return st;
  if (m == 0) return MLA_OK;
  if (!x || !w || !y) return MLA_ERR_NULL;
  if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return MLA_ERR_ALIGN;
  const int cus = cu_count();
  if (cus <= 0) return MLA_ERR_DEVICE;
  const int splits = linear_splits(m, k, n, cus);
  if (splits > 1) {
    if (!workspace) return MLA_ERR_NULL;
    if (workspace_bytes < (size_t)splits * m * n * sizeof(float)) return MLA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MLA_ERR_ALIGN;
  }
  if (mla::launch_linear(x, w, y, (float*)workspace, m, k, n, splits, (hipStream_t)stream) != hipSuccess)
    return MLA_ERR_LAUNCH;
  return MLA_OK;
}

mla_status mla_rope_append(void* q_pe, const void* kv_a, int32_t kv_a_stride, void* kv_pool,
                           const int32_t* block_table, const int32_t* seq_lens, float rope_base, const mla_params* p,
                           void* stream) {
  mla_status st = check_params(p);
  if (st != MLA_OK) return st;
  if (p->dtype != MLA_BF16) return MLA_ERR_DTYPE;
  const int max_pages = pages_of(p);
  if (p->max_pages_per_seq < max_pages) return MLA_ERR_SHAPE;
  if (kv_a_stride < mla::kRow || kv_a_stride % 8 != 0) return MLA_ERR_SHAPE;
  if (!(rope_base > 0.f) || !std::isfinite(rope_base)) return MLA_ERR_SHAPE;
  if (tokens_of(p) == 0) return MLA_OK;
  if (!q_pe || !kv_a || !kv_pool || !block_table || !seq_lens) return MLA_ERR_NULL;
  if (!aligned16(q_pe) || !aligned16(kv_a) || !aligned16(kv_pool)) return MLA_ERR_ALIGN;
  mla::Bounds bounds;
  st = table_bounds(p, &bounds);
  if (st != MLA_OK) return st;
  if (mla::launch_rope_append(q_pe, kv_a, kv_a_stride, kv_pool, block_table, seq_lens, p->batch, p->q_len,
                              p->max_pages_per_seq, (double)rope_base, bounds, (hipStream_t)stream) != hipSuccess)
    return MLA_ERR_LAUNCH;
  return MLA_OK;
}

size_t mla_fp8_weight_bytes(void) {
  return (size_t)mla::kHeads * mla::kDc * mla::kDh + (size_t)mla::kHeads * 4 * sizeof(float);
}

static mla_status quantize_fp8(const void* w, void* packed, size_t packed_bytes, const mla_params* p, bool transpose,
                               void* stream) {
  mla_status st = check_params(p);
  if (st != MLA_OK) return st;
  if (p->dtype != MLA_BF16) return MLA_ERR_DTYPE;
  if (!w || !packed) return MLA_ERR_NULL;
  if (!aligned16(w) || !aligned16(packed)) return MLA_ERR_ALIGN;
  if (packed_bytes < mla_fp8_weight_bytes()) return MLA_ERR_WORKSPACE;
  if (mla::launch_quantize_weight_fp8(w, packed, transpose, (hipStream_t)stream) != hipSuccess) return MLA_ERR_LAUNCH;
  return MLA_OK;
}

mla_status mla_quantize_w_uk_fp8(const void* w_uk, void* packed, size_t packed_bytes, const mla_params* p,
                                 void* stream) {
  return quantize_fp8(w_uk, packed, packed_bytes, p, false, stream);
}

mla_status mla_quantize_w_uv_fp8(const void* w_uv, void* packed, size_t packed_bytes, const mla_params* p,
                                 void* stream) {
  return quantize_fp8(w_uv, packed, packed_bytes, p, true, stream);
}

mla_status mla_absorb_q_fp8(const void* q_nope, const void* w_uk_fp8, void* q_lat, const mla_params* p,
                            void* stream) {
  mla_status st = check_params(p);
  if (st != MLA_OK) return st;
  if (p->dtype != MLA_BF16) return MLA_ERR_DTYPE;
  if (tokens_of(p) == 0) return MLA_OK;
  if (!q_nope || !w_uk_fp8 || !q_lat) return MLA_ERR_NULL;
  if (!aligned16(q_nope) || !aligned16(w_uk_fp8) || !aligned16(q_lat)) return MLA_ERR_ALIGN;
  if (mla::launch_absorb_q_fp8(q_nope, w_uk_fp8, q_lat, (int)tokens_of(p), (hipStream_t)stream) != hipSuccess)
    return MLA_ERR_LAUNCH;
  return MLA_OK;
}

mla_status mla_out_proj_fp8(const float* o_lat, const void* w_uv_fp8, void* out, const mla_params* p, void* stream) {
  mla_status st = check_params(p);
  if (st != MLA_OK) return st;
  if (p->dtype != MLA_BF16) return MLA_ERR_DTYPE;
  if (tokens_of(p) == 0) return MLA_OK;
  if (!o_lat || !w_uv_fp8 || !out) return MLA_ERR_NULL;
  if (!aligned16(o_lat) || !aligned16(w_uv_fp8) || !aligned16(out)) return MLA_ERR_ALIGN;
  if (mla::launch_out_proj_fp8(o_lat, w_uv_fp8, out, (int)tokens_of(p), (hipStream_t)stream) != hipSuccess)
    return MLA_ERR_LAUNCH;
  return MLA_OK;
}

mla_status mla_debug_attn_schedule(int32_t ntiles, int32_t* a_buffer, int32_t* b_buffer, int32_t* p_buffer) {
  if (ntiles < 1) return MLA_ERR_SHAPE;
  if (!a_buffer || !b_buffer || !p_buffer) return MLA_ERR_NULL;
  for (int u = 0; u < ntiles; ++u) {
    a_buffer[u] = mla::attn_a_buffer(u + mla::kLoadAhead);
    b_buffer[u] = mla::attn_b_buffer(u + mla::kLoadAhead);
    p_buffer[u] = mla::attn_p_buffer(u);
  }
  return MLA_OK;
}

}  // extern "C"
