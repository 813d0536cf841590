// Launch interface between the C-ABI host layer and the HIP kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

// Fixed head geometry of the DeepSeek-V2/V3 MLA layer the kernels are specialised for.
constexpr int kHeads = 128;   // query heads: the M dimension of the attention MFMAs
constexpr int kDc = 512;      // latent width (kv_lora_rank)
constexpr int kDr = 64;       // shared RoPE key width
constexpr int kRow = 576;     // cached row: [c_KV | k_pe]
constexpr int kDh = 128;      // no-RoPE head dim = value head dim
constexpr int kPage = 64;     // tokens per cache page
constexpr int kMaxSplitPages = 512;  // pages one attention workgroup may walk (32768 tokens)
constexpr int kF32Heads = 16;  // heads per workgroup of the fp32 attention kernel

// Preconditions on the page table that only the device can check.  In the bounds-checked build
// (MLA_DEBUG_BOUNDS) every kernel that walks the table tests each seq_lens entry it uses against
// [0, max_seq_len] and each page id against [0, num_pages) (num_pages 0: only negative ids are
// caught); a violation sets its bit in err[0], counts in err[1], and the kernel goes on with a safe
// value instead (the length clamped; a read from page 0; no write).  err is the device address of
// the library's error word (bounds_error_word); the other build carries the fields and tests nothing.
struct Bounds {
  uint32_t* err;
  int max_seq_len, num_pages;
};
constexpr uint32_t kBoundsBadSeqLen = 1u;  // a seq_lens entry outside [0, max_seq_len]
constexpr uint32_t kBoundsBadPage = 2u;    // a block_table entry outside [0, num_pages)
// Device address of the error word on the current device (bounds-checked build), else null.
uint32_t* bounds_error_word();

struct AttnArgs {
  const void* q_lat;           // (B,S,H,512) bf16 or fp32
  const void* q_pe;            // (B,S,H,64)
  const void* pool;            // (P,64,576)
  const int32_t* block_table;  // (B,max_pages)
  const int32_t* seq_lens;     // (B)
  void* o_out;                 // final o_lat (B,S,H,512) fp32, or partials (B*S, splits, H, 512):
                               // bf16 for the bf16 kernel, fp32 for the fp32 kernel
  float* lse_out;              // final lse (B,S,H) (may be null), or partial lse (B*S, splits, H)
  const int32_t* tree_parents;  // (B,S) draft-tree parents in [-1, j), or null (then `causal` applies)
  // With num_splits > 1: word 0 = 1 if every row r has the fixed slots r * num_splits + j, then
  // from word 4 (first partial slot, number of key ranges) of each row; written by the attention
  // (range j of row r goes to slot first + j) and read by the merges; null otherwise.
  int32_t* row_plan;
  int B, S, max_pages, pages_per_split, num_splits, causal, final_out, dtype_bf16;
  // Key ranges (and partial slots, and workgroups) the plan may use: B * S * num_splits, or more
  // when ranges of rows of unequal length are dispatched longest first (see plan_ranges)
  int range_budget;
  float scale;       // softmax scale
  float scale_log2;  // softmax scale * log2(e)
  Bounds bounds;
};

// Key ranges with num_splits > 1: up to this many rows the ranges follow the rows' lengths (see
// the key-range plan in decode_attn.hip); above it every row gets num_splits fixed ranges.
constexpr int kPlanRows = 256;

// decode attention over rows = B*S (b, i) pairs; range_budget workgroups (bf16; at least rows *
// num_splits), rows * num_splits * 8 for fp32
hipError_t launch_decode_attn(const AttnArgs& a, int rows, hipStream_t stream);
// merge of the partial slots (`slots` of H rows, bf16 or fp32; at least rows * num_splits) into
// o_lat (rows, H, 512) and lse (rows, H) (lse may be null); row_plan gives each row's slots
hipError_t launch_lse_merge(const void* o_part, bool part_bf16, const float* lse_part, const int32_t* row_plan,
                            float* o_lat, float* lse, int rows, int num_splits, int slots, hipStream_t stream);
// q_lat[n,h,:] = W_UK[h] q_nope[n,h,:] for n < tokens
hipError_t launch_absorb_q(const void* q_nope, const void* w_uk, void* q_lat, int tokens, bool bf16,
                           hipStream_t stream);
// out[n,h,:] = W_UV[h]^T o_lat[n,h,:] for n < tokens
// Split merge + out-proj in one kernel (bf16 partials; W_UV bf16, or with w_fp8 the packed FP8 codes
// and scales of launch_quantize_weight_fp8; o_lat and lse optional).
hipError_t launch_merge_out_proj(const void* o_part, const float* lse_part, const int32_t* row_plan, const void* w_uv,
                                 bool w_fp8, void* out, float* o_lat, float* lse, int rows, int num_splits,
                                 int slots, hipStream_t stream);
hipError_t launch_out_proj(const float* o_lat, const void* w_uv, void* out, int tokens, bool bf16,
                           hipStream_t stream);
// fp32, at most kGemvMergeTokens query rows: the split merge (fp32 partials, `slots` of them, each
// row's from row_plan) inside the out-projection GEMV; o_lat and lse optional
constexpr int kGemvMergeTokens = 4;
hipError_t launch_merge_out_proj_f32(const float* o_part, const float* lse_part, const int32_t* row_plan,
                                     const float* w_uv, float* out, float* o_lat, float* lse, int tokens, int num_splits,
                                     int slots, hipStream_t stream);

// Prefill in multi-head form (bf16).  kv (B,H,Lp,256) = [K_nope | V] per head and token and
// kpe (B,Lp,64) = the shared RoPE key, Lp = max_pages * 64; rows from seq_lens[b] up to the end of
// its last page are zeros.
// One workgroup per (head, K or V) walks pages [0, pages_max) of every sequence; max_pages is the
// block-table row stride.
hipError_t launch_kv_up_grid(const void* pool, const int32_t* block_table, const int32_t* seq_lens,
                             const void* w_uk, const void* w_uv, void* kv, void* kpe, int batch, int max_pages,
                             int pages_max, const Bounds& bounds, hipStream_t stream);

struct PrefillArgs {
  const void* q_nope;  // (B,S,H,128) bf16
  const void* q_pe;    // (B,S,H,64) bf16
  const void* kv;      // (B,H,Lp,256) bf16
  const void* kpe;     // (B,Lp,64) bf16
  const int32_t* seq_lens;
  void* out;           // (B,S,H,128) bf16
  float* lse;          // (B,S,H) or null
  int B, S, Lp, nqb, causal;
  float scale_log2;    // softmax scale * log2(e)
  Bounds bounds;
};
hipError_t launch_prefill_attn(const PrefillArgs& a, hipStream_t stream);

// y (M x N) = x (M x K) W (K x N), bf16 row-major, fp32 accumulation; K % 64 == 0, N % 64 == 0.
// splits > 1 splits K (K / splits % 64 == 0) and needs partial = splits * M * N floats.
hipError_t launch_linear(const void* x, const void* w, void* y, float* partial, int M, int K, int N, int splits,
                         hipStream_t stream);
// FP8 block-quantised per-head products.  Packed weight = E4M3 codes (H x 512 x 128 bytes; W_UV's
// stored transposed as (H, 128, 512)) followed by H x 4 fp32 scales (one per 128 x 128 block).
hipError_t launch_quantize_weight_fp8(const void* w, void* packed, bool transpose, hipStream_t stream);
hipError_t launch_absorb_q_fp8(const void* q_nope, const void* packed, void* q_lat, int tokens, hipStream_t stream);
hipError_t launch_out_proj_fp8(const float* o_lat, const void* packed, void* out, int tokens, hipStream_t stream);
// rotary embedding of q_pe (B,S,H,64, in place) and of the k_pe part of kv_a rows (stride
// kv_stride elements, [c_KV 512 | k_pe 64] at the row start), and AppendKV of [c_KV | k_pe] into
// the paged pool at positions seq_lens[b] - S + i.
hipError_t launch_rope_append(void* q_pe, const void* kv_a, int kv_stride, void* pool, const int32_t* block_table,
                              const int32_t* seq_lens, int B, int S, int max_pages, double base, const Bounds& bounds,
                              hipStream_t stream);

}  // namespace mla
