/*
 * mla_latent.h — Multi-head Latent Attention (MLA) on MI355X (gfx950): absorbed decode, and
 * prefill in multi-head form.
 *
 * One decode step of one MLA layer, as three enqueue-only calls:
 *
 *   mla_absorb_q     q_lat = W_UK^T q_nope   per head (the no-RoPE query moved into the
 *                    512-d latent space, so per-head keys are never built)
 *   mla_decode_attn  softmax over the cached context of scale*(q_lat.c_j + q_pe.k_pe_j),
 *                    reduced to a latent output o_lat = sum_j p_j c_j, plus its log-sum-exp
 *   mla_out_proj     out = W_UV^T o_lat      per head (values are never built)
 *
 * mla_decode_attn_out_proj does the last two in one call (the split merge inside the W_UV
 * kernel, so o_lat need not pass through memory).
 *
 * The method: "DeepSeek-V2的推理成本如何计算？" (izhida.com), answer "专家" — W_K is applied
 * transposed to q and W_V after the latent attention-weighted average, so neither K nor V is
 * computed; RoPE is a separate key shared by all heads whose score is added to the latent
 * score. Shapes and computation order: "【笔记】MLA矩阵吸收分析" (wkq9411.github.io), §二.2
 * (order 2: (b,s,h,k) query, (b,h,s,t) scores) and §三.2 (order 2: (b,h,s,k) latent output,
 * then W_UV). The three calls are the BMM -> Attn -> BMM span of the decode stages listed in
 * "Lower latency and higher throughput with multi-node DeepSeek deployment" (Perplexity),
 * section "Наложение вычислений и взаимодействия", with kv_b_proj split into a K part and a
 * V part (section "Слой MLA") and a paged cache addressed through a page table (same
 * section).
 *
 * Conventions for every call
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library allocates and
 *     frees nothing, never synchronises, and keeps no mutable global state (it caches the
 *     device's compute-unit count once per device). Each call only enqueues kernels on
 *     `stream` (a hipStream_t; NULL = the default stream), so calls are thread-safe and can be
 *     captured into a HIP graph.
 *   - Layouts are dense row-major with the last index fastest, exactly as the comments give.
 *   - Every condition the host can check is checked BEFORE any launch; on failure the call
 *     returns a negative mla_status, enqueues nothing and writes nothing.
 *   - Supported dims: num_heads 128, kv_lora_rank 512, rope_dim 64, head_dim 128,
 *     page_size 64. Other values give MLA_ERR_UNSUPPORTED.
 *   - Pointers must be 16-byte aligned (MLA_ERR_ALIGN).
 *   - Device-side preconditions: 0 <= seq_lens[b] <= max_seq_len; block_table[b][p] in
 *     [0, num_pages) for every page p that holds one of the first seq_lens[b] tokens (P = the
 *     pool's page count). libmla_latent.so does not check them (violating them is undefined
 *     behaviour). The bounds-checked build of the same library, libmla_latent_debug.so
 *     (compiled with MLA_DEBUG_BOUNDS), checks every entry a kernel uses, on the device, and
 *     reports violations in an error word (mla_debug_bounds_read); see there. With causal and
 *     q_len S, query i sees the first seq_lens[b] - S + i + 1 tokens (fewer than one: an empty
 *     set).
 *   - An empty key set yields o_lat = 0 and lse = -inf.
 */
#ifndef MLA_LATENT_H_
#define MLA_LATENT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL = -1,        /* a required pointer is NULL */
  MLA_ERR_SHAPE = -2,       /* a size is out of range (batch < 0, q_len < 1, tables too small ...) */
  MLA_ERR_DTYPE = -3,       /* dtype is not MLA_F32 or MLA_BF16 (prefill, FP8 calls: not MLA_BF16) */
  MLA_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned */
  MLA_ERR_WORKSPACE = -5,   /* workspace / kv buffer smaller than its _bytes() query */
  MLA_ERR_UNSUPPORTED = -6, /* head dims / page size other than the supported set */
  MLA_ERR_LAUNCH = -7,      /* the HIP runtime rejected a launch */
  MLA_ERR_DEVICE = -8,      /* no usable HIP device */
  MLA_ERR_SCRATCH = -9      /* the request needs more than MLA_STATIC_SCRATCH_BYTES of static scratch */
} mla_status;

typedef enum { MLA_F32 = 0, MLA_BF16 = 1 } mla_dtype;

typedef struct {
  int32_t batch;             /* B >= 0 sequences */
  int32_t q_len;             /* S >= 1 query tokens per sequence (2 = MTP / speculative verify) */
  int32_t num_heads;         /* H = 128 */
  int32_t kv_lora_rank;      /* d_c = 512: latent width */
  int32_t rope_dim;          /* d_R = 64: shared RoPE key width */
  int32_t head_dim;          /* d_h = 128: no-RoPE query/key width and value width */
  int32_t page_size;         /* 64 tokens per cache page */
  int32_t max_pages_per_seq; /* row stride of block_table (>= ceil(max_seq_len / page_size)) */
  int32_t max_seq_len;       /* host-known upper bound on seq_lens[]: sizes the grid, no D2H copy */
  float softmax_scale;       /* > 0; multiplies the whole logit (latent + RoPE parts), e.g. 1/sqrt(192) */
  int32_t causal;            /* 1: query i of S sees seq_lens[b] - S + i + 1 keys; 0: all keys */
  mla_dtype dtype;           /* of q_nope, q_pe, q_lat, cache, W_UK, W_UV, out; accumulation is fp32 */
  int32_t num_pages;         /* >= 0: pages in kv_pool, 0 = not given. Only the bounds-checked build
                                reads it (page ids >= num_pages are violations; with 0, only
                                negative ids are) */
} mla_params;

/*
 * q_lat[b,s,h,c] = sum_d W_UK[h,c,d] * q_nope[b,s,h,d]
 *   q_nope (B,S,H,d_h)  dtype         — no-RoPE query
 *   w_uk   (H,d_c,d_h)  dtype         — key up-projection, head-major
 *   q_lat  (B,S,H,d_c)  dtype (out)   — absorbed query; fp32 accumulation, rounded once
 * Cites: izhida answer "专家" (W_K applied transposed to q); absorption note §二.2 step 2.
 */
mla_status mla_absorb_q(const void* q_nope, const void* w_uk, void* q_lat, const mla_params* p,
                        void* stream);

/*
 * Bytes of scratch memory mla_decode_attn needs for `num_splits` (0 = the library's choice),
 * 0 when the call needs none. Returns 0 as well for an invalid `p` (the call will reject it).
 */
size_t mla_decode_workspace_bytes(const mla_params* p, int32_t num_splits);

/*
 * Number of key splits mla_decode_attn uses for `num_splits` (0 = the library's choice);
 * returns a negative mla_status for an invalid `p`.
 */
int32_t mla_decode_num_splits(const mla_params* p, int32_t num_splits);

/*
 * Latent-space attention over a paged cache.
 *   q_lat       (B,S,H,d_c)        dtype   absorbed query (from mla_absorb_q)
 *   q_pe        (B,S,H,d_R)        dtype   RoPE query, already rotated
 *   kv_pool     (P,page,d_c+d_R)   dtype   cache pages; row = [c_KV (d_c) | k_pe (d_R)]
 *   block_table (B,max_pages_per_seq) int32  token j of sequence b lives in page
 *                                         block_table[b][j / page] at slot j % page
 *   seq_lens    (B)                int32   L_b = cached tokens of sequence b (the S new ones included)
 *   o_lat       (B,S,H,d_c)        fp32 (out)  sum_j p_j c_j
 *   lse         (B,S,H)            fp32 (out, may be NULL)  natural-log log-sum-exp of the
 *                                         scaled logits
 *   workspace / workspace_bytes           scratch of at least mla_decode_workspace_bytes()
 *                                         (may be NULL when that is 0); contents are scratch
 *   num_splits                            0 = library's choice; k > 1 reduces the keys in
 *                                         B * S * k contiguous page ranges, merged per query row
 *                                         by log-sum-exp. Up to 256 query rows the ranges follow
 *                                         the rows' lengths: with C the smallest page count for
 *                                         which the rows need at most B * S * k ranges of C pages
 *                                         (at least one per row), each row is cut into ranges of
 *                                         C pages (equal lengths give k ranges per row); above
 *                                         256 rows every row gets k ranges. With num_splits = 0,
 *                                         bf16 and 33..256 query rows, the bound is
 *                                         R = max(B * S * k, ceil(9/8 * compute units)) ranges
 *                                         instead, and rows of unequal length are cut to fill it,
 *                                         run longest first (the ranges past the first wave of
 *                                         one per compute unit fill the units that finish early).
 *                                         Results for a fixed split count and fixed lengths are
 *                                         bitwise reproducible.
 * Cites: izhida answer "DeepSeek" (per head a 512-d latent and a 64-d RoPE inner product and a
 * weighted sum over the 512-d latent, per cached token) and answer "专家"; cache row of 576
 * per layer (same answer; Perplexity post, section "Одноузловое против многоузлового").
 */
mla_status mla_decode_attn(const void* q_lat, const void* q_pe, const void* kv_pool,
                           const int32_t* block_table, const int32_t* seq_lens, float* o_lat,
                           float* lse, void* workspace, size_t workspace_bytes, int32_t num_splits,
                           const mla_params* p, void* stream);

/*
 * mla_decode_attn with a draft-tree mask in place of the causal rule (tree-masked verify of
 * EAGLE-style speculation, which predicts several tokens arranged as a tree: Perplexity post,
 * section "Будущая работа"). The S = q_len new tokens of sequence b are the nodes of a tree,
 * cached at positions seq_lens[b] - S .. seq_lens[b] - 1 in an order where every parent comes
 * before its children.
 *   tree_parents (B,S) int32   node j's parent in [-1, j); -1 = a child of the last committed
 *                              token. Query i sees the committed keys 0 .. seq_lens[b] - S - 1
 *                              and the keys of node i's ancestors and of node i itself; a chain
 *                              (parent j - 1) is the causal rule. A parent outside [-1, j) ends
 *                              node j's ancestor walk (the node then has no further ancestors);
 *                              node positions below 0 are not visible.
 * Every other argument, the split count and the workspace (mla_decode_num_splits /
 * mla_decode_workspace_bytes for the same p) are as for mla_decode_attn; p->causal is ignored.
 * Errors: q_len > 64 gives MLA_ERR_SHAPE; tree_parents NULL (with B*S > 0) gives MLA_ERR_NULL.
 * A split whose keys are all masked contributes nothing (lse -inf); an empty visible set gives
 * o_lat = 0, lse = -inf.
 */
mla_status mla_decode_attn_tree(const void* q_lat, const void* q_pe, const void* kv_pool,
                                const int32_t* block_table, const int32_t* seq_lens, const int32_t* tree_parents,
                                float* o_lat, float* lse, void* workspace, size_t workspace_bytes,
                                int32_t num_splits, const mla_params* p, void* stream);

/*
 * out[b,s,h,v] = sum_c o_lat[b,s,h,c] * W_UV[h,c,v]
 *   o_lat (B,S,H,d_c)  fp32          — latent attention output (from mla_decode_attn)
 *   w_uv  (H,d_c,d_h)  dtype         — value up-projection, head-major
 *   out   (B,S,H,d_h)  dtype (out)   — per-head attention output (before W_O)
 * Cites: izhida answer "专家" (W_V applied after the latent average) and the same answer's
 * batched GEMV whose cost is reading W_V; absorption note §三.2 step 2.
 */
mla_status mla_out_proj(const float* o_lat, const void* w_uv, void* out, const mla_params* p,
                        void* stream);

/*
 * Workspace bytes of mla_decode_attn_out_proj for this p and split request (0 for an invalid p),
 * with k = mla_decode_num_splits(p, num_splits) and R the range bound of mla_decode_attn (B * S * k
 * unless the library's own choice allows more): R * H * (d_c * 2 + 4) (the bf16 split partials)
 * plus 16 + B * S * 8 rounded up to a multiple of 16 (the range plan) when bf16, B * S >= 16 and
 * k > 1; mla_decode_workspace_bytes(p, num_splits) when fp32, B * S <= 4 and k > 1 (the fp32
 * partials and the plan); otherwise the call runs the separate kernels, and the workspace is
 * mla_decode_workspace_bytes(p, num_splits) plus B * S * H * d_c * 4 bytes for o_lat.
 */
size_t mla_decode_attn_out_proj_workspace_bytes(const mla_params* p, int32_t num_splits);

/*
 * mla_decode_attn followed by mla_out_proj in two launches: the split attention, then the
 * log-sum-exp merge of its partials fused with the W_UV product, so the merged latent output
 * need not round-trip through memory. dtype MLA_BF16 or MLA_F32 (w_uv and out in that dtype).
 *   tree_parents (B,S) int32 or NULL  NULL: the causal / full rule of p (as mla_decode_attn);
 *                                     otherwise the draft-tree rule of mla_decode_attn_tree
 *                                     (q_len > 64 gives MLA_ERR_SHAPE)
 *   w_uv  (H,d_c,d_h) dtype           value up-projection, head-major
 *   out   (B,S,H,d_h) dtype (out)     per-head attention output (before W_O)
 *   o_lat (B,S,H,d_c) fp32 (out, may be NULL)  the merged latent output
 *   lse   (B,S,H)     fp32 (out, may be NULL)
 *   workspace / workspace_bytes       at least mla_decode_attn_out_proj_workspace_bytes(p,
 *                                     num_splits); contents are scratch
 * The other arguments are as for mla_decode_attn. In bf16 with B * S >= 16 query rows and more
 * than one split the merge of the bf16 partials runs in fp32 inside the W_UV kernel; in fp32 with
 * B * S <= 4 query rows and more than one split the merge of the fp32 partials runs inside the
 * out-projection's per-row dot products; otherwise (fewer bf16 rows would leave most of the W_UV
 * kernel's lanes idle, and one split has no merge to save) the call makes exactly the launches of
 * mla_decode_attn followed by mla_out_proj, with o_lat in the workspace when o_lat is NULL. Errors as for mla_decode_attn / mla_decode_attn_tree, plus
 * MLA_ERR_NULL for a NULL w_uv or out (with B*S > 0).
 * Cites: absorption note §三.2 steps 1-2 (the latent weighted sum, then W_V after it); izhida
 * answer "专家" (W_V applied after the latent average).
 */
mla_status mla_decode_attn_out_proj(const void* q_lat, const void* q_pe, const void* kv_pool,
                                    const int32_t* block_table, const int32_t* seq_lens,
                                    const int32_t* tree_parents, const void* w_uv, void* out, float* o_lat,
                                    float* lse, void* workspace, size_t workspace_bytes, int32_t num_splits,
                                    const mla_params* p, void* stream);

/*
 * mla_decode_attn_out_proj with the W_UV product FP8 block-quantised (the Perplexity post, sections
 * "Слой MLA" and "Квантование"): w_uv_fp8 is the packed buffer mla_quantize_w_uv_fp8 writes, and
 * each merged latent row is coded on the fly with one scale per 128-long vector, the scheme of
 * mla_out_proj_fp8. Every other argument, the workspace (mla_decode_attn_out_proj_workspace_bytes)
 * and every error are those of mla_decode_attn_out_proj. With at least 16 query rows and more than
 * one split, the merge, the coding and the FP8 product run in one kernel; otherwise the call runs
 * the attention (with its merge) and then mla_out_proj_fp8's kernel on o_lat.
 */
mla_status mla_decode_attn_out_proj_fp8(const void* q_lat, const void* q_pe, const void* kv_pool,
                                        const int32_t* block_table, const int32_t* seq_lens,
                                        const int32_t* tree_parents, const void* w_uv_fp8, void* out, float* o_lat,
                                        float* lse, void* workspace, size_t workspace_bytes, int32_t num_splits,
                                        const mla_params* p, void* stream);

/*
 * Static scratch of mla_decode_attn_out_proj_static: 64 MiB of device memory per GPU, held from the
 * library's load until the process ends (the split partials of 32 sequences x 8 key ranges, or of
 * 256 query rows x 2 ranges, take 33.7 MB).
 */
#define MLA_STATIC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * mla_decode_attn_out_proj without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP-graph capture, serving loops and harnesses that forbid allocation): the
 * scratch the call needs (mla_decode_attn_out_proj_workspace_bytes(p, num_splits) bytes) is taken
 * from a static device array of MLA_STATIC_SCRATCH_BYTES that each GPU holds for the life of the
 * process. The call allocates and frees nothing. Every other argument, every output and every error
 * is as for mla_decode_attn_out_proj, plus MLA_ERR_SCRATCH (returned before any launch) when the
 * scratch needed exceeds MLA_STATIC_SCRATCH_BYTES, and MLA_ERR_DEVICE when the array's device
 * address cannot be looked up. The array keeps what the last call left in it; all calls on one
 * GPU share it, so calls that overlap on one GPU (on different streams, or from different
 * threads without ordering) race and give undefined results.
 */
mla_status mla_decode_attn_out_proj_static(const void* q_lat, const void* q_pe, const void* kv_pool,
                                           const int32_t* block_table, const int32_t* seq_lens,
                                           const int32_t* tree_parents, const void* w_uv, void* out,
                                           float* o_lat, float* lse, int32_t num_splits, const mla_params* p,
                                           void* stream);

/*
 * ---- Prefill in multi-head form ("order 1") --------------------------------------------------
 * When the query tokens are the prompt itself (t = s), up-projecting K and V from the latent and
 * attending per head costs fewer FLOPs than the absorbed route: "【笔记】MLA矩阵吸收分析" §二.4.1
 * (order 1 minus order 2 is negative at t = s), with the order-1 steps of §二.1 and §三.1; the
 * Perplexity post plans the same for its prefill (section "Будущая работа": project the latent
 * into K/V space, then compute in MHA form). Two calls, bf16 only (MLA_F32 gives MLA_ERR_DTYPE):
 *
 *   mla_prefill_kv_up   K_nope and V of every cached token, per head, from the paged latent cache
 *   mla_prefill_attn    attention per head over those keys/values with the shared RoPE key
 *
 * q_len S is the number of new (query) tokens per sequence; they are the last S of the
 * seq_lens[b] cached tokens, with the same causal rule as decode (S = seq_lens[b]: a whole prompt).
 */

/*
 * Bytes of the K/V buffer the two prefill calls exchange (0 for an invalid `p`):
 * B * Lp * (H * 256 + 64) * 2 with Lp = max_pages_per_seq * page_size. Layout: [K_nope | V]
 * (B, H, Lp, 256) bf16, then k_pe (B, Lp, 64) bf16.
 */
size_t mla_prefill_kv_bytes(const mla_params* p);

/*
 * K_nope[b,h,j,:] = sum_c c_j[c] W_UK[h,c,:] and V[b,h,j,:] = sum_c c_j[c] W_UV[h,c,:] for
 * every cached token j < seq_lens[b] (page lookup as in mla_decode_attn), and a dense copy of
 * k_pe_j. Rows from seq_lens[b] to the end of that sequence's last page are written as zeros;
 * rows after that are not written.
 *   kv_pool, block_table, seq_lens  as for mla_decode_attn
 *   w_uk, w_uv (H,d_c,d_h) bf16
 *   kv / kv_bytes                   the buffer above (at least mla_prefill_kv_bytes(p) bytes)
 * Cites: absorption note §二.1 step 2 ((b,t,h,d) keys) and §三.1 step 1 ((b,t,h,v) values).
 */
mla_status mla_prefill_kv_up(const void* kv_pool, const int32_t* block_table, const int32_t* seq_lens,
                             const void* w_uk, const void* w_uv, void* kv, size_t kv_bytes,
                             const mla_params* p, void* stream);

/*
 * out[b,i,h,:] = sum_j p_j V[b,h,j,:] with p = softmax over the visible keys j of
 * scale * (q_nope[b,i,h,:] . K_nope[b,h,j,:] + q_pe[b,i,h,:] . k_pe_j); lse as in
 * mla_decode_attn.
 *   q_nope (B,S,H,d_h), q_pe (B,S,H,d_R) bf16   query (q_pe already rotated)
 *   kv / kv_bytes                               written by mla_prefill_kv_up with the same p
 *   out    (B,S,H,d_h) bf16 (out)               per-head attention output (before W_O)
 *   lse    (B,S,H) fp32 (out, may be NULL)
 * Equal (up to rounding) to mla_absorb_q + mla_decode_attn + mla_out_proj on the same inputs.
 * Cites: absorption note §二.1 step 3 and §三.1 step 2; izhida answer "专家" (the RoPE part is
 * a key shared by all heads whose score is added).
 */
mla_status mla_prefill_attn(const void* q_nope, const void* q_pe, const void* kv, size_t kv_bytes,
                            const int32_t* seq_lens, void* out, float* lse, const mla_params* p,
                            void* stream);

/*
 * ---- The step before the path -----------------------------------------------------------------
 * The stage before attention is InputNorm, QKVProj, AppendKV, BMM (Perplexity post, section
 * "Наложение вычислений и взаимодействия"), with q_a_proj and kv_a_proj fused into one projection
 * (section "Слой MLA"). The absorption note (§二.1) gives the compressed widths. The
 * normalisations are not part of these calls.
 */

/*
 * Bytes of scratch memory mla_linear needs for an m x k by k x n product (0 when none, or for
 * invalid sizes). It depends on the device's compute-unit count: query it on the device that
 * will run the call.
 */
size_t mla_linear_workspace_bytes(int32_t m, int32_t k, int32_t n);

/*
 * y = x W: x (m, k) bf16, W (k, n) bf16, y (m, n) bf16 (out), all row-major; fp32 accumulation,
 * rounded once. k and n must be multiples of 64. For a few rows the layer is a weight stream:
 * the library splits k so the grid fills the chip, and sums the fp32 partials in a fixed order
 * in `workspace` (at least mla_linear_workspace_bytes(); its contents are scratch). Results are
 * bitwise reproducible on one device. Serves the fused a-projection
 * (y = [c^Q | c^KV | k_pe before rotation], k = d_model, n = q_lora_rank + 512 + 64) and any
 * other plain projection in the same form.
 * Cites: Perplexity post, section "Слой MLA" (fused qkv_a_proj); absorption note §二.1 (widths).
 */
mla_status mla_linear(const void* x, const void* w, void* y, int32_t m, int32_t k, int32_t n,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Rotary position embedding, then AppendKV, for the S = q_len new tokens of each sequence. Token
 * i of sequence b is at position pos = seq_lens[b] - S + i, so seq_lens already counts the new
 * tokens.
 *   q_pe    (B,S,H,64) bf16, rotated in place
 *   kv_a    rows of kv_a_stride elements (>= 576, a multiple of 8), one per token (b, i), each
 *           starting with [c_KV (512) | k_pe (64) before rotation]; e.g. the fused projection's
 *           output at column offset q_lora_rank
 *   kv_pool, block_table, seq_lens as for mla_decode_attn; the slot of pos receives
 *           [c_KV | rotated k_pe]. A token at a negative position (seq_lens[b] < S) is rotated
 *           but not written.
 *   rope_base  the rotation base (10000)
 * Rotation: each consecutive pair (x[2j], x[2j+1]) turns by pos * rope_base^(-2j/64) (the
 * rotation of Su et al., RoFormer; the pages give no formula). Angles are formed in fp64; the
 * rotation is done in fp32 and rounded once to bf16. c_KV is copied bit for bit.
 * bf16 only (MLA_ERR_DTYPE otherwise).
 * Cites: Perplexity post, sections "Наложение вычислений и взаимодействия" (AppendKV before
 * attention) and "Слой MLA" (paged cache); izhida answer "专家" (the RoPE key is one per token,
 * shared by the heads).
 */
mla_status mla_rope_append(void* q_pe, const void* kv_a, int32_t kv_a_stride, void* kv_pool,
                           const int32_t* block_table, const int32_t* seq_lens, float rope_base,
                           const mla_params* p, void* stream);

/*
 * ---- FP8 block-quantised per-head products ----------------------------------------------------
 * The k_b_proj / v_b_proj products (W_UK, W_UV) as an FP8 block-quantised batched matmul
 * (Perplexity post, section "Слой MLA"), with the scheme of section "Квантование": weights
 * quantised statically, one scale per 128 x 128 block; activations on the fly, one scale per
 * 128-element vector along the reduction dimension. Format E4M3 (bias 7, largest finite 448;
 * the pages name no format). A block's scale is amax / 448 in fp32; a value is coded as
 * x * (448 / amax) (the factor one fp32 division per block, the product an fp32 multiplication)
 * rounded to the nearest E4M3 value, ties to even (the hardware conversion, subnormals kept).
 * An all-zero block has scale 0 and codes 0. The products accumulate in fp32 per block, then
 * scale. bf16 activations only.
 *
 * Packed weight (mla_fp8_weight_bytes() bytes, 16-byte aligned, owned by the caller): E4M3 codes,
 * H x 512 x 128 bytes (W_UK: (H, 512 c, 128 d) as the weight; W_UV: transposed, (H, 128 v, 512 c)),
 * then H x 4 fp32 scales (head h, latent block c / 128).
 */
size_t mla_fp8_weight_bytes(void);

/* Static quantisation of W_UK (H,512,128) bf16 / W_UV (H,512,128) bf16 into a packed weight. */
mla_status mla_quantize_w_uk_fp8(const void* w_uk, void* packed, size_t packed_bytes,
                                 const mla_params* p, void* stream);
mla_status mla_quantize_w_uv_fp8(const void* w_uv, void* packed, size_t packed_bytes,
                                 const mla_params* p, void* stream);

/*
 * As mla_absorb_q, in FP8: q_nope (B,S,H,128) bf16 quantised per (token, head) vector;
 * q_lat (B,S,H,512) bf16 = s_q * s_w[h][c/128] * sum_d code(q) code(W).
 * Cites: Perplexity post, sections "Слой MLA" (FP8 block-quantised BMM for k_b_proj) and
 * "Квантование" (128-element activation vectors, 128 x 128 weight blocks).
 */
mla_status mla_absorb_q_fp8(const void* q_nope, const void* w_uk_fp8, void* q_lat,
                            const mla_params* p, void* stream);

/*
 * As mla_out_proj, in FP8: o_lat (B,S,H,512) fp32 quantised per 128-long latent block of each
 * (token, head); out (B,S,H,128) bf16 = sum over the four blocks of s_o * s_w * sum code*code.
 * Cites: as mla_absorb_q_fp8 (v_b_proj).
 */
mla_status mla_out_proj_fp8(const float* o_lat, const void* w_uv_fp8, void* out, const mla_params* p,
                            void* stream);

/* Static string for a status code (never NULL). */
const char* mla_status_str(mla_status s);

/*
 * Introspection for tests (host only, touches no device): the LDS ring schedule the bf16
 * attention kernel follows over a key range of ntiles 32-token tiles. For each iteration
 * u < ntiles: a_buffer[u] and b_buffer[u] receive the ring-A buffer (0..3, latent rows) and the
 * ring-B buffer (0..2, RoPE-key rows) that the loads issued in iteration u write (those of tile
 * u + 2, which carry data only while u + 2 < ntiles), and p_buffer[u] the ring-P buffer (0..1)
 * that the probabilities of tile u are written to. The arrays are caller-owned host arrays of at
 * least ntiles entries. Returns MLA_ERR_SHAPE if ntiles < 1, MLA_ERR_NULL if an array is NULL,
 * else MLA_OK.
 */
mla_status mla_debug_attn_schedule(int32_t ntiles, int32_t* a_buffer, int32_t* b_buffer, int32_t* p_buffer);

/*
 * Bounds-checked build. mla_debug_bounds_enabled() is 1 in libmla_latent_debug.so and 0 in
 * libmla_latent.so.
 *
 * In the bounds-checked build, every kernel that walks the page table (mla_decode_attn,
 * mla_decode_attn_tree, mla_decode_attn_out_proj and its static-scratch form, mla_prefill_kv_up,
 * mla_prefill_attn, mla_rope_append) tests each entry it uses: a seq_lens entry outside
 * [0, max_seq_len] sets bit 1 of the error word and is clamped into that range; a block_table entry
 * outside [0, num_pages) (num_pages 0: a negative entry) sets bit 2, a read then takes page 0 and
 * the cache append skips its write. The outputs of an affected sequence are then meaningless, but
 * no access leaves the buffers the preconditions describe. Reports are device atomics on a
 * per-device word pair; the calls themselves stay asynchronous.
 *
 * mla_debug_bounds_read(words, clear) waits for the device (hipDeviceSynchronize), copies
 *   words[0] = union of the violation bits since the last clear (1: seq_lens, 2: block_table),
 *   words[1] = number of reports (one per GPU lane that saw a violation; 0 iff words[0] == 0),
 * and with clear != 0 resets both to zero. words: HOST pointer to 2 uint32 (MLA_ERR_NULL if
 * NULL). MLA_ERR_DEVICE if the device cannot be reached; MLA_ERR_UNSUPPORTED in libmla_latent.so.
 * Cites: the page table of the Perplexity post, section "Слой MLA".
 */
int32_t mla_debug_bounds_enabled(void);
mla_status mla_debug_bounds_read(uint32_t* words, int32_t clear);

#ifdef __cplusplus
}
#endif

#endif /* MLA_LATENT_H_ */
