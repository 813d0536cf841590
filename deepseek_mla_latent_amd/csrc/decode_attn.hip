// Latent-space attention for absorbed MLA decode, gfx950.
//
// For every (sequence b, query token i, head h):
//   z_j   = scale * (q_lat[b,i,h,:] . c_j + q_pe[b,i,h,:] . k_pe_j)   over the visible cached tokens j
//   o_lat = sum_j softmax(z)_j c_j ,  lse = log sum_j exp(z_j)
// The latent c_j serves as key (with the shared RoPE key k_pe_j added to the score) and as value
// for all 128 heads: "DeepSeek-V2的推理成本如何计算？" (izhida.com), answers "DeepSeek" (512-d
// latent + 64-d RoPE inner product, 512-d weighted sum per head and cached token) and "专家"
// (RoPE as a shared-key MQA whose score is added). Scores and the weighted sum are steps 3 and 1
// of order 2 in "【笔记】MLA矩阵吸收分析" §二.2 and §三.2.
//
// bf16 kernel (one workgroup = 4 waves = 128 heads of one (b, i), one contiguous page range):
//   * the key range is walked in tiles of 32 tokens (half a page).  Tiles stream HBM -> LDS by
//     direct-to-LDS loads (16 B per lane, no register staging) into a ring of 4 LDS buffers,
//     three tiles ahead of the one being computed, so about 100 KiB per CU are in flight;
//   * each LDS tile is XOR-swizzled in 16-byte units so both read patterns below are free of
//     bank conflicts;
//   * scores are computed transposed, S^T = tile * Q^T, on 32x32x16 bf16 MFMAs: the tile is the
//     A operand (ds_read_b128), the wave's 32 heads' [q_lat | q_pe] stay in registers as the B
//     operand.  The accumulator layout then gives every lane one head and 16 tokens, which is
//     already the B-operand layout of the next product (no cross-lane shuffle for P);
//   * O^T (latent x heads) += tile^T * P^T reuses the same LDS tile as the value; its transposed
//     A operand comes from ds_read_b64_tr_b16 (4 tokens x 1 latent column per lane per read);
//   * online softmax in base 2 with the scale folded in; the running max is only raised (and O
//     rescaled) when a tile's max exceeds it by more than 2^8, which keeps exp2 arguments <= 8
//     and skips almost every rescale of the 256 accumulator registers.
// Long contexts are split into page ranges (split-K over tokens); each range writes a normalised
// partial (o_k, lse_k) and lse_merge_kernel combines them.
// Tree-masked verify (EAGLE-style draft trees: the Perplexity post, section "Будущая работа"): the
// S new tokens are tree nodes cached at positions L-S .. L-1, parents before children; query i
// sees the committed keys and the keys of its ancestors and itself.  The row's visibility of the
// S new keys is one 64-bit mask (S <= 64), built once per workgroup by walking parent links and
// applied only to tiles that reach position L-S.
#include "attn_schedule.h"
#include "common.h"
#include "kernels.h"

namespace mla {

constexpr int kTile = 32;                             // tokens per LDS tile (half a page)
constexpr int kUnitsA = kDc / 8;                      // 16-byte units of c_KV per token (64)
constexpr int kUnitsB = kDr / 8;                      // 16-byte units of k_pe per token (8)
constexpr int kRegionA = kTile * kUnitsA * 16;        // 32768 B: c_KV part of a tile
constexpr int kBufBytes = kRegionA + kTile * kUnitsB * 16;  // 36864 B per tile buffer
constexpr int kDmaPerTile = 9;                        // direct-to-LDS loads per wave per tile
constexpr float kRescaleSlack = 8.0f;                 // log2 units

__device__ __forceinline__ uint32_t lds_addr(const MLA_LDS char* p) { return (uint32_t)(uintptr_t)p; }

// Swizzle: 16-byte unit u of token t is stored at unit (u ^ swz(t)) of the token's LDS row.
// Region A (64 units per row): bit-rotated low 4 bits of t, so 16 consecutive tokens at one unit
// (the score A-operand read) and 8 tokens x 4 units (the transposed read) both spread over banks.
__device__ __forceinline__ int swz_a(int t) { return ((t & 3) << 2) | ((t >> 2) & 3); }
__device__ __forceinline__ int swz_b(int t) { return (t >> 1) & 7; }
__device__ __forceinline__ int off_a(int t, int u) { return (t * kUnitsA + (u ^ swz_a(t))) * 16; }
__device__ __forceinline__ int off_b(int t, int u) { return kRegionA + (t * kUnitsB + (u ^ swz_b(t))) * 16; }

// Direct-to-LDS load of 16 bytes per lane: lane l's bytes land at LDS address lds + 16 l.
// Issued from asm: the compiler models this instruction as pending in the LDS counter as well,
// which would turn every LDS operand wait of the tile computed meanwhile into a full drain.  It
// has no register outputs; completion is awaited explicitly (dma_wait_tiles) before the barrier
// that publishes a tile.  M0 is not otherwise used by this kernel.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds) : "memory");
}
// The same from a wave-uniform base plus a 32-bit per-lane byte offset (no 64-bit vector math).
__device__ __forceinline__ void dma16_s(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds)
               : "memory");
}
// Wait until at most `younger` tiles' loads (kDmaPerTile each) of this wave are still in flight.
// Vector-memory loads complete in order, so this retires every older tile; loads the compiler
// issues itself only ever make the wait stricter.
__device__ __forceinline__ void dma_wait_tiles(int younger) {
  if (younger >= 2)
    asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
  else if (younger == 1)
    asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// The 256 O accumulators live in AGPRs and are otherwise only touched by MFMAs.  The two VALU
// uses (rare rescale, final normalisation) go through inline asm that reads/writes the AGPRs
// directly; written as plain C++, the register allocator moves all of O into VGPRs and spills.
// Inline asm is opaque to the hazard recognizer, so the first access waits out the MFMA
// write-to-read latency explicitly (s_nop 15 + s_nop 3 >= the 16-pass XDL requirement).
__device__ __forceinline__ void acc_wait_mfma() { asm volatile("s_nop 15\n\ts_nop 3" ::); }

__device__ __forceinline__ void acc_scale(f32x16& acc, float alpha) {
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    float x = acc[e];
    float tmp;
    asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                 : "+a"(x), "=&v"(tmp)
                 : "v"(alpha));
    acc[e] = x;
  }
}

__device__ __forceinline__ float acc_read_scaled(float x, float scale) {
  float tmp;
  asm volatile("v_accvgpr_read_b32 %0, %1\n\tv_mul_f32 %0, %0, %2" : "=&v"(tmp) : "a"(x), "v"(scale));
  return tmp;
}

// MFMAs of the main loop are issued from asm volatile statements with a memory clobber: the
// compiler keeps them in program order and cannot move the LDS operand loads (ordinary builtins,
// whose waits it still inserts exactly) across them, so the software pipeline below is executed
// as written.  Being opaque, these statements also hide hazards from the compiler; the few that
// matter are handled explicitly:
//   * VALU write -> MFMA source read needs 2 wait states: the first score MFMA takes SrcC = 0
//     (no VALU zeroing) and P goes through pin_after_valu() before use;
//   * MFMA result -> VALU read needs 18 wait states (16-pass XDL op): the last score MFMA of a
//     chain carries them (mfma_acc_v_last), O goes through acc_wait_mfma();
//   * dependent accumulation chains (same SrcC/Dst) need none.
__device__ __forceinline__ void mfma_first_v(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b) : "memory");
}
__device__ __forceinline__ void mfma_acc_v(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b) : "memory");
}
__device__ __forceinline__ void mfma_acc_a(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b) : "memory");
}
// Last MFMA of a chain whose result the VALU reads: the wait is part of the same statement, so
// no copy the compiler places after it (it cannot see the MFMA) can read the result too early.
__device__ __forceinline__ void mfma_acc_v_last(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 15\n\ts_nop 3" : "+v"(d) : "v"(a), "v"(b) : "memory");
}
__device__ __forceinline__ void pin_after_valu(bf16x8& x, bf16x8& y) { asm volatile("s_nop 1" : "+v"(x), "+v"(y)); }

__device__ __forceinline__ bf16x8 lds_read_b128(const MLA_LDS char* p) { return *(const MLA_LDS bf16x8*)p; }

// max of three (no NaN canonicalisation: inputs are scores or -inf)
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ __forceinline__ bf16x8 lds_read_tr_pair(const MLA_LDS char* lo, const MLA_LDS char* hi) {
  i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)lo);
  i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)hi);
  i16x8 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, r);
}

// Token range and output slots of one workgroup; shared by both dtypes.
// Visibility of the S new keys to query (b, i) under a draft tree (S <= 64), wave-uniform: bit j
// set iff node j is node i or one of its ancestors.  Lane j loads node j's parent once; the walk
// then follows parent links through readlane while they point strictly backwards, so it ends
// after at most S steps whatever the table holds.
__device__ __forceinline__ int tree_parent_of_lane(const int32_t* parents, int b, int S, int lane) {
  return lane < S ? parents[(size_t)b * S + lane] : -1;
}
__device__ __forceinline__ uint64_t tree_walk(int par, int S, int i) {
  uint64_t m = 0;
  int j = i;
  for (int step = 0; step < S && j >= 0; ++step) {
    m |= 1ull << j;
    const int pj = __builtin_amdgcn_readlane(par, j);
    j = pj < j ? pj : -1;
  }
  return m;
}

struct WorkItem {
  int b, i, split;
  int tok_begin, tok_end;  // [tok_begin, tok_end) of sequence b, page aligned at tok_begin
  int tail;                // L - S: position of the first new token (node 0 of a draft tree)
  size_t out_row;          // index of (head 0) in the o/lse output rows
};

__device__ __forceinline__ WorkItem make_work(const AttnArgs& a, int id) {
  WorkItem w;
  w.i = id % a.S;
  const int rest = id / a.S;
  w.split = rest % a.num_splits;
  w.b = rest / a.num_splits;
  const int L = a.seq_lens[w.b];
  int n = a.causal && !a.tree_parents ? L - a.S + w.i + 1 : L;
  n = n < 0 ? 0 : (n > L ? L : n);
  const int p_begin = w.split * a.pages_per_split;
  const int pages_L = (L + kPage - 1) / kPage;
  int p_end = p_begin + a.pages_per_split;
  p_end = p_end < pages_L ? p_end : pages_L;
  w.tok_begin = p_begin * kPage;
  w.tail = L - a.S;
  const int e = p_end * kPage;
  w.tok_end = e < n ? e : n;
  const size_t bi = (size_t)w.b * a.S + w.i;
  w.out_row = a.final_out ? bi * kHeads : (bi * a.num_splits + w.split) * kHeads;
  return w;
}

template <bool kTree>
__global__ __launch_bounds__(256, 1) void decode_attn_bf16_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds_raw[kNumBufs * kBufBytes];
  // Page ids of the range, then 12 words for kTree: word 0 = the first tile of the range that
  // reaches a draft-tree key; words 2-3 = zeros (no key of an earlier tile is masked); words 4-11
  // = the masked-key windows of that tile and the next three, two per tile (lanes 0-31, lanes
  // 32-63).  Read back per tile: held in registers across the loop they would not fit, and kept in
  // the page-id array so that both are addressed from one base.
  __shared__ __attribute__((aligned(16))) int lds_pages[kMaxSplitPages + 12];
  int* const lds_tree = lds_pages + kMaxSplitPages;
  MLA_LDS char* const smem = (MLA_LDS char*)lds_raw;

  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const WorkItem w = make_work(a, id);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, hf = lane >> 5;
  const int h = wave * 32 + l32;
  // kTree: node `lane`'s parent, loaded here and walked once the query prologue has waited for its
  // loads
  const int tpar = kTree ? tree_parent_of_lane(a.tree_parents, w.b, a.S, lane) : -1;

  // Output slots of this lane (head h, latent columns 8 g + 4 hf + 32 cb ..).  Computed where
  // they are used: held across the loop they would cost two 64-bit registers.
  // Final outputs are fp32; split partials are bf16 (the merge widens them again).
  auto out_ptrs = [&](int ln, size_t& o_idx, float*& lse_ptr) {
    const int hh = wave * 32 + (ln & 31);
    o_idx = (w.out_row + hh) * kDc + 4 * (ln >> 5);
    lse_ptr = a.lse_out ? a.lse_out + w.out_row + hh : nullptr;
  };
  // Element e of the 4 at (cb, g): latent column 32 cb + 8 g + 4 hf + e.
  auto store4 = [&](size_t o_idx, int cb, int g, const f32x4& v) {
    if (a.final_out) {
      *(f32x4*)((float*)a.o_out + o_idx + 32 * cb + 8 * g) = v;
    } else {
      const uint2 pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      *(uint2*)((uint16_t*)a.o_out + o_idx + 32 * cb + 8 * g) = pk;
    }
  };

  const int ntok = w.tok_end - w.tok_begin;
  if (ntok <= 0) {  // empty key range: o = 0, lse = -inf
    size_t o_idx;
    float* lse_ptr;
    out_ptrs(lane, o_idx, lse_ptr);
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cb = 0; cb < 16; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) store4(o_idx, cb, g, z);
    if (hf == 0 && lse_ptr) *lse_ptr = -INFINITY;
    return;
  }
  const int ntiles = (ntok + kTile - 1) / kTile;
  const int32_t* bt = a.block_table + (size_t)w.b * a.max_pages + w.tok_begin / kPage;
  const uint16_t* pool = (const uint16_t*)a.pool;

  // The range's page ids are staged in LDS once (at most kMaxSplitPages; the host sizes splits
  // accordingly), so the loop reads them with ds_read + readfirstlane.  A global load in the
  // loop would make the compiler drain the vector-memory counter, i.e. wait for the tiles in
  // flight; a scalar load would share the LDS counter and make every operand wait a full drain.
  // Their loads are issued here and stored to LDS after the query loads below, so the two
  // round trips overlap; the barrier that hands the buffers to the tiles also publishes them.
  const int npages = (ntok + kPage - 1) / kPage;
  constexpr int kPidPerThread = kMaxSplitPages / 256;
  int pid[kPidPerThread];
#pragma unroll
  for (int k = 0; k < kPidPerThread; ++k) {
    const int j = threadIdx.x + 256 * k;
    pid[k] = j < npages ? bt[j] : 0;
  }
  auto row_of = [&](int t, int page) -> const uint16_t* {  // first token row of tile t
    return pool + ((size_t)page * kPage + (t & 1) * kTile) * kRow;
  };
  auto tile_count = [&](int t) { return ntok - t * kTile < kTile ? ntok - t * kTile : kTile; };

  // One step of copying a tile (cnt valid tokens, rows from `src`) into LDS buffer `dst`:
  // steps 0-7 fill this wave's 8 tokens' 1 KiB c_KV rows (region A), step 8 the 128 B k_pe rows
  // of 8 tokens (region B).  Tokens past cnt re-read token 0 (always valid), so LDS never holds
  // bytes from outside the sequence; their scores are masked.
  // lane16 = 16 * lane: the per-lane part of every address is one XOR with a wave-uniform value.
  auto dma_step = [&](const uint16_t* src, int cnt, uint32_t dst, int k, uint32_t lane16) {
    const char* base = (const char*)src;
    if (k < 8) {
      const int t = wave * 8 + k;  // wave-uniform
      const int ts = t < cnt ? t : 0;
      dma16_s(base + ts * (kRow * 2), lane16 ^ (swz_a(t) * 16), dst + t * 1024);
    } else {
      const int t = wave * 8 + (int)(lane16 >> 7);
      const int ts = t < cnt ? t : 0;
      const uint32_t u = ((lane16 >> 4) & 7) ^ swz_b(t);
      dma16_s(base, ts * (kRow * 2) + kDc * 2 + u * 16, dst + kRegionA + wave * 1024);
    }
  };
  // Prologue.  The query rows come in first, through LDS: each wave copies its 32 heads' q_lat
  // rows (1 KiB each, one load per row, 16-byte unit u of row r stored at u ^ (r & 15)) into the
  // tile buffers, which are still free, and reads its B operands from there; q_pe (4 loads) comes
  // straight from memory.  Then tiles 0-2 start streaming into the buffers.
  bf16x8 q[36];  // this lane's head as the score B operand: [q_lat | q_pe][16 ks + 8 hf .. +7]
  {
    const size_t qrow0 = ((size_t)w.b * a.S + w.i) * kHeads + wave * 32;
    const char* qsrc = (const char*)((const uint16_t*)a.q_lat + qrow0 * kDc);
    const uint32_t qdst = lds_addr(smem) + wave * 32 * 1024;
#pragma unroll
    for (int r = 0; r < 32; ++r) dma16_s(qsrc + r * 1024, (uint32_t)((lane ^ (r & 15)) * 16), qdst + r * 1024);
    const bf16x8* qp = (const bf16x8*)((const uint16_t*)a.q_pe + (qrow0 + l32) * kDr + 8 * hf);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) q[32 + ks] = qp[2 * ks];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) asm volatile("" ::"v"(q[32 + ks]));
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int k = 0; k < kPidPerThread; ++k)
      if (threadIdx.x + 256 * k < npages) lds_pages[threadIdx.x + 256 * k] = pid[k];
    const MLA_LDS char* qrowp = smem + wave * 32 * 1024 + l32 * 1024;
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) q[ks] = lds_read_b128(qrowp + (((2 * ks + hf) ^ (l32 & 15)) * 16));
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) asm volatile("" ::"v"(q[ks]));
  }
  if (kTree && wave == 0) {
    // Window of tile t for lane half hf: bit k (k = (e/4)*8 + e%4 for element e) is the
    // visibility of the key at kpos(t) + 4 hf + k, i.e. node j = kpos(t) - tail + 4 hf + k.  With
    // E = [32 ones | the row's 64-bit mask | 32 zeros], E bit j + 32 is node j (negative:
    // committed), so the window is E bits u .. u + 31 for u = kpos(t) - tail + 4 hf + 32.
    const uint64_t m = tree_walk(tpar, a.S, w.i);
    const int t_first = w.tail - w.tok_begin < kTile ? 0 : (w.tail - w.tok_begin) / kTile;
    if (lane < 8) {
      int u = w.tok_begin + (t_first + (lane >> 1)) * kTile - w.tail + 4 * (lane & 1) + 32;
      u = u < 0 ? 0 : (u > 96 ? 96 : u);  // below 0: all committed; above 96: all past node 63
      const int qw = u >> 5, r = u & 31;
      const uint32_t lo = (uint32_t)m, hi = (uint32_t)(m >> 32);
      const uint32_t lo_w = qw == 0 ? 0xffffffffu : (qw == 1 ? lo : (qw == 2 ? hi : 0u));
      const uint32_t hi_w = qw == 0 ? lo : (qw == 1 ? hi : 0u);
      lds_tree[4 + lane] = (int32_t)~__builtin_amdgcn_alignbit(hi_w, lo_w, r);  // 1 = masked
    }
    if (lane == 0) lds_tree[0] = t_first;
    if (lane == 2 || lane == 3) lds_tree[lane] = 0;
  }
  __syncthreads();  // every wave has its q and the page ids are in LDS: the buffers take the tiles now
  auto prologue_tile = [&](int t) {
    const uint16_t* src = row_of(t, __builtin_amdgcn_readfirstlane(lds_pages[t >> 1]));
    const int cnt = tile_count(t);
    const uint32_t dst = lds_addr(smem) + t * kBufBytes;
#pragma unroll
    for (int k = 0; k < kDmaPerTile; ++k) dma_step(src, cnt, dst, k, lane * 16);
  };
  for (int t = 0; t < kNumBufs - 1 && t < ntiles; ++t) prologue_tile(t);
  dma_wait_tiles(ntiles - 1 < 2 ? ntiles - 1 : 2);  // tile 0 has landed (this wave's part)

  // Per-lane LDS byte offsets of the swizzled reads, relative to smem; the score offsets follow
  // the tile being scored, the sum offsets the (previous) tile being summed, one buffer per tile.
  // score step r (r < 32): qk_a[r % 8] + 256 (r / 8); (r >= 32): qk_b[r - 32].
  // sum step m: latent block cb = m / 2, token step kk = m % 2 -> pv_lo/hi[cb % 4] + 256 (cb / 4)
  // + 16384 kk.  All immediates stay below 64 KiB.
  int qk_a[8], qk_b[4], pv_lo[4], pv_hi[4];
#pragma unroll
  for (int k = 0; k < 8; ++k) qk_a[k] = off_a(l32, 2 * k + hf);
#pragma unroll
  for (int k = 0; k < 4; ++k) qk_b[k] = off_b(l32, 2 * k + hf);
  {
    const int r4 = (lane >> 2) & 3;
    const int colq = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const int tb = 4 * hf + r4;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = 32 * k + colq;
      pv_lo[k] = off_a(tb, c >> 3) + (c & 7) * 2;
      pv_hi[k] = off_a(tb + 8, c >> 3) + (c & 7) * 2;
    }
  }
  auto read_qk = [&](int g) -> bf16x8 {  // A operand of score MFMA g (0..35)
    if (g < 32) return lds_read_b128(smem + qk_a[g & 7] + 256 * (g >> 3));
    return lds_read_b128(smem + qk_b[g - 32]);
  };
  auto read_pv = [&](int m) -> bf16x8 {  // A operand of sum MFMA m (0..31)
    const int cb = m >> 1, kk = m & 1;
    const int imm = 256 * (cb >> 2) + 16384 * kk;
    return lds_read_tr_pair(smem + pv_lo[cb & 3] + imm, smem + pv_hi[cb & 3] + imm);
  };
  auto step_of = [](int t) { return (t % kNumBufs) == kNumBufs - 1 ? -(kNumBufs - 1) * kBufBytes : kBufBytes; };
  auto advance_qk = [&](int t) {  // from tile t's buffer to tile t+1's
    const int s = step_of(t);
#pragma unroll
    for (int k = 0; k < 8; ++k) qk_a[k] += s;
#pragma unroll
    for (int k = 0; k < 4; ++k) qk_b[k] += s;
  };
  auto advance_pv = [&](int t) {
    const int s = step_of(t);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      pv_lo[k] += s;
      pv_hi[k] += s;
    }
  };

  f32x16 o[16];
#pragma unroll
  for (int cb = 0; cb < 16; ++cb)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[cb][e] = 0.f;
  // The reference starts at the lowest finite float, so a tile whose keys are all masked (a draft
  // tree can hide whole tiles, even the first of a range) gives exp2(-inf) = 0, never inf - inf.
  float m_run = -3.402823466e38f, l_run = 0.f;
  bool started = false;  // wave-uniform: a first visible key has been seen
  // Consume every scalar kernel argument the loop uses here, so no scalar load is still in
  // flight inside the loop (it would share the LDS counter and force full drains there).
  const float scale_log2 = a.scale_log2;
  asm volatile("" ::"s"(scale_log2), "s"(ntiles), "s"(ntok));


  // ---- online softmax of one tile's raw scores sc (element e = token (e/4)*8 + 4 hf + e%4 of
  // the tile), in base 2 with the scale folded into the exponent's FMA, cut into stages so that
  // its instructions can ride between the MFMAs of the next tile's scores.  Masked keys get a raw
  // score of -inf.  Output: P in bf16 (pk), already in the B layout of the weighted sum.
  bf16x8 pk[2];
  float mx[5], mt = 0.f, alpha = 1.f;
  bool rescale = false;  // wave-uniform
  // Stage s runs in score slot s: 0-2 the tile max and the new reference, then one probability in
  // every second slot (3, 5, .., 33), so no slot holds more VALU work than one MFMA's duration.
  auto softmax_stage = [&](int s, int cnt, f32x16& sc) {
    if (s == 0) {
      if (cnt < kTile) {  // wave-uniform: only the last tile of a range can be partial
        const int lim = cnt - 4 * hf;  // element e is valid iff (e/4)*8 + e%4 < lim
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if ((e >> 2) * 8 + (e & 3) >= lim) sc[e] = -INFINITY;
      }
#pragma unroll
      for (int i = 0; i < 5; ++i) mx[i] = max3(sc[3 * i], sc[3 * i + 1], sc[3 * i + 2]);
    } else if (s == 1) {  // lanes l and l^32 hold the same head
      mt = fmaxf(max3(mx[0], mx[1], mx[2]), max3(mx[3], mx[4], sc[15]));
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
      mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * scale_log2;
    } else if (s == 2) {
      // Branch-free on purpose: a branch here lets the compiler duplicate the rest of the score
      // chain per outcome.  O itself is rescaled right before the sum, outside the chain.
      const bool raise = __any(mt > m_run + kRescaleSlack);  // wave-uniform
      const float m_new = raise ? fmaxf(m_run, mt) : m_run;
      rescale = raise && started;  // O and l hold something: rescale them to the new reference
      alpha = rescale ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
      l_run *= alpha;
      m_run = m_new;
      started = started || raise;
    } else if (s >= 3 && s < 35 && (s & 1)) {
      const int e = (s - 3) >> 1;
      const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e], scale_log2, -m_run));
      l_run += pv;
      pk[e >> 3][e & 7] = (__bf16)pv;
      // keep this stage here: without the pin the compiler sinks all of them to the first use
      asm volatile("" : "+v"(pk[e >> 3]), "+v"(l_run));
    }
  };
  constexpr int kSoftmaxStages = 35;

  // kTree: raw scores of tile t.  A key of a node that is neither the query's node nor one of its
  // ancestors gets -inf; committed keys stay.  Tiles before the first one that reaches the tree
  // keep everything; a range meets at most three such tiles (64 nodes), a fourth entry covers the
  // stale tile scored past the end.
  // Element e: a signed extract of its masked-key bit (0 or all ones) selects the score or -inf
  // (an instruction literal), two temporaries at a time.  The kernel has no register to spare
  // across the loop, so nothing here may be hoisted out of it: the LDS address and the lane half
  // are hidden from loop-invariant code motion.
  auto tree_mask_tile = [&](f32x16& sc, int t) {
    int z = 0;  // an opaque zero in the addresses: a constant LDS address would be hoisted
    asm volatile("" : "+s"(z));
    int ci = t - __builtin_amdgcn_readfirstlane(lds_tree[z]);  // wave-uniform
    ci = ci < -1 ? -1 : (ci > 3 ? 3 : ci);
    int ln = lane;  // an opaque copy of the lane id (live anyway): its half is not hoisted either
    asm volatile("" : "+v"(ln));
    const uint32_t mwin = (uint32_t)lds_tree[z + 4 + 2 * ci + (ln >> 5)];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float x = sc[e];
      uint32_t m, ninf;  // m = masked ? ~0 : 0; ninf = m & bits(-inf); x = m ? -inf : x
      asm volatile(
          "v_bfe_i32 %1, %3, %4, 1\n\tv_and_b32 %2, 0xff800000, %1\n\tv_bfi_b32 %0, %1, %2, %0"
          : "+v"(x), "=&v"(m), "=&v"(ninf)
          : "v"(mwin), "i"((e >> 2) * 8 + (e & 3)));
      sc[e] = x;
    }
  };

  // ---- scores of tile 0 (nothing to overlap yet)
  __builtin_amdgcn_s_barrier();  // every wave's part of tile 0 has landed
  bf16x8 ring[4];
  f32x16 sa, sb;  // raw scores: the two buffers swap roles every tile (no copy between them)
#pragma unroll
  for (int g = 0; g < 4; ++g) ring[g] = read_qk(g);
#pragma unroll
  for (int ks = 0; ks < 36; ++ks) {
    if (ks == 0)
      mfma_first_v(sa, ring[0], q[0]);
    else if (ks < 35)
      mfma_acc_v(sa, ring[ks & 3], q[ks]);
    else
      mfma_acc_v_last(sa, ring[ks & 3], q[ks]);
    if (ks + 4 < 36) ring[ks & 3] = read_qk(ks + 4);
  }
  if constexpr (kTree) tree_mask_tile(sa, 0);
  if (ntiles > 1) {  // tile 1 has landed everywhere; start its operand reads
    dma_wait_tiles(ntiles > 2 ? 1 : 0);
    __builtin_amdgcn_s_barrier();
    advance_qk(0);
#pragma unroll
    for (int g = 0; g < 4; ++g) ring[g] = read_qk(g);
  }
  // page id of tile 3 (the first one the loop streams in)
  int page_ahead = ntiles > 3 ? __builtin_amdgcn_readfirstlane(lds_pages[3 >> 1]) : 0;

  // ---- steady state, iteration t: scores of tile t+1 with the softmax of tile t riding in the
  // gaps of that MFMA chain, then the weighted sum of tile t.  Tile t+3 streams in meanwhile, into
  // the buffer tile t-1 used.  One barrier per tile follows the sum: every read of tile t has
  // completed (the sum MFMAs consumed them) and tile t+2 has landed; then the first operand reads
  // of tile t+2's scores are issued.
  // The last iteration scores a stale buffer (its result is never used) to keep a single copy of
  // the softmax and the sum in the code.
  auto iteration = [&](int t, f32x16& sc, f32x16& sn) {
    const int cnt = tile_count(t);
    const int tn = t + kNumBufs - 1;
    // Past the last tile the nine loads still issue (a branch per load in the MFMA stream costs
    // more than the load), but every lane then reads the same 16 bytes at the start of the pool,
    // into a buffer that the ring schedule (attn_schedule.h) proves no other wave is reading.
    const bool more = tn < ntiles;
    const uint16_t* nsrc = more ? row_of(tn, page_ahead) : pool;
    const int ncnt = more ? tile_count(tn) : 0;
    const uint32_t ndst = lds_addr(smem) + attn_dma_buffer(t, ntiles) * kBufBytes;
    // The per-lane DMA offsets are loop-invariant; recomputing them (one XOR each) is cheaper than
    // the registers LICM would pin across the loop, so hide the lane id from it.
    uint32_t lane16 = lane * 16;
    asm volatile("" : "+v"(lane16));
    lane16 = more ? lane16 : 0u;

    int pid_v = 0;
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) {
      if (ks == 0)
        mfma_first_v(sn, ring[0], q[0]);
      else
        mfma_acc_v(sn, ring[ks & 3], q[ks]);
      ring[ks & 3] = ks + 4 < 36 ? read_qk(ks + 4) : read_pv(ks + 4 - 36);
      if (ks % 7 == 2) dma_step(nsrc, ncnt, ndst, ks / 7, lane16);  // loads 0-4 (slots 2, 9, .., 30)
      if (ks < kSoftmaxStages) softmax_stage(ks, cnt, sc);
      if (ks == 12) pid_v = lds_pages[((t + kNumBufs) >> 1) < npages ? (t + kNumBufs) >> 1 : 0];
      __builtin_amdgcn_sched_barrier(0);
    }
    if (rescale) {
      acc_wait_mfma();
#pragma unroll
      for (int cb = 0; cb < 16; ++cb) acc_scale(o[cb], alpha);
      asm volatile("s_nop 4" ::: "memory");
    }
    pin_after_valu(pk[0], pk[1]);

#pragma unroll
    for (int m = 0; m < 32; ++m) {
      mfma_acc_a(o[m >> 1], ring[m & 3], pk[m & 1]);
      if (m + 4 < 32) ring[m & 3] = read_pv(m + 4);
      if (m % 7 == 3 && m < 28) dma_step(nsrc, ncnt, ndst, 5 + m / 7, lane16);  // loads 5-8 (slots 3, .., 24)
      if (m == 8) page_ahead = __builtin_amdgcn_readfirstlane(pid_v);
      __builtin_amdgcn_sched_barrier(0);
    }
    // kTree: mask the next tile's scores here, where the operand ring is dead (its registers are
    // what the masking needs) and 32 MFMAs separate the last write of sn from these reads
    if constexpr (kTree) tree_mask_tile(sn, t + 1);
    if (attn_barrier_after(t, ntiles)) {  // every read of tile t done, tile t+2 landed: publish, then prefetch
      dma_wait_tiles(1);
      __builtin_amdgcn_s_barrier();
      advance_qk(t + 1);
#pragma unroll
      for (int g = 0; g < 4; ++g) ring[g] = read_qk(g);
    } else if constexpr (kTree) {
      // Past the last tile the ring keeps its spent values for the stale scores; refilled from the
      // current buffer instead (any LDS bytes do), its old values die before the masking above.
#pragma unroll
      for (int g = 0; g < 4; ++g) ring[g] = read_qk(g);
    }
    advance_pv(t);
  };
  // Unrolled twice so that the two score buffers alternate: a loop-carried copy of an MFMA result
  // (which the compiler cannot see being written) could be placed before the write completes.
  for (int t = 0; t < ntiles; t += 2) {
    iteration(t, sa, sb);
    if (t + 1 < ntiles) iteration(t + 1, sb, sa);
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;  // every key masked: o = 0, lse = -inf
  size_t o_idx;
  float* lse_ptr;
  {
    int lane_e = lane;
    asm volatile("" : "+v"(lane_e));
    out_ptrs(lane_e, o_idx, lse_ptr);
  }
  // The last loads (stale prefetches) land in LDS before the staging below reuses it, and every
  // wave has finished reading the tile buffers.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  acc_wait_mfma();
  if (a.final_out) {
#pragma unroll
    for (int cb = 0; cb < 16; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v = {acc_read_scaled(o[cb][4 * g], inv), acc_read_scaled(o[cb][4 * g + 1], inv),
                   acc_read_scaled(o[cb][4 * g + 2], inv), acc_read_scaled(o[cb][4 * g + 3], inv)};
        store4(o_idx, cb, g, v);
      }
  } else {
    // bf16 partial rows go out through LDS: each lane holds 4-value pieces of one head's row, so
    // direct stores would write 32 rows x 16 B per instruction; staged, one store writes one
    // whole 1 KiB row.  Rows are 1040 B apart in LDS (2-way bank conflicts on the writes).
    constexpr int kStageRow = kDc * 2 + 16;
    MLA_LDS char* stage = smem + wave * (32 * kStageRow);
#pragma unroll
    for (int cb = 0; cb < 16; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x2 v = {pack_bf16x2(acc_read_scaled(o[cb][4 * g], inv), acc_read_scaled(o[cb][4 * g + 1], inv)),
                         pack_bf16x2(acc_read_scaled(o[cb][4 * g + 2], inv), acc_read_scaled(o[cb][4 * g + 3], inv))};
        *(MLA_LDS u32x2*)(stage + l32 * kStageRow + (32 * cb + 8 * g + 4 * hf) * 2) = v;
      }
    uint16_t* rows = (uint16_t*)a.o_out + (w.out_row + wave * 32) * kDc + 8 * lane;
#pragma unroll 8
    for (int r = 0; r < 32; ++r)
      *(u32x4*)(rows + (size_t)r * kDc) = *(const MLA_LDS u32x4*)(stage + r * kStageRow + 16 * lane);
  }
  if (hf == 0 && lse_ptr) *lse_ptr = (m_run + __log2f(l_tot)) * 0.69314718055994531f;
}

// fp32 path: one workgroup per (b, i, split, head); 256 threads.  Logits one token per thread,
// block-wide max/sum, then each thread accumulates two latent columns over the chunk's tokens.
// Natural-exp online softmax with the exact rescale at every 256-token chunk.
__global__ __launch_bounds__(256) void decode_attn_f32_kernel(AttnArgs a) {
  __shared__ float qs[kRow];
  __shared__ float ps[256];
  __shared__ float red[8];
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int h = id % kHeads;
  const WorkItem w = make_work(a, id / kHeads);
  const int tid = threadIdx.x;
  const float* pool = (const float*)a.pool;

  const size_t qrow = ((size_t)w.b * a.S + w.i) * kHeads + h;
  for (int c = tid; c < kDc; c += 256) qs[c] = ((const float*)a.q_lat)[qrow * kDc + c];
  if (tid < kDr) qs[kDc + tid] = ((const float*)a.q_pe)[qrow * kDr + tid];
  __syncthreads();

  const int32_t* bt = a.block_table + (size_t)w.b * a.max_pages;
  const uint64_t tmask =
      a.tree_parents ? tree_walk(tree_parent_of_lane(a.tree_parents, w.b, a.S, tid & 63), a.S, w.i) : 0ull;
  auto visible = [&](int tkn) {
    const int j = tkn - w.tail;
    return !a.tree_parents || j < 0 || (j < 64 && ((tmask >> j) & 1ull));
  };
  float m_run = -INFINITY, l_run = 0.f, acc0 = 0.f, acc1 = 0.f;
  for (int start = w.tok_begin; start < w.tok_end; start += 256) {
    const int tkn = start + tid;
    float z = -INFINITY;
    if (tkn < w.tok_end && visible(tkn)) {
      const float* row = pool + ((size_t)bt[tkn / kPage] * kPage + tkn % kPage) * kRow;
      float d = 0.f;
      for (int c = 0; c < kRow; ++c) d = fmaf(qs[c], row[c], d);
      z = d * a.scale;
    }
    float m = z;
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float m_new = fmaxf(m_run, m);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;  // a chunk with every key masked
    const float alpha = expf(m_run - m_use);
    const float p = expf(z - m_use);  // masked keys and keys past the range have z = -inf
    ps[tid] = p;
    float sm = p;
    for (int off = 32; off > 0; off >>= 1) sm += __shfl_xor(sm, off);
    __syncthreads();
    if ((tid & 63) == 0) red[4 + (tid >> 6)] = sm;
    __syncthreads();
    l_run = l_run * alpha + (red[4] + red[5] + red[6] + red[7]);
    acc0 *= alpha;
    acc1 *= alpha;
    const int cnt = w.tok_end - start < 256 ? w.tok_end - start : 256;
    for (int j = 0; j < cnt; ++j) {
      const int tj = start + j;
      const float* row = pool + ((size_t)bt[tj / kPage] * kPage + tj % kPage) * kRow;
      acc0 = fmaf(ps[j], row[tid], acc0);
      acc1 = fmaf(ps[j], row[tid + 256], acc1);
    }
    m_run = m_new;
    __syncthreads();
  }
  float* o_ptr = (float*)a.o_out + (w.out_row + h) * kDc;
  const bool empty = w.tok_end <= w.tok_begin || l_run == 0.f;
  o_ptr[tid] = empty ? 0.f : acc0 / l_run;
  o_ptr[tid + 256] = empty ? 0.f : acc1 / l_run;
  if (tid == 0 && a.lse_out) a.lse_out[w.out_row + h] = empty ? -INFINITY : m_run + logf(l_run);
}

// Merge the per-split partials of every (b, i, h): lse = log sum_k e^{lse_k},
// o = sum_k e^{lse_k - lse} o_k.  Empty splits carry lse_k = -inf, o_k = 0 and weight 0.
// One wave per (row = b*S+i, head); lane l owns latent columns [8 l, 8 l + 8).  The split lse
// values are read one per lane (64 splits per load) and their weights broadcast with readlane;
// the partial rows are taken eight splits at a time with all sixteen loads issued before the
// first use.  Workgroup ids go through the same XCD renumbering as the attention grid, so row b
// is merged on the XCD whose L2 received its partials.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// Lane l's 8 partial values of one split (latent columns 8 l .. 8 l + 7), kept as loaded (bf16
// words stay packed until use: the register count decides how many merge waves fit on a CU).
template <typename PartT>
struct PartRow;
template <>
struct PartRow<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = ((const f32x4*)p)[0];
    b = ((const f32x4*)p)[1];
  }
  __device__ __forceinline__ f32x4 lo() const { return a; }
  __device__ __forceinline__ f32x4 hi() const { return b; }
};
template <>
struct PartRow<uint16_t> {
  u32x4 u;
  __device__ __forceinline__ void load(const uint16_t* p) { u = *(const u32x4*)p; }
  __device__ __forceinline__ f32x4 lo() const {
    return f32x4{__uint_as_float(u[0] << 16), __uint_as_float(u[0] & 0xffff0000u), __uint_as_float(u[1] << 16),
                 __uint_as_float(u[1] & 0xffff0000u)};
  }
  __device__ __forceinline__ f32x4 hi() const {
    return f32x4{__uint_as_float(u[2] << 16), __uint_as_float(u[2] & 0xffff0000u), __uint_as_float(u[3] << 16),
                 __uint_as_float(u[3] & 0xffff0000u)};
  }
};

template <typename PartT>
__global__ __launch_bounds__(256) void lse_merge_kernel(const PartT* __restrict__ o_part,
                                                        const float* __restrict__ lse_part, float* __restrict__ o_lat,
                                                        float* __restrict__ lse, int num_splits) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int rh = xcd_remap(blockIdx.x, gridDim.x) * 4 + wave;  // row * kHeads + h
  const int row = rh / kHeads, h = rh % kHeads;
  const size_t base = (size_t)row * num_splits * kHeads + h;  // split k at base + k * kHeads
  const float* lp = lse_part + base;
  const PartT* op = o_part + base * kDc + 8 * lane;
  constexpr float kLog2e = 1.4426950408889634f;
  auto lse_of = [&](int k) { return k < num_splits ? lp[(size_t)k * kHeads] : -INFINITY; };

  PartRow<PartT> x[8];
  auto load_batch = [&](int kb) {  // splits kb .. kb+7 (clamped to the last one)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = kb + j < num_splits ? kb + j : num_splits - 1;
      x[j].load(op + (size_t)k * kHeads * kDc);
    }
  };
  load_batch(0);  // does not depend on the weights: in flight while they are formed
  const float lse0 = lse_of(lane);
  float m = lse0;
  for (int k0 = 64; k0 < num_splits; k0 += 64) m = fmaxf(m, lse_of(k0 + lane));
  m = wave_max(m);
  const float m_ref = m == -INFINITY ? 0.f : m;  // all splits empty: every weight is 0

  f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
  float sum = 0.f, w_lane = 0.f;
  for (int kb = 0; kb < num_splits; kb += 8) {
    if ((kb & 63) == 0)  // weights of splits kb .. kb+63, one per lane (0 past the end)
      w_lane = __builtin_amdgcn_exp2f(((kb == 0 ? lse0 : lse_of(kb + lane)) - m_ref) * kLog2e);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float w = kb + j < num_splits
                          ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_lane), (kb & 63) + j))
                          : 0.f;
      sum += w;
      a0 += w * x[j].lo();
      a1 += w * x[j].hi();
    }
    if (kb + 8 < num_splits) load_batch(kb + 8);
  }
  const float inv = sum > 0.f ? 1.0f / sum : 0.f;
  f32x4* dst = (f32x4*)(o_lat + (size_t)rh * kDc + 8 * lane);
  dst[0] = a0 * inv;
  dst[1] = a1 * inv;
  if (lane == 0 && lse) lse[rh] = m == -INFINITY ? -INFINITY : m + logf(sum);
}

hipError_t launch_decode_attn(const AttnArgs& a, int rows, hipStream_t stream) {
  forget_stale_error();
  const int nwg = rows * a.num_splits;
  if (a.dtype_bf16 && a.tree_parents)
    hipLaunchKernelGGL(decode_attn_bf16_kernel<true>, dim3(nwg), dim3(256), 0, stream, a);
  else if (a.dtype_bf16)
    hipLaunchKernelGGL(decode_attn_bf16_kernel<false>, dim3(nwg), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(decode_attn_f32_kernel, dim3(nwg * kHeads), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_lse_merge(const void* o_part, bool part_bf16, const float* lse_part, float* o_lat, float* lse,
                            int rows, int num_splits, hipStream_t stream) {
  forget_stale_error();
  const dim3 grid(rows * (kHeads / 4));
  if (part_bf16)
    hipLaunchKernelGGL(lse_merge_kernel<uint16_t>, grid, dim3(256), 0, stream, (const uint16_t*)o_part, lse_part,
                       o_lat, lse, num_splits);
  else
    hipLaunchKernelGGL(lse_merge_kernel<float>, grid, dim3(256), 0, stream, (const float*)o_part, lse_part, o_lat,
                       lse, num_splits);
  return hipGetLastError();
}

}  // namespace mla
