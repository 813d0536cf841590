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
#include "common.h"
#include "kernels.h"

namespace mla {

constexpr int kTile = 32;                             // tokens per LDS tile (half a page)
constexpr int kUnitsA = kDc / 8;                      // 16-byte units of c_KV per token (64)
constexpr int kUnitsB = kDr / 8;                      // 16-byte units of k_pe per token (8)
constexpr int kRegionA = kTile * kUnitsA * 16;        // 32768 B: c_KV part of a tile
constexpr int kBufBytes = kRegionA + kTile * kUnitsB * 16;  // 36864 B per tile buffer
constexpr int kNumBufs = 4;                           // LDS ring: tile t lives in buffer t % 4
constexpr int kAhead = kNumBufs - 1;                  // tiles in flight ahead of the computed one
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
//   * MFMA result -> VALU read needs more than 11 wait states: scores go through
//     wait_mfma_result(), O through acc_wait_mfma();
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
__device__ __forceinline__ void wait_mfma_result(f32x16& d) { asm volatile("s_nop 15\n\ts_nop 3" : "+v"(d)); }
__device__ __forceinline__ void pin_after_valu(bf16x8& x, bf16x8& y) { asm volatile("s_nop 1" : "+v"(x), "+v"(y)); }

__device__ __forceinline__ bf16x8 lds_read_b128(const MLA_LDS char* p) { return *(const MLA_LDS bf16x8*)p; }

__device__ __forceinline__ bf16x8 lds_read_tr_pair(const MLA_LDS char* lo, const MLA_LDS char* hi) {
  i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)lo);
  i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)hi);
  i16x8 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, r);
}

// Token range and output slots of one workgroup; shared by both dtypes.
struct WorkItem {
  int b, i, split;
  int tok_begin, tok_end;  // [tok_begin, tok_end) of sequence b, page aligned at tok_begin
  size_t out_row;          // index of (head 0) in the o/lse output rows
};

__device__ __forceinline__ WorkItem make_work(const AttnArgs& a, int id) {
  WorkItem w;
  w.i = id % a.S;
  const int rest = id / a.S;
  w.split = rest % a.num_splits;
  w.b = rest / a.num_splits;
  const int L = a.seq_lens[w.b];
  int n = a.causal ? L - a.S + w.i + 1 : L;
  n = n < 0 ? 0 : (n > L ? L : n);
  const int p_begin = w.split * a.pages_per_split;
  const int pages_L = (L + kPage - 1) / kPage;
  int p_end = p_begin + a.pages_per_split;
  p_end = p_end < pages_L ? p_end : pages_L;
  w.tok_begin = p_begin * kPage;
  const int e = p_end * kPage;
  w.tok_end = e < n ? e : n;
  const size_t bi = (size_t)w.b * a.S + w.i;
  w.out_row = a.final_out ? bi * kHeads : (bi * a.num_splits + w.split) * kHeads;
  return w;
}

__global__ __launch_bounds__(256, 1) void decode_attn_bf16_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds_raw[kNumBufs * kBufBytes];
  __shared__ int lds_pages[kMaxSplitPages];
  MLA_LDS char* const smem = (MLA_LDS char*)lds_raw;

  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const WorkItem w = make_work(a, id);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, hf = lane >> 5;
  const int h = wave * 32 + l32;

  float* o_ptr = a.o_out + (w.out_row + h) * kDc + 4 * hf;
  float* lse_ptr = a.lse_out ? a.lse_out + w.out_row + h : nullptr;

  const int ntok = w.tok_end - w.tok_begin;
  if (ntok <= 0) {  // empty key range: o = 0, lse = -inf
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cb = 0; cb < 16; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) *(f32x4*)(o_ptr + 32 * cb + 8 * g) = z;
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
  const int npages = (ntok + kPage - 1) / kPage;
  for (int j = threadIdx.x; j < npages; j += 256) lds_pages[j] = bt[j];
  __syncthreads();
  auto tile_src = [&](int t) -> const uint16_t* {  // first token row of tile t (t < ntiles)
    const int page = __builtin_amdgcn_readfirstlane(lds_pages[t >> 1]);
    return pool + ((size_t)page * kPage + (t & 1) * kTile) * kRow;
  };
  auto tile_count = [&](int t) { return ntok - t * kTile < kTile ? ntok - t * kTile : kTile; };

  // One step of copying tile `t` (cnt valid tokens, rows from `src`) into LDS buffer `dst`:
  // steps 0-7 fill this wave's 8 tokens' 1 KiB c_KV rows (region A), step 8 the 128 B k_pe rows
  // of 8 tokens (region B).  Tokens past cnt re-read token 0 (always valid), so LDS never holds
  // bytes from outside the sequence; their scores are masked.
  auto dma_step = [&](const uint16_t* src, int cnt, uint32_t dst, int k, int lane_v) {
    if (k < 8) {
      const int t = wave * 8 + k;
      const int ts = t < cnt ? t : 0;
      dma16(src + ts * kRow + (lane_v ^ swz_a(t)) * 8, dst + t * 1024);
    } else {
      const int t = wave * 8 + (lane_v >> 3);
      const int ts = t < cnt ? t : 0;
      dma16(src + ts * kRow + kDc + ((lane_v & 7) ^ swz_b(t)) * 8, dst + kRegionA + wave * 1024);
    }
  };
  // Prologue: tiles 0 .. kAhead-1.
  for (int t = 0; t < kAhead && t < ntiles; ++t) {
    const uint16_t* src = tile_src(t);
    const int cnt = tile_count(t);
    const uint32_t dst = lds_addr(smem) + t * kBufBytes;
#pragma unroll
    for (int k = 0; k < kDmaPerTile; ++k) dma_step(src, cnt, dst, k, lane);
  }

  // This lane's head, as the B operand of the score MFMA: q[ks] = [q_lat | q_pe][16 ks + 8 hf .. +7].
  bf16x8 q[36];
  {
    const size_t qrow = ((size_t)w.b * a.S + w.i) * kHeads + h;
    const bf16x8* ql = (const bf16x8*)((const uint16_t*)a.q_lat + qrow * kDc + 8 * hf);
    const bf16x8* qp = (const bf16x8*)((const uint16_t*)a.q_pe + qrow * kDr + 8 * hf);
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) q[ks] = ql[2 * ks];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) q[32 + ks] = qp[2 * ks];
    // Wait for q here, once: otherwise the loop inherits "q may be in flight" and carries
    // vector-memory waits that the in-flight tile loads would then trip.
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) asm volatile("" ::"v"(q[ks]));
  }

  // Per-lane LDS byte offsets of the swizzled reads in the current tile's buffer; advanced by one
  // buffer per tile.  score step r (r < 32): qk_a[r % 8] + 256 (r / 8); (r >= 32): qk_b[r - 32].
  // sum step m: latent block cb = m / 2, token step kk = m % 2 -> pv_lo/hi[cb % 4] + 256 (cb / 4)
  // + 16384 kk.  All immediates stay below 64 KiB.
  const int base0 = 0;  // offsets are relative to smem
  int qk_a[8], qk_b[4], pv_lo[4], pv_hi[4];
#pragma unroll
  for (int k = 0; k < 8; ++k) qk_a[k] = base0 + off_a(l32, 2 * k + hf);
#pragma unroll
  for (int k = 0; k < 4; ++k) qk_b[k] = base0 + off_b(l32, 2 * k + hf);
  {
    const int r4 = (lane >> 2) & 3;
    const int colq = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const int tb = 4 * hf + r4;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = 32 * k + colq;
      pv_lo[k] = base0 + off_a(tb, c >> 3) + (c & 7) * 2;
      pv_hi[k] = base0 + off_a(tb + 8, c >> 3) + (c & 7) * 2;
    }
  }
  auto read_op = [&](int g) -> bf16x8 {  // A operand of MFMA g of the tile (0..67)
    const MLA_LDS char* z = smem;
    if (g < 32) return lds_read_b128(z + qk_a[g & 7] + 256 * (g >> 3));
    if (g < 36) return lds_read_b128(z + qk_b[g - 32]);
    const int m = g - 36, cb = m >> 1, kk = m & 1;
    const int imm = 256 * (cb >> 2) + 16384 * kk;
    return lds_read_tr_pair(z + pv_lo[cb & 3] + imm, z + pv_hi[cb & 3] + imm);
  };

  f32x16 o[16];
#pragma unroll
  for (int cb = 0; cb < 16; ++cb)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[cb][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  bool started = false;  // wave-uniform: a first key has been seen (m_run finite)
  // Consume every scalar kernel argument the loop uses here, so no scalar load is still in
  // flight inside the loop (it would share the LDS counter and force full drains there).
  const float scale_log2 = a.scale_log2;
  asm volatile("" ::"s"(scale_log2), "s"(ntiles), "s"(ntok));

  for (int t = 0; t < ntiles; ++t) {
    {  // tile t is in LDS for every wave; every wave is done with tile t-1's buffer
      const int younger = ntiles - 1 - t;
      dma_wait_tiles(younger < kAhead - 1 ? younger : kAhead - 1);
    }
    __syncthreads();
    const int cnt = tile_count(t);
    // The next tile to stream in goes to the buffer tile t-1 used.
    const int tn = t + kAhead;
    const bool more = tn < ntiles;
    const uint16_t* nsrc = more ? tile_src(tn) : pool;
    const int ncnt = more ? tile_count(tn) : 0;
    const uint32_t ndst = lds_addr(smem) + (tn % kNumBufs) * kBufBytes;
    // The per-lane DMA addresses are loop-invariant; recomputing them (a few VALU ops) is far
    // cheaper than the registers LICM would pin across the loop, so hide the lane id from it.
    int lane_v = lane;
    asm volatile("" : "+v"(lane_v));

    // One stream of 68 MFMAs: 36 for the scores (K = 512 latent + 64 RoPE in steps of 16), then
    // 32 for the weighted sum (16 latent blocks x 2 token steps).  Their A operands come from LDS
    // through a 4-deep register ring: the read for MFMA g + 4 is issued right after MFMA g, so
    // LDS latency hides behind MFMAs; the score tail already fetches the first weighted-sum
    // operands (they do not depend on the softmax), which land while the softmax runs.  The next
    // tile's 9 load instructions are spread over the score MFMAs, at the same slots in all four
    // waves (staggering them across waves measured half again slower).
    bf16x8 ring[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) ring[g] = read_op(g);

    // ---- raw scores S^T (32 tokens x 32 heads)
    f32x16 sc;
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) {
      if (ks == 0)
        mfma_first_v(sc, ring[0], q[0]);
      else
        mfma_acc_v(sc, ring[ks & 3], q[ks]);
      ring[ks & 3] = read_op(ks + 4);
      if ((ks & 3) == 1 && more) dma_step(nsrc, ncnt, ndst, ks >> 2, lane_v);
    }
    wait_mfma_result(sc);

    // ---- online softmax in base 2 (scale folded into the exponent's FMA); element e of sc is
    // token (e/4)*8 + 4 hf + e%4 of the tile.  Masked keys get a raw score of -inf.
    if (cnt < kTile) {  // wave-uniform: only the last tile of a range can be partial
      const int lim = cnt - 4 * hf;  // element e is valid iff (e/4)*8 + e%4 < lim
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if ((e >> 2) * 8 + (e & 3) >= lim) sc[e] = -INFINITY;
    }
    float mt = sc[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mt = fmaxf(mt, sc[e]);
    {  // lanes l and l^32 hold the same head
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
      mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * scale_log2;
    }
    if (__any(mt > m_run + kRescaleSlack)) {
      const float m_new = fmaxf(m_run, mt);
      if (started) {  // O and l hold something: rescale them to the new reference
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
        acc_wait_mfma();
#pragma unroll
        for (int cb = 0; cb < 16; ++cb) acc_scale(o[cb], alpha);
        asm volatile("s_nop 4" ::: "memory");
      }
      m_run = m_new;
      started = true;
    }
    bf16x8 pk[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[8 * kk + j], scale_log2, -m_run));
        l_run += pv;
        pk[kk][j] = (__bf16)pv;
      }
    pin_after_valu(pk[0], pk[1]);

    // ---- O^T (latent x heads) += tile^T * P^T.  k slot j of lane half hf in token step kk is
    // token 16 kk + (j/4)*8 + 4 hf + j%4; the transposed read gives lane l latent column l%32 of
    // 4 such tokens (source lane s of each 16-lane group supplies token row s/4, columns
    // 4(s%4)..+3).
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      mfma_acc_a(o[m >> 1], ring[m & 3], pk[m & 1]);
      if (m + 4 < 32) ring[m & 3] = read_op(36 + m + 4);
    }

    // advance the read offsets to the next tile's buffer
    const int step = (t % kNumBufs) == kNumBufs - 1 ? -(kNumBufs - 1) * kBufBytes : kBufBytes;
#pragma unroll
    for (int k = 0; k < 8; ++k) qk_a[k] += step;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      qk_b[k] += step;
      pv_lo[k] += step;
      pv_hi[k] += step;
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  acc_wait_mfma();
#pragma unroll
  for (int cb = 0; cb < 16; ++cb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x4 v = {acc_read_scaled(o[cb][4 * g], inv), acc_read_scaled(o[cb][4 * g + 1], inv),
                 acc_read_scaled(o[cb][4 * g + 2], inv), acc_read_scaled(o[cb][4 * g + 3], inv)};
      *(f32x4*)(o_ptr + 32 * cb + 8 * g) = v;
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
  float m_run = -INFINITY, l_run = 0.f, acc0 = 0.f, acc1 = 0.f;
  for (int start = w.tok_begin; start < w.tok_end; start += 256) {
    const int tkn = start + tid;
    float z = -INFINITY;
    if (tkn < w.tok_end) {
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
    const float alpha = expf(m_run - m_new);
    const float p = tkn < w.tok_end ? expf(z - m_new) : 0.f;
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
  float* o_ptr = a.o_out + (w.out_row + h) * kDc;
  const bool empty = w.tok_end <= w.tok_begin;
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

__global__ __launch_bounds__(256) void lse_merge_kernel(const float* __restrict__ o_part,
                                                        const float* __restrict__ lse_part, float* __restrict__ o_lat,
                                                        float* __restrict__ lse, int num_splits) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int rh = xcd_remap(blockIdx.x, gridDim.x) * 4 + wave;  // row * kHeads + h
  const int row = rh / kHeads, h = rh % kHeads;
  const size_t base = (size_t)row * num_splits * kHeads + h;  // split k at base + k * kHeads
  const float* lp = lse_part + base;
  const float* op = o_part + base * kDc + 8 * lane;
  constexpr float kLog2e = 1.4426950408889634f;
  auto lse_of = [&](int k) { return k < num_splits ? lp[(size_t)k * kHeads] : -INFINITY; };

  f32x4 x0[8], x1[8];
  auto load_batch = [&](int kb) {  // splits kb .. kb+7 (clamped to the last one)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = kb + j < num_splits ? kb + j : num_splits - 1;
      const f32x4* src = (const f32x4*)(op + (size_t)k * kHeads * kDc);
      x0[j] = src[0];
      x1[j] = src[1];
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
      a0 += w * x0[j];
      a1 += w * x1[j];
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
  const int nwg = rows * a.num_splits;
  if (a.dtype_bf16)
    hipLaunchKernelGGL(decode_attn_bf16_kernel, dim3(nwg), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(decode_attn_f32_kernel, dim3(nwg * kHeads), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_lse_merge(const float* o_part, const float* lse_part, float* o_lat, float* lse, int rows,
                            int num_splits, hipStream_t stream) {
  hipLaunchKernelGGL(lse_merge_kernel, dim3(rows * (kHeads / 4)), dim3(256), 0, stream, o_part, lse_part, o_lat,
                     lse, num_splits);
  return hipGetLastError();
}

}  // namespace mla
