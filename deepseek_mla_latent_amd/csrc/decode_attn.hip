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
//   * the key range is walked in tiles of 32 tokens (half a page), streamed HBM -> LDS by
//     direct-to-LDS loads (16 B per lane, no register staging): the latent rows into a ring of 4
//     buffers, the RoPE-key rows into a ring of 3, two tiles ahead (attn_schedule.h);
//   * each LDS tile is XOR-swizzled in 16-byte units so that both read patterns below are free of
//     bank conflicts;
//   * scores: wave w takes heads 32w..32w+31.  S^T = tile * Q^T on 32x32x16 bf16 MFMAs, the tile as
//     the A operand (ds_read_b128), the wave's [q_lat | q_pe] in registers as the B operand.  Each
//     lane ends up with one head and 16 tokens, which is already the B-operand layout of the
//     weighted sum (no cross-lane shuffle for P);
//   * online softmax in base 2 with the scale folded in; the running max is only raised (and O
//     rescaled) when a tile's max exceeds it by more than 2^8;
//   * weighted sum: wave w holds O^T for latent columns 128w..128w+127 of all 128 heads.  The
//     probabilities of a tile pass between the waves through LDS (32 tokens x 128 heads, 8 KiB), so
//     each transposed A operand (ds_read_b64_tr_b16 from the same LDS tile: c_KV is key and value)
//     feeds four MFMAs, one per head block.  Per tile a wave reads 52 KiB from LDS in 60
//     instructions instead of the 68 KiB in 100 that a wave holding all 512 columns of its own 32
//     heads needs;
//   * iteration u: scores of tile u, then the weighted sum of tile u-1 with the softmax of tile u
//     in the gaps of its MFMA chain; one workgroup barrier per tile.
// Long contexts are split into page ranges (split-K over tokens); each range writes a normalised
// partial (o_k, lse_k) and lse_merge_kernel (or the merge in the out-projection) combines them.
// Tree-masked verify (EAGLE-style draft trees: the Perplexity post, section "Будущая работа"): the
// S new tokens are tree nodes cached at positions L-S .. L-1, parents before children; query i
// sees the committed keys and the keys of its ancestors and itself.  The row's visibility of the
// S new keys is one 64-bit mask (S <= 64), built once per workgroup by walking parent links and
// applied only to tiles that reach position L-S.
#include "attn_schedule.h"
#include "common.h"
#include "kernels.h"

namespace mla {

constexpr int kTile = 32;                        // tokens per LDS tile (half a page)
constexpr int kUnitsA = kDc / 8;                 // 16-byte units of c_KV per token (64)
constexpr int kUnitsB = kDr / 8;                 // 16-byte units of k_pe per token (8)
constexpr int kBufA = kTile * kUnitsA * 16;      // 32768 B: latent rows of a tile
constexpr int kBufB = kTile * kUnitsB * 16;      // 4096 B: RoPE-key rows of a tile
constexpr int kBufP = 4 * 2 * 64 * 16;           // 8192 B: bf16 P of a tile, [head block][token half][lane]
// LDS layout of the bf16 kernel (bytes)
constexpr int kOffB = kNumBufsA * kBufA;                 // ring B
constexpr int kOffP = kOffB + kNumBufsB * kBufB;         // ring P
constexpr int kOffAlpha = kOffP + kNumBufsP * kBufP;     // per ring-P buffer: rescale factor per head
constexpr int kOffFlags = kOffAlpha + kNumBufsP * kHeads * 4;  // per ring-P buffer: rescale flag per head block
constexpr int kOffInvL = kOffFlags + kNumBufsP * 16;     // final 1 / sum of weights per head
constexpr int kOffPages = kOffInvL + kHeads * 4;         // page ids of the range
constexpr int kOffTree = kOffPages + kMaxSplitPages * 4;  // draft-tree masked-key windows (12 words)
constexpr int kLdsBytes = kOffTree + 12 * 4;
static_assert(kLdsBytes <= 160 * 1024, "LDS of one workgroup");
static_assert(kNumBufsA * kBufA >= kHeads * 1024, "the query rows are staged through ring A");
constexpr int kStageRow = kDc * 2 + 16;  // bf16 output row staged in LDS (1040 B: 2-way bank conflicts)
static_assert(kHeads * kStageRow <= kOffP, "output staging fits in rings A and B");
constexpr int kDmaPerTile = 9;           // direct-to-LDS loads per wave per tile
constexpr float kRescaleSlack = 8.0f;    // log2 units

__device__ __forceinline__ uint32_t lds_addr(const MLA_LDS char* p) { return (uint32_t)(uintptr_t)p; }

// Swizzle: 16-byte unit u of token t is stored at unit (u ^ swz(t)) of the token's LDS row.
// Ring A (64 units per row): bit-rotated low 4 bits of t, so 16 consecutive tokens at one unit
// (the score A-operand read) and 8 tokens x 4 units (the transposed read) both spread over banks.
__device__ __forceinline__ int swz_a(int t) { return ((t & 3) << 2) | ((t >> 2) & 3); }
__device__ __forceinline__ int swz_b(int t) { return (t >> 1) & 7; }
__device__ __forceinline__ int off_a(int t, int u) { return (t * kUnitsA + (u ^ swz_a(t))) * 16; }

// Direct-to-LDS load of 16 bytes per lane from a wave-uniform base plus a 32-bit per-lane byte
// offset: lane l's bytes land at LDS address lds + 16 l.  Issued from asm: the compiler models
// this instruction as pending in the LDS counter as well, which would turn every LDS operand wait
// of the tile computed meanwhile into a full drain.  It has no register outputs; completion is
// awaited explicitly (dma_wait_tiles) before the barrier that publishes a tile.  M0 is not
// otherwise used by this kernel.  The loads carry the non-temporal hint: cache rows are read once
// per step, and streamed without it they push out of L2 and the MALL the weights and split
// partials that the projection and merge kernels of the same step read back (with it, those
// kernels and this one each ran faster, 3-4 us per step on every decode workload).
__device__ __forceinline__ void dma16_s(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase), "s"(lds)
               : "memory");
}
// Wait until at most `younger` tiles' loads (kDmaPerTile each) of this wave are still in flight.
// Vector-memory loads complete in order, so this retires every older tile; loads the compiler
// issues itself only ever make the wait stricter.
__device__ __forceinline__ void dma_wait_tiles(int younger) {
  if (younger >= 1)
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

// MFMAs are issued from asm volatile statements with a memory clobber: the compiler keeps them in
// program order and cannot move the LDS operand loads (ordinary builtins, whose waits it still
// inserts exactly) across them, so the software pipeline below is executed as written.  Being
// opaque, these statements also hide hazards from the compiler; the few that matter are handled
// explicitly:
//   * VALU write -> MFMA source read needs 2 wait states: the first score MFMA takes SrcC = 0
//     (no VALU zeroing), and the VALU rescale of O is followed by s_nop 4;
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

// ---- key ranges.  With num_splits = k > 1 the grid has G = rows * k workgroups, each one key range
// of one row (row r = b S + i).  Up to kPlanRows rows the ranges follow the rows' lengths, so that
// a ragged batch does not leave its longest rows' workgroups walking while the others idle:
//   P_r  = pages of the keys row r sees, capped at k * pages_per_split (all the fixed ranges cover);
//   C    = the smallest page count with sum_r max(1, ceil(P_r / C)) <= G (C <= pages_per_split, which
//          always fits);
//   row r gets s_r = max(1, ceil(P_r / C)) ranges of C pages (the last one shorter, an empty row one
//   empty range), numbered row after row: range j of row r is workgroup and partial slot first_r + j
//   (first_r = s_0 + .. + s_{r-1}); workgroups past the last range have nothing to do.
// Rows with equal page counts P get C = max(1, ceil(P / k)) and ceil(P / C) ranges each: the k fixed
// ranges whenever P spans them.  Above kPlanRows rows every row gets the k fixed ranges of
// pages_per_split pages.  Every wave computes the plan itself from seq_lens (wave-uniform results,
// no barrier): equal counts in closed form; otherwise C by bisection between the bounds
// ceil(T / G) <= C <= ceil(T / (G - rows)) (T = sum_r P_r; max(1, ceil(x)) <= x + 1 makes the upper
// one fit), and the slots by a prefix sum over the rows.

// Inclusive prefix sum over each row of 16 lanes (DPP row shifts).
__device__ __forceinline__ int row16_scan(int v, int lane) {
  int t = __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  if ((lane & 15) >= 1) v += t;
  t = __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  if ((lane & 15) >= 2) v += t;
  t = __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  if ((lane & 15) >= 4) v += t;
  t = __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  if ((lane & 15) >= 8) v += t;
  return v;
}
// Sum over the wave (every lane gets it), from the row scans' last lanes.
__device__ __forceinline__ int wave_total(int scanned) {
  return (__builtin_amdgcn_readlane(scanned, 15) + __builtin_amdgcn_readlane(scanned, 31)) +
         (__builtin_amdgcn_readlane(scanned, 47) + __builtin_amdgcn_readlane(scanned, 63));
}
// ceil(p / c) for p >= 0, c >= 1 (rc = 1 / c, within an ulp).  Below 2^22 the quotient from the
// reciprocal is off by at most one, and one correction each way makes it exact; larger p (not met
// by any batch that fits a GPU's memory) take the integer division.
__device__ __forceinline__ int ceil_div_small(int p, int c, float rc) {
  if (p >= (1 << 22)) return (int)(((unsigned)p + (unsigned)c - 1u) / (unsigned)c);
  int q = (int)((float)p * rc);
  int r = p - q * c;
  q += (r >= c ? 1 : 0) - (r < 0 ? 1 : 0);
  r = p - q * c;
  return q + (r > 0 ? 1 : 0);
}

// floor(p / c), likewise.
__device__ __forceinline__ int floor_div_small(int p, int c, float rc) {
  if (p >= (1 << 22)) return (int)((unsigned)p / (unsigned)c);
  int q = (int)((float)p * rc);
  const int r = p - q * c;
  return q + (r >= c ? 1 : 0) - (r < 0 ? 1 : 0);
}

// Keys row r = b S + i sees (the decode rule: causal without a tree, else all L).
__device__ __forceinline__ int visible_keys(const AttnArgs& a, int L, int i) {
  int n = a.causal && !a.tree_parents ? L - a.S + i + 1 : L;
  return n < 0 ? 0 : (n > L ? L : n);
}

struct RangePlan {
  int r, j;          // row and key range of this workgroup
  int first, count;  // the row's first partial slot and number of ranges
  int chunk;         // pages per range
  int L;             // cached tokens of the row's sequence (-1: not loaded yet)
  bool live;         // false: past the last range
  bool fixed;        // every row has k ranges (slot r k + j), as without the plan
};

// The common case, every row seeing the same number of keys, is recognised from scalar loads of
// seq_lens (at most kUniformScan sequences, each row seeing its whole sequence): one round trip,
// like the single length a workgroup loads without the plan, and a closed form after it.  They read
// seq_lens through the constant address space (the kernel never writes it, and each launch starts
// its scalar cache afresh), which keeps them scalar wherever they stand.
constexpr int kUniformScan = 32;
typedef __attribute__((address_space(4))) const int32_t const_i32;
struct LenScan {
  int v[kUniformScan];
  bool on;
};
__device__ __forceinline__ LenScan scan_lengths(const AttnArgs& a) {
  LenScan ls;
  ls.on = a.num_splits > 1 && a.B * a.S <= kPlanRows && a.B <= kUniformScan &&
          !(a.S > 1 && a.causal && !a.tree_parents);
  if (ls.on) {
    const_i32* sl = (const_i32*)a.seq_lens;
    if (a.B == kUniformScan) {  // all in bounds: contiguous, so merged into wide scalar loads
#pragma unroll
      for (int q = 0; q < kUniformScan; ++q) ls.v[q] = sl[q];
    } else if (a.B <= 8) {  // entries past B repeat sequence 0
#pragma unroll
      for (int q = 0; q < kUniformScan; ++q) ls.v[q] = sl[q < 8 && q < a.B ? q : 0];
    } else {
#pragma unroll
      for (int q = 0; q < kUniformScan; ++q) ls.v[q] = sl[q < a.B ? q : 0];
    }
  }
  return ls;
}
// The length every sequence has, or -1 (lengths differ, or no scan).
__device__ __forceinline__ int uniform_length(const AttnArgs& a, LenScan& ls) {
  if (!ls.on) return -1;
  int diff = 0;
#pragma unroll
  for (int q = 1; q < kUniformScan; ++q) diff |= ls.v[q] ^ ls.v[0];
  return diff == 0 ? checked_len(a.bounds, ls.v[0]) : -1;
}

// Longest first.  With more ranges than compute units, the workgroups past the first wave start
// as earlier ones finish, in workgroup order; ordering the ranges by decreasing length then pairs
// the short ranges of the second wave with the compute units whose first range was short (the
// longest-processing-time rule).  Row r's ranges are f_r = floor(P_r / C) full ranges of C pages
// and, when C does not divide P_r (or P_r = 0), one remainder range of P_r - f_r C pages.
// Workgroup `pos` (dispatch order) takes:
//   pos < F = sum f_r: full range t = xcd_remap(pos, F) in row-major order, so that a row's full
//     ranges share an XCD;
//   F <= pos < F + R: the remainder of rank pos - F, ranks by decreasing size, ties by row;
//   otherwise nothing.
// Partial slots stay row-major (row r's ranges at first_r .. first_r + s_r - 1, s_r = f_r + [it
// has a remainder]), the layout the merges read from the row table.
__device__ __forceinline__ RangePlan plan_longest_first(const AttnArgs& a, const int* P, const int* Ls, int C,
                                                        float rc, RangePlan p) {
  constexpr int M = kPlanRows / 64;
  const int k = a.num_splits;
  const int lane = threadIdx.x & 63;
  const int pos = blockIdx.x;
  int f[M], rem[M], sfirst[M], ffirst[M];
  bool has[M];
  int base_s = 0, base_f = 0;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    f[m] = 0;
    rem[m] = 0;
    has[m] = false;
    if (P[m] >= 0) {
      f[m] = floor_div_small(P[m], C, rc);
      rem[m] = P[m] - f[m] * C;
      has[m] = rem[m] > 0 || P[m] == 0;
    }
    const int sm = f[m] + (has[m] ? 1 : 0);
    p.fixed = p.fixed && __ballot(P[m] >= 0 && sm != k) == 0;
    const int scs = row16_scan(sm, lane), scf = row16_scan(f[m], lane);
    const int q16 = lane >> 4;
    const int s15 = __builtin_amdgcn_readlane(scs, 15), s31 = __builtin_amdgcn_readlane(scs, 31),
              s47 = __builtin_amdgcn_readlane(scs, 47), s63 = __builtin_amdgcn_readlane(scs, 63);
    const int f15 = __builtin_amdgcn_readlane(scf, 15), f31 = __builtin_amdgcn_readlane(scf, 31),
              f47 = __builtin_amdgcn_readlane(scf, 47), f63 = __builtin_amdgcn_readlane(scf, 63);
    sfirst[m] = base_s + (q16 >= 1 ? s15 : 0) + (q16 >= 2 ? s31 : 0) + (q16 >= 3 ? s47 : 0) + scs - sm;
    ffirst[m] = base_f + (q16 >= 1 ? f15 : 0) + (q16 >= 2 ? f31 : 0) + (q16 >= 3 ? f47 : 0) + scf - f[m];
    base_s += (s15 + s31) + (s47 + s63);
    base_f += (f15 + f31) + (f47 + f63);
  }
  const int F = base_f, NR = base_s;  // full ranges; all ranges
  int r = -1, m_hit = 0, l_hit = 0, j = 0;
  if (pos < F) {
    const int t = xcd_remap(pos, F);
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const uint64_t hit = __ballot(f[m] > 0 && t >= ffirst[m] && t < ffirst[m] + f[m]);
      if (hit) {
        m_hit = m;
        l_hit = __builtin_ctzll(hit);
        r = 64 * m + l_hit;
        j = t - __builtin_amdgcn_readlane(ffirst[m], l_hit);
      }
    }
  } else if (pos < NR) {
    const int q = pos - F;
    auto count_ge = [&](int v) {  // rows whose remainder range has at least v pages
      int c = 0;
#pragma unroll
      for (int m = 0; m < M; ++m) c += __builtin_popcountll(__ballot(has[m] && rem[m] >= v));
      return c;
    };
    int lo = 0, hi = C - 1;  // the remainder of rank q has the largest size v with count_ge(v) > q
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (count_ge(mid) > q)
        lo = mid;
      else
        hi = mid - 1;
    }
    int t = q - (lo + 1 <= C - 1 ? count_ge(lo + 1) : 0);  // rank among the rows of that size
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const bool eq = has[m] && rem[m] == lo;
      const uint64_t mask = __ballot(eq);
      const int c = __builtin_popcountll(mask);
      if (r < 0 && t < c) {
        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
        const uint64_t sel = __ballot(eq && below == t);
        m_hit = m;
        l_hit = __builtin_ctzll(sel);
        r = 64 * m + l_hit;
        j = __builtin_amdgcn_readlane(f[m], l_hit);
      } else if (r < 0) {
        t -= c;
      }
    }
  }
  if (r >= 0) {
    int sf = sfirst[0], fr = f[0], L = Ls[0];
    bool hs = has[0];
#pragma unroll
    for (int m = 1; m < M; ++m)
      if (m_hit == m) {
        sf = sfirst[m];
        fr = f[m];
        L = Ls[m];
        hs = has[m];
      }
    p.r = r;
    p.j = j;
    p.first = __builtin_amdgcn_readlane(sf, l_hit);
    p.count = __builtin_amdgcn_readlane(fr + (hs ? 1 : 0), l_hit);
    p.L = __builtin_amdgcn_readlane(L, l_hit);
    p.live = true;
  }
  return p;
}

// L0: the common length of all sequences when every row sees all of its keys, else -1.
// With a range budget above rows * k (set by the host only for at most kPlanRows rows), rows of
// unequal length get up to that many ranges, dispatched longest first (see the end of this
// function); equal rows keep the k-per-row numbering over the first rows * k workgroups.
__device__ RangePlan plan_ranges(const AttnArgs& a, int g, int L0) {
  const int rows = a.B * a.S, k = a.num_splits, pps = a.pages_per_split;
  const bool longest_first = a.range_budget > rows * k;
  if (longest_first) g = (int)blockIdx.x < rows * k ? xcd_remap(blockIdx.x, rows * k) : rows * k;
  RangePlan p;
  if (rows > kPlanRows) {
    p.r = g / k;
    p.j = g % k;
    p.first = p.r * k;
    p.count = k;
    p.chunk = pps;
    p.L = -1;
    p.live = true;
    p.fixed = true;
    return p;
  }
  const int lane = threadIdx.x & 63;
  const int cap = k * pps;
  const int G = longest_first ? a.range_budget : rows * k;  // ranges the rows of unequal length may take
  if (L0 >= 0) {  // every row sees all L0 keys: the closed form below, from P = pages of L0
    const int pg = (L0 + kPage - 1) / kPage;
    const int P0 = pg < cap ? pg : cap;
    int C = (P0 + k - 1) / k;
    C = C > 1 ? C : 1;
    int sr = (P0 + C - 1) / C;
    sr = sr > 1 ? sr : 1;
    p.r = sr == k ? g / k : g / sr;
    p.j = g - p.r * sr;
    p.first = p.r * sr;
    p.count = sr;
    p.chunk = C;
    p.live = p.r < rows;
    p.fixed = sr == k;
    p.L = L0;
    return p;
  }
  int P[kPlanRows / 64];   // pages of keys row lane + 64 m sees, capped (-1: no such row)
  int Ls[kPlanRows / 64];  // its sequence's cached tokens
  int tp = 0;
#pragma unroll
  for (int m = 0; m < kPlanRows / 64; ++m) {
    const int r = lane + 64 * m;
    P[m] = -1;
    Ls[m] = 0;
    if (r < rows) {
      const int b = a.S == 1 ? r : r / a.S;
      Ls[m] = checked_len(a.bounds, a.seq_lens[b]);
      const int n = visible_keys(a, Ls[m], r - b * a.S);
      const int pg = (n + kPage - 1) / kPage;
      P[m] = pg < cap ? pg : cap;
      tp += P[m];
    }
  }
  // All rows with the same page count P (the common case): C = max(1, ceil(P / k)) is the smallest
  // with ceil(P / C) <= k, and every row gets ceil(P / C) ranges.
  const int P0 = __builtin_amdgcn_readfirstlane(P[0]);
  bool same = true;
#pragma unroll
  for (int m = 0; m < kPlanRows / 64; ++m)
    if (64 * m < rows) same = same && __ballot(P[m] >= 0 && P[m] != P0) == 0;
  if (__builtin_expect(same, 1)) {
    int C = ceil_div_small(P0, k, __builtin_amdgcn_rcpf((float)k));
    C = C > 1 ? C : 1;
    int sr = ceil_div_small(P0, C, __builtin_amdgcn_rcpf((float)C));
    sr = sr > 1 ? sr : 1;
    p.r = sr == k ? g / k : floor_div_small(g, sr, __builtin_amdgcn_rcpf((float)sr));
    p.j = g - p.r * sr;
    p.first = p.r * sr;
    p.count = sr;
    p.chunk = C;
    p.live = p.r < rows;
    p.fixed = sr == k;
    const int rm = p.r < rows ? p.r : 0;
    int Lr = Ls[0];
#pragma unroll
    for (int m = 1; m < kPlanRows / 64; ++m)
      if ((rm >> 6) == m) Lr = Ls[m];
    p.L = __builtin_amdgcn_readlane(Lr, rm & 63);
    return p;
  }
  const int T = wave_total(row16_scan(tp, lane));
  auto ranges = [&](int c) {  // sum over rows of max(1, ceil(P_r / c))
    const float rc = __builtin_amdgcn_rcpf((float)c);
    int v = 0;
#pragma unroll
    for (int m = 0; m < kPlanRows / 64; ++m)
      if (P[m] >= 0) {
        const int q = ceil_div_small(P[m], c, rc);
        v += q > 1 ? q : 1;
      }
    return wave_total(row16_scan(v, lane));
  };
  int lo = (T + G - 1) / G, hi = (T + (G - rows) - 1) / (G - rows);
  lo = lo > 1 ? lo : 1;
  hi = hi < pps ? hi : pps;
  hi = hi > lo ? hi : lo;
  while (lo < hi) {  // wave-uniform bisection
    const int mid = (lo + hi) >> 1;
    if (ranges(mid) <= G)
      hi = mid;
    else
      lo = mid + 1;
  }
  const int C = lo;
  const float rc = __builtin_amdgcn_rcpf((float)C);
  p.live = false;
  p.r = p.j = p.first = p.count = p.L = 0;
  p.chunk = C;
  p.fixed = true;
  if (longest_first) return plan_longest_first(a, P, Ls, C, rc, p);
  int base = 0;  // slots of the rows before this group of 64
#pragma unroll
  for (int m = 0; m < kPlanRows / 64; ++m) {
    if (64 * m >= rows) break;
    int sr = 0;
    if (P[m] >= 0) {
      sr = ceil_div_small(P[m], C, rc);
      sr = sr > 1 ? sr : 1;
    }
    const int sc = row16_scan(sr, lane);
    const int r15 = __builtin_amdgcn_readlane(sc, 15), r31 = __builtin_amdgcn_readlane(sc, 31),
              r47 = __builtin_amdgcn_readlane(sc, 47), r63 = __builtin_amdgcn_readlane(sc, 63);
    const int q16 = lane >> 4;
    const int before = (q16 >= 1 ? r15 : 0) + (q16 >= 2 ? r31 : 0) + (q16 >= 3 ? r47 : 0);
    const int first = base + before + sc - sr;
    p.fixed = p.fixed && __ballot(P[m] >= 0 && sr != k) == 0;
    const uint64_t hit = __ballot(sr > 0 && g >= first && g < first + sr);
    if (hit) {
      const int l = __builtin_ctzll(hit);
      p.r = 64 * m + l;
      p.first = __builtin_amdgcn_readlane(first, l);
      p.count = __builtin_amdgcn_readlane(sr, l);
      p.L = __builtin_amdgcn_readlane(Ls[m], l);
      p.j = g - p.first;
      p.live = true;
    }
    base += (r15 + r31) + (r47 + r63);
  }
  return p;
}

// Token range and output slots of one workgroup; shared by both dtypes.
struct WorkItem {
  int b, i, split;
  int tok_begin, tok_end;  // [tok_begin, tok_end) of sequence b, page aligned at tok_begin
  int tail;                // L - S: position of the first new token (node 0 of a draft tree)
  size_t out_row;          // index of (head 0) in the o/lse output rows
  int plan_first, plan_count;  // the row's partial slots (num_splits > 1)
  bool live;               // false: a workgroup past the last key range
  bool plan_fixed;         // every row's slots are r * num_splits + j (num_splits > 1)
};

// L0: as for plan_ranges.
__device__ __forceinline__ WorkItem make_work(const AttnArgs& a, int id, int L0) {
  WorkItem w;
  int chunk = a.pages_per_split, r, L = -1;
  w.split = 0;
  w.plan_first = w.plan_count = 0;
  w.live = true;
  w.plan_fixed = true;
  if (a.num_splits > 1) {
    const RangePlan p = plan_ranges(a, id, L0);
    r = p.r;
    w.split = p.j;
    w.plan_first = p.first;
    w.plan_count = p.count;
    w.live = p.live;
    w.plan_fixed = p.fixed;
    chunk = p.chunk;
    L = p.L;
  } else {
    r = id;
  }
  w.i = r % a.S;
  w.b = r / a.S;
  if (L < 0) L = checked_len(a.bounds, a.seq_lens[w.b]);
  const int n = visible_keys(a, L, w.i);
  w.tok_begin = w.split * chunk * kPage;
  w.tail = L - a.S;
  const int e = (w.split + 1) * chunk * kPage;
  w.tok_end = e < n ? e : n;
  w.out_row = a.final_out ? (size_t)r * kHeads : (size_t)(w.plan_first + w.split) * kHeads;
  return w;
}

// With num_splits > 1 the first range of every row records the row's slots for the merges (word
// 4 + 2 r: first slot, 4 + 2 r + 1: count), and that of row 0 whether every row has the fixed
// slots r * num_splits + j (word 0: 1 if so), so that the merges need not read the rows' entries.
__device__ __forceinline__ void record_row_plan(const AttnArgs& a, const WorkItem& w) {
  if (a.row_plan && w.live && w.split == 0 && threadIdx.x == 0) {
    const int r = w.b * a.S + w.i;
    if (r == 0) a.row_plan[0] = w.plan_fixed ? 1 : 0;
    a.row_plan[4 + 2 * r] = w.plan_first;
    a.row_plan[4 + 2 * r + 1] = w.plan_count;
  }
}

template <bool kTree>
__global__ __launch_bounds__(256, 1) void decode_attn_bf16_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds_raw[kLdsBytes];
  MLA_LDS char* const smem = (MLA_LDS char*)lds_raw;
  // Page ids of the range, then for kTree 12 words: word 0 = the first tile of the range that
  // reaches a draft-tree key; words 2-3 = zeros (no key of an earlier tile is masked); words 4-11
  // = the masked-key windows of that tile and the next three, two per tile (lanes 0-31, lanes
  // 32-63).  Read back per tile: held in registers across the loop they would not fit.
  MLA_LDS int* const lds_pages = (MLA_LDS int*)(smem + kOffPages);
  MLA_LDS int* const lds_tree = (MLA_LDS int*)(smem + kOffTree);

  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, hf = lane >> 5;

  // The rows' lengths for the key-range plan (scalar loads, before anything else).
  LenScan lens = scan_lengths(a);
  const WorkItem w = make_work(a, id, uniform_length(a, lens));
  if (!w.live) return;  // past the last key range (uniform over the workgroup)
  record_row_plan(a, w);
  // kTree: node `lane`'s parent, loaded here and walked once the query prologue has waited for its
  // loads
  const int tpar = kTree ? tree_parent_of_lane(a.tree_parents, w.b, a.S, lane) : -1;

  // Final outputs are fp32 (written by this kernel's lanes directly); split partials are bf16
  // rows (the merge widens them again), staged through LDS so each store writes a whole row.
  const int ntok = w.tok_end - w.tok_begin;
  if (ntok <= 0) {  // empty key range: o = 0, lse = -inf (wave w writes the rows of its 32 heads)
    const size_t row = w.out_row + wave * 32 + l32;
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < kDc / 8; c += 2) {  // this lane: 16-byte pieces hf, hf + 2, .. of the row
      const int col = (c + hf) * 8;
      if (a.final_out) {
        *(f32x4*)((float*)a.o_out + row * kDc + col) = z;
        *(f32x4*)((float*)a.o_out + row * kDc + col + 4) = z;
      } else {
        *(u32x4*)((uint16_t*)a.o_out + row * kDc + col) = u32x4{0u, 0u, 0u, 0u};
      }
    }
    if (hf == 0 && a.lse_out) a.lse_out[row] = -INFINITY;
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
  // round trips overlap; the barrier that hands ring A to the tiles also publishes them.
  const int npages = (ntok + kPage - 1) / kPage;
  constexpr int kPidPerThread = kMaxSplitPages / 256;
  int pid[kPidPerThread];
#pragma unroll
  for (int k = 0; k < kPidPerThread; ++k) {
    const int j = threadIdx.x + 256 * k;
    pid[k] = j < npages ? checked_page(a.bounds, bt[j]) : 0;
  }
  auto row_of = [&](int t, int page) -> const uint16_t* {  // first token row of tile t
    return pool + ((size_t)page * kPage + (t & 1) * kTile) * kRow;
  };
  auto tile_count = [&](int t) { return ntok - t * kTile < kTile ? ntok - t * kTile : kTile; };

  // One step of copying a tile (cnt valid tokens, rows from `src`) into ring-A buffer dst_a and
  // ring-B buffer dst_b: steps 0-7 fill this wave's 8 tokens' 1 KiB c_KV rows, step 8 the 128 B
  // k_pe rows of 8 tokens.  Tokens past cnt re-read token 0 (always valid), so LDS never holds
  // bytes from outside the sequence; their scores are masked.  lane16 = 16 * lane: the per-lane
  // part of every address is one XOR with a wave-uniform value (0 for loads past the last tile,
  // which then all read the first 16 bytes of the pool).
  auto dma_step = [&](const uint16_t* src, int cnt, uint32_t dst_a, uint32_t dst_b, int k, uint32_t lane16) {
    const char* base = (const char*)src;
    if (k < 8) {
      const int t = wave * 8 + k;  // wave-uniform
      const int ts = t < cnt ? t : 0;
      dma16_s(base + ts * (kRow * 2), lane16 ^ (swz_a(t) * 16), dst_a + t * 1024);
    } else {
      const int t = wave * 8 + (int)(lane16 >> 7);
      const int ts = t < cnt ? t : 0;
      const uint32_t u = ((lane16 >> 4) & 7) ^ swz_b(t);
      dma16_s(base, ts * (kRow * 2) + kDc * 2 + u * 16, dst_b + wave * 1024);
    }
  };
  struct Group {  // the nine loads of one tile (or of none, past the last tile)
    const uint16_t* src;
    int cnt;
    uint32_t dst_a, dst_b, lane16;
  };
  auto make_group = [&](int u, int page, uint32_t lane16_live) -> Group {
    const bool live = u < ntiles;
    Group g;
    g.src = live ? row_of(u, page) : pool;
    g.cnt = live ? tile_count(u) : 0;
    g.dst_a = lds_addr(smem) + attn_a_buffer(u) * kBufA;
    g.dst_b = lds_addr(smem) + kOffB + attn_b_buffer(u) * kBufB;
    g.lane16 = live ? lane16_live : 0u;
    return g;
  };

  // Prologue.  The query rows come in first, through ring A: each wave copies its 32 heads' q_lat
  // rows (1 KiB each, one load per row, 16-byte unit u of row r stored at u ^ (r & 15)) and reads
  // its B operands from there; q_pe (4 loads) comes straight from memory.
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
  __syncthreads();  // every wave has its q and the page ids are in LDS: ring A takes the tiles now
#pragma unroll
  for (int u = 0; u < kLoadAhead; ++u) {
    const Group g = make_group(u, u < ntiles ? __builtin_amdgcn_readfirstlane(lds_pages[u >> 1]) : 0, lane * 16);
#pragma unroll
    for (int k = 0; k < kDmaPerTile; ++k) dma_step(g.src, g.cnt, g.dst_a, g.dst_b, k, g.lane16);
  }

  // Per-lane LDS byte offsets of the swizzled reads.
  // Score operand g of the tile in ring-A buffer at A0 / ring-B buffer at B0 (g < 32: latent
  // units 2 (g & 7) + hf + 16 (g >> 3); g >= 32: k_pe units 2 (g - 32) + hf):
  //   (A0 + xa) ^ 32 (g & 7), plus 256 (g >> 3);  (B0 + xb) ^ 32 (g - 32).
  // The XOR only touches bits 5-7, which in A0 + xa / B0 + xb come from the swizzled unit alone.
  const uint32_t xa = l32 * 1024 + 16 * (hf ^ swz_a(l32));
  const uint32_t xb = l32 * 128 + 16 * (hf ^ swz_b(l32));
  // Weighted-sum A operand (tile^T) for latent block 4 wave + c, token half kk: the transposed
  // read pair at pv_lo[c] / pv_hi[c] + 16384 kk of the summed tile's ring-A buffer; lanes get the
  // tokens in the same order as the score accumulator hands them to the softmax.
  int pv_lo[4], pv_hi[4];
  {
    const int r4 = (lane >> 2) & 3;
    const int colq = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const int tb = 4 * hf + r4;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = 32 * k + colq;
      pv_lo[k] = off_a(tb, c >> 3) + (c & 7) * 2 + 256 * wave;
      pv_hi[k] = off_a(tb + 8, c >> 3) + (c & 7) * 2 + 256 * wave;
    }
  }
  const uint32_t p_lane = kOffP + lane * 16;  // ring P: [buffer][head block][token half][lane] x 16 B

  f32x16 o[16];  // o[4 c + hb]: O^T for latent block 4 wave + c, heads 32 hb .. 32 hb + 31
#pragma unroll
  for (int k = 0; k < 16; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[k][e] = 0.f;
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
  // its instructions can ride between the MFMAs of the weighted sum.  Masked keys get a raw score
  // of -inf.  Output: P in bf16 (pk), already in the B layout of the weighted sum, and for the
  // other waves the rescale factor of each of this wave's heads.
  bf16x8 pk[2];
  float mx[5], mt = 0.f, alpha = 1.f;
  bool rescale = false;  // wave-uniform
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
      // Branch-free on purpose: a branch here lets the compiler duplicate the rest of the chain
      // per outcome.  O itself is rescaled (by every wave) before the next weighted sum.
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
  constexpr int kSoftmaxStages = 34;

  // kTree: raw scores of tile t.  A key of a node that is neither the query's node nor one of its
  // ancestors gets -inf; committed keys stay.  Tiles before the first one that reaches the tree
  // keep everything; a range meets at most four such tiles (64 nodes).
  // Element e: a signed extract of its masked-key bit (0 or all ones) selects the score or -inf
  // (an instruction literal), two temporaries at a time.  The LDS address and the lane half are
  // hidden from loop-invariant code motion, which would otherwise pin registers across the loop.
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

  f32x16 s;           // raw scores of the tile being scored
  bf16x8 ring[4];     // score A operands in flight
  bf16x8 pp[8];       // weighted-sum B operands: P of the summed tile, [token half * 4 + head block]
  bf16x8 apv[3];      // weighted-sum A operands in flight (group j of four MFMAs uses apv[j % 3])
  uint32_t flags = 0;

  auto read_pv = [&](int c, int kk) -> bf16x8 {
    return lds_read_tr_pair(smem + pv_lo[c] + 16384 * kk, smem + pv_hi[c] + 16384 * kk);
  };
  // P of tile j (all four head blocks) and its rescale flags, from ring P
  auto read_p = [&](int j, int i) -> bf16x8 {  // i = token half * 4 + head block
    const uint32_t base = p_lane + attn_p_buffer(j) * kBufP;
    return lds_read_b128(smem + base + (i & 3) * 2048 + (i >> 2) * 1024);
  };
  auto read_flags = [&](int j) -> uint32_t {
    const u32x4 f = *(const MLA_LDS u32x4*)(smem + kOffFlags + attn_p_buffer(j) * 16);
    return __builtin_amdgcn_readfirstlane(f[0] | (f[1] << 1) | (f[2] << 2) | (f[3] << 3));
  };
  // O columns of the head blocks whose owner raised its reference with tile j: scaled by the
  // owner's factor before tile j's weighted sum adds to them (rare).
  auto rescale_o = [&](int j, uint32_t fl) {
    if (fl != 0) {
      acc_wait_mfma();
#pragma unroll
      for (int hb = 0; hb < 4; ++hb)
        if (fl & (1u << hb)) {
          const float al = *(const MLA_LDS float*)(smem + kOffAlpha + attn_p_buffer(j) * (kHeads * 4) +
                                                   (32 * hb + l32) * 4);
#pragma unroll
          for (int c = 0; c < 4; ++c) acc_scale(o[4 * c + hb], al);
        }
      asm volatile("s_nop 4" ::: "memory");
    }
  };

  // ---- scores of tile t (ring A/B buffers of t), the loads of tile t + 2 (steps 0-4 of 9) and,
  // from step 24 on, the operands of the weighted sum of tile t - 1 (when there is one).
  auto score_chain = [&](int t, bool pv_next) {
    const uint32_t la = (uint32_t)(attn_a_buffer(t) * kBufA) + xa;
    const uint32_t lb = (uint32_t)(kOffB + attn_b_buffer(t) * kBufB) + xb;
    auto rd = [&](int g) -> bf16x8 {
      if (g < 32) return lds_read_b128(smem + ((la ^ (32u * (g & 7))) + 256 * (g >> 3)));
      return lds_read_b128(smem + (lb ^ (32u * (g - 32))));
    };
    const int un = t + kLoadAhead;
    // The per-lane load offsets are loop-invariant; recomputing them (one XOR each) is cheaper than
    // the registers LICM would pin across the loop, so hide the lane id from it.
    uint32_t lane16 = lane * 16;
    asm volatile("" : "+v"(lane16));
#pragma unroll
    for (int k = 0; k < 4; ++k) ring[k] = rd(k);
    // page of tile un, read from LDS here and taken to a scalar register two MFMAs later
    const int pid_v = lds_pages[un < ntiles ? un >> 1 : 0];
    Group g;
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) {
      if (ks == 0)
        mfma_first_v(s, ring[0], q[0]);
      else if (ks < 35)
        mfma_acc_v(s, ring[ks & 3], q[ks]);
      else
        mfma_acc_v_last(s, ring[ks & 3], q[ks]);
      if (ks + 4 < 36) ring[ks & 3] = rd(ks + 4);
      if (ks == 2) g = make_group(un, __builtin_amdgcn_readfirstlane(pid_v), lane16);
      if (ks % 7 == 2) dma_step(g.src, g.cnt, g.dst_a, g.dst_b, ks / 7, g.lane16);  // loads 0-4
      if (pv_next) {
        if (ks == 20) flags = read_flags(t - 1);
        if (ks >= 24 && ks < 32) pp[ks - 24] = read_p(t - 1, ks - 24);
        if (ks == 32) apv[0] = read_pv(0, 0);
        if (ks == 34) apv[1] = read_pv(1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    return g;
  };

  // ---- weighted sum of one tile: O^T[latent block 4 wave + c][head block hb] += tile^T P^T, in
  // the order (token half kk, latent block c, head block hb); each A operand serves four MFMAs.
  // With a softmax (of the tile scored just before), its stages ride in the MFMA gaps, and the
  // last four loads of group g go out in between.
  auto pv_chain = [&](bool with_softmax, int cnt, const Group* g) {
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      const int j = m >> 2, hb = m & 3, kk = j >> 2, c = j & 3;
      mfma_acc_a(o[4 * c + hb], apv[j % 3], pp[kk * 4 + hb]);
      if (hb == 0 && j + 2 < 8) apv[(j + 2) % 3] = read_pv((j + 2) & 3, (j + 2) >> 2);
      if (with_softmax && m < kSoftmaxStages) softmax_stage(m, cnt, s);
      if (g && m % 7 == 3 && m < 28) dma_step(g->src, g->cnt, g->dst_a, g->dst_b, 5 + m / 7, g->lane16);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (with_softmax) {
#pragma unroll
      for (int st = 32; st < kSoftmaxStages; ++st) softmax_stage(st, cnt, s);
    }
  };

  // ---- probabilities of tile t to ring P for every wave, with this wave's rescale word and
  // factors; then the barrier that publishes them and tile t + 1.
  auto publish = [&](int t) {
    const uint32_t pb = attn_p_buffer(t);
    *(MLA_LDS bf16x8*)(smem + p_lane + pb * kBufP + wave * 2048) = pk[0];
    *(MLA_LDS bf16x8*)(smem + p_lane + pb * kBufP + wave * 2048 + 1024) = pk[1];
    *(MLA_LDS float*)(smem + kOffAlpha + pb * (kHeads * 4) + (32 * wave + l32) * 4) = alpha;
    if (lane == 0) *(MLA_LDS uint32_t*)(smem + kOffFlags + pb * 16 + wave * 4) = rescale ? 1u : 0u;
    dma_wait_tiles(1);  // this wave's loads of tile t + 1 have landed
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  auto advance_pv = [&](int t) {  // from tile t's ring-A buffer to tile t + 1's
    const int st = attn_a_buffer(t + 1) * kBufA - attn_a_buffer(t) * kBufA;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      pv_lo[k] += st;
      pv_hi[k] += st;
    }
  };

  dma_wait_tiles(1);  // tile 0 has landed (this wave's part)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  // iteration 0: scores of tile 0, then its softmax alone (no weighted sum yet)
  {
    const Group g = score_chain(0, false);
    if constexpr (kTree) tree_mask_tile(s, 0);
    const int cnt = tile_count(0);
#pragma unroll
    for (int st = 0; st < kSoftmaxStages; ++st) softmax_stage(st, cnt, s);
#pragma unroll
    for (int k = 5; k < kDmaPerTile; ++k) dma_step(g.src, g.cnt, g.dst_a, g.dst_b, k, g.lane16);
    publish(0);
  }
  for (int t = 1; t < ntiles; ++t) {
    const Group g = score_chain(t, true);
    if constexpr (kTree) tree_mask_tile(s, t);
    rescale_o(t - 1, flags);
    pv_chain(true, tile_count(t), &g);
    advance_pv(t - 1);
    publish(t);
  }
  // weighted sum of the last tile
  {
    const int t = ntiles;
    flags = read_flags(t - 1);
#pragma unroll
    for (int i = 0; i < 8; ++i) pp[i] = read_p(t - 1, i);
    apv[0] = read_pv(0, 0);
    apv[1] = read_pv(1, 0);
    rescale_o(t - 1, flags);
    pv_chain(false, 0, nullptr);
  }

  // ---- epilogue: 1 / sum of weights of every head from its owner, then the output rows
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;  // every key masked: o = 0, lse = -inf
  *(MLA_LDS float*)(smem + kOffInvL + (32 * wave + l32) * 4) = inv;
  if (hf == 0 && a.lse_out) a.lse_out[w.out_row + 32 * wave + l32] = (m_run + __log2f(l_tot)) * 0.69314718055994531f;
  // The last loads (past the last tile) land before the staging below reuses the rings, and every
  // wave has finished reading them.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  acc_wait_mfma();
  float invh[4];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) invh[hb] = *(const MLA_LDS float*)(smem + kOffInvL + (32 * hb + l32) * 4);
  // Element e of o[4 c + hb] of this lane: head 32 hb + l32, latent 32 (4 wave + c) + 8 (e/4) + 4 hf + e%4.
  if (a.final_out) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) {
        float* row = (float*)a.o_out + (w.out_row + 32 * hb + l32) * kDc + 32 * (4 * wave + c) + 4 * hf;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x16& acc = o[4 * c + hb];
          const f32x4 v = {acc_read_scaled(acc[4 * g4], invh[hb]), acc_read_scaled(acc[4 * g4 + 1], invh[hb]),
                           acc_read_scaled(acc[4 * g4 + 2], invh[hb]), acc_read_scaled(acc[4 * g4 + 3], invh[hb])};
          *(f32x4*)(row + 8 * g4) = v;
        }
      }
  } else {
    // bf16 partial rows go out through LDS: each lane holds 4-value pieces of four heads' rows, so
    // direct stores would write 32 rows x 8 B per instruction; staged, one store writes one
    // whole 1 KiB row.
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int hb = 0; hb < 4; ++hb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x16& acc = o[4 * c + hb];
          const u32x2 v = {pack_bf16x2(acc_read_scaled(acc[4 * g4], invh[hb]), acc_read_scaled(acc[4 * g4 + 1], invh[hb])),
                           pack_bf16x2(acc_read_scaled(acc[4 * g4 + 2], invh[hb]), acc_read_scaled(acc[4 * g4 + 3], invh[hb]))};
          *(MLA_LDS u32x2*)(smem + (32 * hb + l32) * kStageRow + (32 * (4 * wave + c) + 8 * g4 + 4 * hf) * 2) = v;
        }
    __syncthreads();
    uint16_t* rows = (uint16_t*)a.o_out + (w.out_row + wave * 32) * kDc + 8 * lane;
#pragma unroll 8
    for (int r = 0; r < 32; ++r)
      *(u32x4*)(rows + (size_t)r * kDc) = *(const MLA_LDS u32x4*)(smem + (wave * 32 + r) * kStageRow + 16 * lane);
  }
}

// fp32 path on the fp32 matrix cores (v_mfma_f32_16x16x4_f32): workgroup = (b, i, split, block of
// 16 heads), 4 waves.  fp32 leaves no room for the bf16 kernel's layout (the query of 128 heads is
// 288 KiB), so the 128 heads of a key range are eight workgroups, each reading the range from L2,
// which also spreads a range's matrix work over eight compute units.  Per 32-token tile (half a
// page, so one page id):
//   * the tile's rows are staged in LDS with a padded row of kF32Ld floats; the next tile's rows
//     are loaded into registers during this tile's work;
//   * scores D(token x head), two 16-token blocks: wave w takes k in [144 w, 144 w + 144), lane
//     group g = l / 16 the k values 144 w + 36 g + s at step s, so its tile operand is one 16-byte
//     read per 4 steps and its query operand sits in 36 registers; the four waves' partial sums
//     meet in LDS and every wave adds them in the same order;
//   * the online softmax (base 2, scale folded in) runs redundantly in every wave, each lane on
//     the 8 tokens of its head the score layout gives it; the probabilities go to the wave's own
//     LDS area, read back as the weighted sum's operand;
//   * weighted sum O^T(latent x head) += tile^T x P: wave w holds latent columns 128 w .. +127 of
//     the 16 heads (eight 16 x 16 blocks), lane group g taking tokens (s & 3) + 4 g + 16 (s >> 2).
// Row padding: a 580-float row is 4 banks past a multiple of 64, so a 16-byte score-operand read
// (16 lanes on 16 rows per pass) covers all 64 banks once, and in the weighted-sum reads the four
// lane groups, 4 rows apart, fall on four disjoint 16-bank windows.
constexpr int kF32Tile = 32;             // tokens per tile
constexpr int kF32Ld = kRow + 4;         // floats per staged tile row
constexpr int kF32PLd = kF32Heads + 4;   // floats per probability row
constexpr int kF32Loads = kF32Tile * kRow / 4 / 256;  // 16-byte loads per thread per tile (18)
static_assert(kF32Tile * kRow % (4 * 256) == 0, "whole 16-byte loads per thread");
static_assert(kF32Heads == 16, "one 16 x 16 MFMA column block of heads");

__device__ __forceinline__ f32x4 mfma16x16x4f32(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(256, 1) void decode_attn_f32_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) float tile[kF32Tile * kF32Ld];
  __shared__ __attribute__((aligned(16))) float spart[4 * 8 * 64];          // [wave][element][lane]
  __shared__ __attribute__((aligned(16))) float pw[4 * kF32Tile * kF32PLd];  // [wave][token][head]
  constexpr int kBlocks = kHeads / kF32Heads;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int hb = id % kBlocks;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4;
  const int head = kF32Heads * hb + l16;  // this lane's head (the MFMA column)
  const float* pool = (const float*)a.pool;

  // this lane's query operand: [q_lat | q_pe] of its head at k = 144 wave + 36 g + s, s < 36; loaded
  // for the row of the fixed layout while the key range is worked out, and again if the plan moves
  // the row (a ragged batch)
  float q[36];
  auto load_q = [&](int row) {
    const size_t qrow = (size_t)row * kHeads + head;
    const int k0 = 144 * wave + 36 * g;
#pragma unroll
    for (int s4 = 0; s4 < 9; ++s4) {
      const int k = k0 + 4 * s4;  // four values on one side of the q_lat / q_pe boundary (512 = 4 x 128)
      const f32x4 v = k < kDc ? *(const f32x4*)((const float*)a.q_lat + qrow * kDc + k)
                              : *(const f32x4*)((const float*)a.q_pe + qrow * kDr + (k - kDc));
#pragma unroll
      for (int j = 0; j < 4; ++j) q[4 * s4 + j] = v[j];
    }
  };
  const int piece = id / kBlocks;
  const int row_guess = a.num_splits > 1 ? piece / a.num_splits : piece;
  load_q(row_guess);
  LenScan lens = scan_lengths(a);
  const WorkItem w = make_work(a, piece, uniform_length(a, lens));
  if (!w.live) return;  // past the last key range (uniform over the workgroup)
  if (hb == 0) record_row_plan(a, w);
  if (w.b * a.S + w.i != row_guess) load_q(w.b * a.S + w.i);

  const int ntok = w.tok_end - w.tok_begin;
  if (ntok <= 0) {  // empty key range: o = 0, lse = -inf; thread t writes 32 columns of head t / 16
    const int hh = kF32Heads * hb + (threadIdx.x >> 4);
    float* row = (float*)a.o_out + (w.out_row + hh) * kDc + 32 * (threadIdx.x & 15);
#pragma unroll
    for (int c = 0; c < 32; c += 4) *(f32x4*)(row + c) = f32x4{0.f, 0.f, 0.f, 0.f};
    if ((threadIdx.x & 15) == 0 && a.lse_out) a.lse_out[w.out_row + hh] = -INFINITY;
    return;
  }
  const int ntiles = (ntok + kF32Tile - 1) / kF32Tile;
  const int32_t* bt = a.block_table + (size_t)w.b * a.max_pages;
  // draft tree: visibility of the S new keys to this query row (wave-uniform)
  const uint64_t tmask =
      a.tree_parents ? tree_walk(tree_parent_of_lane(a.tree_parents, w.b, a.S, lane), a.S, w.i) : 0ull;

  // The next tile's rows in registers: load r of thread t is float4 (t + 256 r) of the tile, row
  // (t + 256 r) / 144.  Rows past the range re-read the tile's first token (finite values, masked).
  f32x4 stage[kF32Loads];
  auto fetch = [&](int t) {
    const int t0 = w.tok_begin + kF32Tile * t;
    const int cnt = w.tok_end - t0 < kF32Tile ? w.tok_end - t0 : kF32Tile;
    const int page = checked_page(a.bounds, bt[t0 / kPage]);
    const float* src = pool + ((size_t)page * kPage + t0 % kPage) * kRow;
#pragma unroll
    for (int r = 0; r < kF32Loads; ++r) {
      const int u = threadIdx.x + 256 * r, row = u / (kRow / 4), c4 = u % (kRow / 4);
      stage[r] = *(const f32x4*)(src + (size_t)(row < cnt ? row : 0) * kRow + 4 * c4);
    }
  };
  auto put = [&]() {
#pragma unroll
    for (int r = 0; r < kF32Loads; ++r) {
      const int u = threadIdx.x + 256 * r, row = u / (kRow / 4), c4 = u % (kRow / 4);
      *(MLA_LDS f32x4*)(tile + row * kF32Ld + 4 * c4) = stage[r];
    }
  };
  fetch(0);

  float m_run = -INFINITY, l_run = 0.f;  // of this lane's head, in log2 units
  f32x4 o[8];                            // block b: latent 128 wave + 16 b + 4 g + e, head l16
#pragma unroll
  for (int b = 0; b < 8; ++b) o[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  MLA_LDS float* const my_p = (MLA_LDS float*)(pw + wave * kF32Tile * kF32PLd);

  for (int t = 0; t < ntiles; ++t) {
    const int t0 = w.tok_begin + kF32Tile * t;
    const int cnt = w.tok_end - t0 < kF32Tile ? w.tok_end - t0 : kF32Tile;
    put();
    __syncthreads();  // the tile is in LDS
    if (t + 1 < ntiles) fetch(t + 1);

    // scores over this wave's k range, token blocks tb = 0, 1
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      f32x4 sc = {0.f, 0.f, 0.f, 0.f};
      const MLA_LDS float* arow = (const MLA_LDS float*)(tile + (16 * tb + l16) * kF32Ld + 144 * wave + 36 * g);
#pragma unroll
      for (int s4 = 0; s4 < 9; ++s4) {
        const f32x4 av = *(const MLA_LDS f32x4*)(arow + 4 * s4);
#pragma unroll
        for (int j = 0; j < 4; ++j) sc = mfma16x16x4f32(av[j], q[4 * s4 + j], sc);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) spart[(wave * 8 + 4 * tb + e) * 64 + lane] = sc[e];
    }
    __syncthreads();  // every wave's partial scores
    float z[8];
    float mt = -INFINITY;
#pragma unroll
    for (int e8 = 0; e8 < 8; ++e8) {
      const float v = (spart[e8 * 64 + lane] + spart[(8 + e8) * 64 + lane]) +
                      (spart[(16 + e8) * 64 + lane] + spart[(24 + e8) * 64 + lane]);
      const int i = 16 * (e8 >> 2) + 4 * g + (e8 & 3);  // token of element e8 within the tile
      const int jn = t0 + i - w.tail;                    // draft-tree node index of that key
      const bool vis = i < cnt && (!a.tree_parents || jn < 0 || (jn < 64 && ((tmask >> jn) & 1ull)));
      z[e8] = vis ? v * a.scale_log2 : -INFINITY;
      mt = fmaxf(mt, z[e8]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;  // every key so far masked
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float ls = 0.f;
#pragma unroll
    for (int e8 = 0; e8 < 8; ++e8) {
      const float pe = __builtin_amdgcn_exp2f(z[e8] - m_use);  // masked keys: exp2(-inf) = 0
      ls += pe;
      my_p[(16 * (e8 >> 2) + 4 * g + (e8 & 3)) * kF32PLd + l16] = pe;
    }
    ls += __shfl_xor(ls, 16);
    ls += __shfl_xor(ls, 32);
    l_run = l_run * alpha + ls;
    m_run = m_new;
#pragma unroll
    for (int b = 0; b < 8; ++b) o[b] *= alpha;

    // weighted sum: this wave's latent columns, the tile as value
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int k = (s & 3) + 4 * g + 16 * (s >> 2);
      const float pb = my_p[k * kF32PLd + l16];
      const MLA_LDS float* crow = (const MLA_LDS float*)(tile + k * kF32Ld + 128 * wave + l16);
#pragma unroll
      for (int b = 0; b < 8; ++b) o[b] = mfma16x16x4f32(crow[16 * b], pb, o[b]);
    }
    __syncthreads();  // the tile, the partial scores and the probabilities are free again
  }

  const bool empty = l_run == 0.f;
  const float inv = empty ? 0.f : 1.0f / l_run;
  float* orow = (float*)a.o_out + (w.out_row + head) * kDc + 128 * wave + 4 * g;
#pragma unroll
  for (int b = 0; b < 8; ++b) *(f32x4*)(orow + 16 * b) = o[b] * inv;
  if (wave == 0 && g == 0 && a.lse_out)
    a.lse_out[w.out_row + head] = empty ? -INFINITY : (m_run + __log2f(l_run)) * 0.69314718055994531f;
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
                                                        const float* __restrict__ lse_part,
                                                        const int32_t* __restrict__ row_plan, float* __restrict__ o_lat,
                                                        float* __restrict__ lse, int num_splits) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int rh = xcd_remap(blockIdx.x, gridDim.x) * 4 + wave;  // row * kHeads + h
  const int row = rh / kHeads, h = rh % kHeads;
  // The row's slots (first, count) come from the attention's plan.  The first partials are issued
  // for the fixed layout (row * num_splits, num_splits) while the plan's flag loads, and issued
  // again in the rare case that the layout differs (a ragged batch).
  const int first_fixed = row * num_splits;
  int first = first_fixed, nsp = num_splits;
  if (!__builtin_amdgcn_readfirstlane(row_plan[0])) {
    first = __builtin_amdgcn_readfirstlane(row_plan[4 + 2 * row]);
    nsp = __builtin_amdgcn_readfirstlane(row_plan[4 + 2 * row + 1]);
  }
  constexpr float kLog2e = 1.4426950408889634f;

  PartRow<PartT> x[8];
  auto load_batch = [&](const PartT* op, int n, int kb) {  // splits kb .. kb+7 (clamped to the last one)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = kb + j < n ? kb + j : n - 1;
      x[j].load(op + (size_t)k * kHeads * kDc);
    }
  };
  // does not depend on the weights: in flight while they are formed
  load_batch(o_part + ((size_t)first_fixed * kHeads + h) * kDc + 8 * lane, num_splits, 0);
  const size_t base = (size_t)first * kHeads + h;  // split k at base + k * kHeads
  const float* lp = lse_part + base;
  const PartT* op = o_part + base * kDc + 8 * lane;
  if (first != first_fixed || nsp != num_splits) load_batch(op, nsp, 0);
  auto lse_of = [&](int k) { return k < nsp ? lp[(size_t)k * kHeads] : -INFINITY; };
  const float lse0 = lse_of(lane);
  float m = lse0;
  for (int k0 = 64; k0 < nsp; k0 += 64) m = fmaxf(m, lse_of(k0 + lane));
  m = wave_max(m);
  const float m_ref = m == -INFINITY ? 0.f : m;  // all splits empty: every weight is 0

  f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
  float sum = 0.f, w_lane = 0.f;
  for (int kb = 0; kb < nsp; kb += 8) {
    if ((kb & 63) == 0)  // weights of splits kb .. kb+63, one per lane (0 past the end)
      w_lane = __builtin_amdgcn_exp2f(((kb == 0 ? lse0 : lse_of(kb + lane)) - m_ref) * kLog2e);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float w = kb + j < nsp ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_lane), (kb & 63) + j))
                                   : 0.f;
      sum += w;
      a0 += w * x[j].lo();
      a1 += w * x[j].hi();
    }
    if (kb + 8 < nsp) load_batch(op, nsp, kb + 8);
  }
  const float inv = sum > 0.f ? 1.0f / sum : 0.f;
  f32x4* dst = (f32x4*)(o_lat + (size_t)rh * kDc + 8 * lane);
  dst[0] = a0 * inv;
  dst[1] = a1 * inv;
  if (lane == 0 && lse) lse[rh] = m == -INFINITY ? -INFINITY : m + logf(sum);
}
hipError_t launch_decode_attn(const AttnArgs& a, int rows, hipStream_t stream) {
  forget_stale_error();
  const int nwg = a.dtype_bf16 ? a.range_budget : rows * a.num_splits;
  if (a.dtype_bf16 && a.tree_parents)
    hipLaunchKernelGGL(decode_attn_bf16_kernel<true>, dim3(nwg), dim3(256), 0, stream, a);
  else if (a.dtype_bf16)
    hipLaunchKernelGGL(decode_attn_bf16_kernel<false>, dim3(nwg), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(decode_attn_f32_kernel, dim3(nwg * (kHeads / kF32Heads)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_lse_merge(const void* o_part, bool part_bf16, const float* lse_part, const int32_t* row_plan,
                            float* o_lat, float* lse, int rows, int num_splits, int slots, hipStream_t stream) {
  (void)slots;  // the merge reads each row's slots from row_plan
  forget_stale_error();
  const dim3 grid(rows * (kHeads / 4));
  if (part_bf16)
    hipLaunchKernelGGL(lse_merge_kernel<uint16_t>, grid, dim3(256), 0, stream, (const uint16_t*)o_part, lse_part,
                       row_plan, o_lat, lse, num_splits);
  else
    hipLaunchKernelGGL(lse_merge_kernel<float>, grid, dim3(256), 0, stream, (const float*)o_part, lse_part, row_plan,
                       o_lat, lse, num_splits);
  return hipGetLastError();
}

}  // namespace mla
