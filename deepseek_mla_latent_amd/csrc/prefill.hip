// Prefill in multi-head form ("order 1"), gfx950.
//
// For prompt processing the number of query tokens equals the number of keys (t = s), and the
// non-absorbed order costs fewer FLOPs than the absorbed one: "【笔记】MLA矩阵吸收分析" §二.4.1
// (order 1 minus order 2 is negative when t = s) with the order-1 steps of §二.1 and §三.1
// (up-project K and V from the latent per head, then score and weight per head).  The Perplexity
// post ("Lower latency and higher throughput with multi-node DeepSeek deployment", section
// "Будущая работа") plans the same for its prefill: project the latent into K/V space, then
// attend in MHA form.  Two kernels:
//
//   kv_up_kernel         K_nope[b,h,j] = W_UK[h]^T c_j and V[b,h,j] = W_UV[h]^T c_j for every cached
//                        token j (pages gathered through the block table), plus a dense copy of
//                        the shared RoPE key k_pe_j.  One GEMM per head, 32x32x16 bf16 MFMAs.
//   prefill_attn_kernel  causal attention per head with a 192-wide key [K_nope | k_pe] and a
//                        128-wide value, online softmax over 64-key tiles.
//
// Both take bf16 operands and accumulate in fp32.
#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

constexpr int kKvRow = 2 * kDh;             // 256 elements per (head, token): [K_nope | V]

constexpr int kPfQueries = 256;              // queries per attention workgroup (8 waves x 32)
constexpr int kPfKeys = kPage;               // keys per LDS tile
constexpr int kPfKvBytes = kPfKeys * kKvRow * 2;          // 32 KiB: [K_nope | V] rows
constexpr int kPfBufBytes = kPfKvBytes + kPfKeys * kDr * 2;  // + 8 KiB of k_pe rows

__device__ __forceinline__ bf16x8 lds_b128(const MLA_LDS char* p) { return *(const MLA_LDS bf16x8*)p; }

// Transposed 16-bit read: within each group of 16 lanes, lane i names the 8-byte piece
// (row i/4, columns 4(i%4) .. +3) of a 4 x 16 block and receives column i of that block.
// Two reads (rows 0-3 and 4-7 of an operand's 8 k-values) make one MFMA operand.
__device__ __forceinline__ bf16x8 lds_tr_pair(const MLA_LDS char* lo, const MLA_LDS char* hi) {
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)lo);
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)hi);
  const i16x8 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, r);
}

// Direct-to-LDS load of 16 bytes per lane (lane l's bytes land at lds + 16 l) from a wave-uniform
// base plus a per-lane byte offset.  Completion is awaited with an explicit vmcnt wait.  The base
// goes through readfirstlane so that it is always held in scalar registers (the instruction's
// scalar-address form), whatever the compiler's uniformity analysis concluded.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds) {
  const uint64_t a = (uint64_t)(uintptr_t)sbase;
  const uint64_t base = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base),
               "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}
__device__ __forceinline__ uint32_t lds_u32(const MLA_LDS char* p) { return (uint32_t)(uintptr_t)p; }

// 4 consecutive fp32 -> 4 bf16 (8 bytes)
__device__ __forceinline__ u32x2 pack4(float a, float b, float c, float d) {
  u32x2 r;
  r[0] = pack_bf16x2(a, b);
  r[1] = pack_bf16x2(c, d);
  return r;
}

}  // namespace

// ------------------------------------------------------------------------------------------------
// K/V up-projection.  Workgroup = (head h, half of the pages); 256 workgroups.  Wave w owns 64
// output columns: matrix m = w / 2 (0: W_UK -> K_nope, 1: W_UV -> V), columns 64 (w % 2) ..
// +63.  Its slice of W (512 x 64) is held in registers for the whole walk as 64 MFMA A operands
// (W^T rows = output columns), read once through LDS with transposed reads.  The cached pages then
// stream through LDS (two 64 KiB buffers, one page ahead) by direct-to-LDS loads of whole 1 KiB
// latent rows, and each wave computes out^T[n][token] = sum_k W[k][n] c[token][k] for its 64
// columns and the page's 64 tokens: the B operand (8 consecutive k of one token per lane) is a
// ds_read_b128 of the staged row.  The page's output rows ([K_nope | V] of 64 consecutive tokens,
// one contiguous 32 KiB block) are assembled in LDS and written with 1 KiB-contiguous stores one
// page late.  Roles keep store latency out of the page waits: wave 0 issues every page load and
// waits for it (a vector-memory wait covers all of a wave's outstanding loads and stores), waves
// 1-3 issue every store and never wait on vector memory.  The shared RoPE key is copied by
// kpe_copy_kernel.
//
// LDS layouts: W staging row k (256 B), unit u at u ^ ((k & 3) << 2) (transposed reads of 4 rows
// x 4 units hit 16 distinct units); page row t (1 KiB) and output row t (512 B), unit u at
// u ^ (t & 15) (16 tokens at one unit hit 16 distinct units).
__global__ __launch_bounds__(256, 1) void kv_up_kernel(const uint16_t* __restrict__ pool,
                                                       const int32_t* __restrict__ block_table,
                                                       const int32_t* __restrict__ seq_lens,
                                                       const uint16_t* __restrict__ w_uk,
                                                       const uint16_t* __restrict__ w_uv, uint16_t* __restrict__ kv,
                                                       int batch, int max_pages, int pages_max, Bounds bounds) {
  constexpr int kPageBytes = kPage * kDc * 2;     // 64 KiB: the latent rows of one page
  constexpr int kOutBytes = kPage * kKvRow * 2;   // 32 KiB: the page's [K_nope | V] rows
  __shared__ __attribute__((aligned(16))) char lds_raw[2 * kPageBytes + kOutBytes];
  MLA_LDS char* lds = (MLA_LDS char*)lds_raw;

  const int h = blockIdx.x >> 1, part = blockIdx.x & 1;  // workgroups of one part share an XCD parity
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int m = wave >> 1, n0 = 64 * (wave & 1);
  const size_t Lp = (size_t)max_pages * kPage;

  // W slice -> registers: two rounds (W_UK, then W_UV) of 128 KiB through both page buffers.
  bf16x8 wf[32][2];
  {
    const int tr_row = 8 * hf + ((lane >> 2) & 3);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    auto tr_off = [&](int r, int n) { return r * 256 + ((((n >> 3) ^ ((r & 3) << 2))) << 4) + (n & 7) * 2; };
#pragma unroll
    for (int round = 0; round < 2; ++round) {
      const char* w = (const char*)((round ? w_uv : w_uk) + (size_t)h * kDc * kDh);
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const int pc = wave * 32 + j;
        const int r = 4 * pc + (lane >> 4), p = lane & 15;
        dma16(w, (uint32_t)(r * kDh * 2 + ((p ^ ((r & 3) << 2)) << 4)), lds_u32(lds + pc * 1024));
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (m == round) {
#pragma unroll
        for (int ks = 0; ks < 32; ++ks)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            const int r = ks * 16 + tr_row, n = n0 + nb * 32 + tr_col;
            wf[ks][nb] = lds_tr_pair(lds + tr_off(r, n), lds + tr_off(r + 4, n));
          }
      }
      __syncthreads();  // reads done before the buffers are reused
    }
  }

  // pages of this part: virtual pages v = b * pages_max + p with v % 2 == part, walked from a
  // start that depends on the head (so that at any moment the workgroups write to different
  // addresses of the output rather than to the same page offset of 128 heads' rows) and wrapping
  const int nv = batch * pages_max;
  const int count = (nv - part + 1) / 2;  // virtual pages of this part
  const int j0 = count ? (int)(((long long)h * count) / kHeads) : 0;
  struct Page {
    int jj, v, valid;  // jj: position in the walk (count = done)
    const uint16_t* rows;
  };
  // (wave-uniform values; read with readfirstlane so that the page base is a scalar address)
  auto find = [&](int jj) -> Page {  // first page at or after walk position jj that holds tokens
    for (; jj < count; ++jj) {
      int j = j0 + jj;
      j = j >= count ? j - count : j;
      const int v = __builtin_amdgcn_readfirstlane(part + 2 * j);
      const int b = v / pages_max, p = v - b * pages_max;
      const int L = checked_len(bounds, seq_lens[b]);  // uniform address: a scalar load, no vector-memory wait
      if (p * kPage < L) {
        const int pid = __builtin_amdgcn_readfirstlane(checked_page(bounds, block_table[(size_t)b * max_pages + p]));
        return {jj, v, min(kPage, L - p * kPage), pool + (size_t)pid * kPage * kRow};
      }
    }
    return {count, nv, 0, pool};
  };
  // one page: 64 latent rows of 1 KiB, all issued by wave 0; LDS position q of row t gets unit
  // q ^ (t & 15).  Rows [t0, t1) at a time: the vector-memory counter tracks at most 63 loads, and
  // a 64th would hold wave 0 at its issue until the first returned, so the next page goes out in
  // three parts spread over the current page's MFMAs.
  auto issue_rows = [&](const Page& pg, int buf, int t0, int t1) {
#pragma unroll
    for (int t = t0; t < t1; ++t)
      dma16(pg.rows, (uint32_t)(t * kRow * 2 + ((lane ^ (t & 15)) << 4)), lds_u32(lds + buf * kPageBytes + t * 1024));
  };
  auto issue_page = [&](const Page& pg, int buf) {
    issue_rows(pg, buf, 0, 32);
    issue_rows(pg, buf, 32, 63);
    issue_rows(pg, buf, 63, 64);
  };
  const int b_off[2] = {(l32 * 1024), ((32 + l32) * 1024)};  // this lane's token rows (tb = 0, 1)

  MLA_LDS char* ostage = lds + 2 * kPageBytes;
  f32x16 acc[2][2];
  // results -> output staging: element e of block (nb, tb) is out^T[32 nb + 8 (e/4) + 4 hf + e%4]
  // [32 tb + l32]; rows past the sequence end (to the page end) are zeros
  auto stage_out = [&](int valid) {
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int tok = tb * 32 + l32;
      const bool ok = tok < valid;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16& x = acc[nb][tb];
          const u32x2 v = ok ? pack4(x[4 * g], x[4 * g + 1], x[4 * g + 2], x[4 * g + 3]) : u32x2{0u, 0u};
          const int u = (m * kDh + n0 + nb * 32 + g * 8) >> 3;  // 16-byte unit of the row
          *(MLA_LDS u32x2*)(ostage + tok * 512 + (((u & 16) | ((u & 15) ^ (tok & 15))) << 4) + hf * 8) = v;
        }
    }
  };
  // staged rows -> HBM (waves 1-3): the page's 32 KiB block, 1 KiB per instruction
  auto write_out = [&](const Page& pg) {
    const int b = pg.v / pages_max, p = pg.v - b * pages_max;
    char* dst = (char*)(kv + (((size_t)b * kHeads + h) * Lp + (size_t)p * kPage) * kKvRow);
    for (int piece = wave - 1; piece < 32; piece += 3) {
      const int row = 2 * piece + (lane >> 5), u = lane & 31;
      const u32x4 v = *(const MLA_LDS u32x4*)(ostage + row * 512 + (((u & 16) | ((u & 15) ^ (row & 15))) << 4));
      *(u32x4*)(dst + row * 512 + u * 16) = v;
    }
  };

  Page cur = find(0), prev = {count, nv, 0, pool};
  if (wave == 0 && cur.jj < count) issue_page(cur, 0);
  for (int idx = 0; cur.jj < count; ++idx) {
    if (wave == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this page (wave 0 stores nothing)
    __syncthreads();  // page in LDS; the other buffer is free; the previous results are staged
    const Page next = find(cur.jj + 1);
    const bool issue = wave == 0 && next.jj < count;  // wave-uniform
    if (issue) issue_rows(next, (idx + 1) & 1, 0, 32);
    if (wave != 0 && prev.jj < count) write_out(prev);
    const MLA_LDS char* pg = lds + (idx & 1) * kPageBytes;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) acc[nb][tb] = f32x16{};
    // B operands stream through a ring three k-steps deep: the reads for step ks + 2 are issued
    // (and pinned there by a scheduling barrier) before the MFMAs of step ks
    auto read_b = [&](int ks, bf16x8 (&bf)[2]) {
      const int u = 2 * ks + hf;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) bf[tb] = lds_b128(pg + b_off[tb] + ((u ^ (l32 & 15)) << 4));
    };
    bf16x8 ring[3][2];
    read_b(0, ring[0]);
    read_b(1, ring[1]);
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) {
      if (ks == 10 && issue) issue_rows(next, (idx + 1) & 1, 32, 63);
      if (ks == 20 && issue) issue_rows(next, (idx + 1) & 1, 63, 64);
      if (ks + 2 < 32) read_b(ks + 2, ring[(ks + 2) % 3]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) acc[nb][tb] = mfma32x32x16(wf[ks][nb], ring[ks % 3][tb], acc[nb][tb]);
    }
    __syncthreads();  // every wave has read the staged rows of the previous page
    stage_out(cur.valid);
    prev = cur;
    cur = next;
  }
  if (prev.jj < count) {
    __syncthreads();
    if (wave != 0) write_out(prev);
  }
}

// The shared RoPE key of every cached token, copied densely: kpe[b, j] = k_pe_j for j < seq_lens[b],
// zeros to the end of the last page.  One 64-lane workgroup per (b, page).
__global__ __launch_bounds__(64) void kpe_copy_kernel(const uint16_t* __restrict__ pool,
                                                      const int32_t* __restrict__ block_table,
                                                      const int32_t* __restrict__ seq_lens, uint16_t* __restrict__ kpe,
                                                      int max_pages, int pages_max, Bounds bounds) {
  const int b = blockIdx.x / pages_max, p = blockIdx.x % pages_max;
  const int valid = min(kPage, checked_len(bounds, seq_lens[b]) - p * kPage);
  if (valid <= 0) return;
  const uint16_t* rows = pool + (size_t)checked_page(bounds, block_table[(size_t)b * max_pages + p]) * kPage * kRow;
  uint16_t* dst = kpe + ((size_t)b * max_pages + p) * kPage * kDr;
  const int lane = threadIdx.x;
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int q = it * 64 + lane, row = q >> 3, u = q & 7;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row < valid) v = *(const u32x4*)(rows + (size_t)row * kRow + kDc + u * 8);
    *(u32x4*)(dst + (size_t)row * kDr + u * 8) = v;
  }
}

hipError_t launch_kv_up_grid(const void* pool, const int32_t* block_table, const int32_t* seq_lens,
                             const void* w_uk, const void* w_uv, void* kv, void* kpe, int batch, int max_pages,
                             int pages_max, const Bounds& bounds, hipStream_t stream) {
  forget_stale_error();
  if (batch == 0 || pages_max == 0) return hipSuccess;
  hipLaunchKernelGGL(kv_up_kernel, dim3(2 * kHeads), dim3(256), 0, stream, (const uint16_t*)pool, block_table,
                     seq_lens, (const uint16_t*)w_uk, (const uint16_t*)w_uv, (uint16_t*)kv, batch, max_pages,
                     pages_max, bounds);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kpe_copy_kernel, dim3((unsigned)(batch * pages_max)), dim3(64), 0, stream, (const uint16_t*)pool,
                     block_table, seq_lens, (uint16_t*)kpe, max_pages, pages_max, bounds);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------
// Causal multi-head attention over the up-projected keys.  Workgroup = (b, h, 256-query block),
// 8 waves (two per SIMD); wave w owns 32 queries.  Per 64-key tile:
//   S^T (keys x queries) = [K_nope | k_pe] Q^T: 2 key blocks x 12 k-steps, keys as the A operand
//   (ds_read_b128 rows), the wave's queries as the B operand held in registers for the whole walk;
//   online softmax per query column (the lane pair l, l^32 holds one query);
//   O^T (dv x queries) += V^T P^T: 4 dv blocks x 4 key steps, V^T read transposed from the tile.
// The accumulator layout of S^T is the B-operand layout of P^T when the 16 keys of an MFMA step
// are taken in the order the accumulator holds them; the V^T reads use the same key order.
// Software pipeline across tiles, so that the matrix cores are not idle during the softmax:
//   scores(t)  ->  [sum(t-1) | softmax(t)]
// where "[x | y]" issues the MFMAs of x interleaved with the VALU work of y.
// Tile layout: key row r of [K_nope | V] (32 units of 16 B), unit u at u ^ swz(r) (low 4 bits),
// k_pe row r (8 units) at u ^ ((r >> 1) & 7): both read patterns hit 16 distinct units per
// 16 lanes.  Tiles stream in by direct-to-LDS loads into a ring of 4 buffers, two tiles ahead
// (tile t - 1 is still read during tile t).  A wave stops computing at the first tile past its
// last query's keys (it still takes part in loads and barriers).  The running max is only raised
// when a tile's max exceeds it by more than 2^8 (log2 units).
__device__ __forceinline__ int pf_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int pf_swz_pe(int r) { return (r >> 1) & 7; }

// max of three / two without NaN canonicalisation (inputs are scores or -inf): written as fmaxf the
// compiler adds a canonicalising max per MFMA result, which doubles the VALU work of the tile max
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float vmax2(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
constexpr int kPfWaves = 8;
constexpr int kPfRing = 4;
constexpr int kPfAhead = 2;  // tiles in flight beyond the one being computed

// wait until at most `younger` tiles' loads (5 per wave each) are in flight (loads retire in order)
__device__ __forceinline__ void pf_wait_tiles(int younger) {
  if (younger >= 1)
    asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

__global__ __launch_bounds__(64 * kPfWaves, 1) void prefill_attn_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) char lds_raw[kPfRing * kPfBufBytes];  // 160 KiB
  MLA_LDS char* lds = (MLA_LDS char*)lds_raw;

  const int nbh = a.B * kHeads;
  const int id = xcd_remap(blockIdx.x, gridDim.x);  // one XCD walks all query blocks of a few heads
  const int bh = id / a.nqb;
  const int qb = a.nqb - 1 - id % a.nqb;  // longest key ranges first
  if (bh >= nbh) return;
  const int b = bh / kHeads, h = bh % kHeads;
  const int L = checked_len(a.bounds, a.seq_lens[b]), S = a.S;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int q0 = qb * kPfQueries, qw = q0 + wave * 32;  // first query of the block / of the wave
  const int qi = qw + l32;                              // this lane's query (column)
  auto visible = [&](int q) { return a.causal ? max(0, min(L, L - S + q + 1)) : L; };
  const int vis = visible(min(qi, S - 1));             // padding queries behave like the last one
  const int kend = visible(min(S - 1, q0 + kPfQueries - 1));  // keys any query of the workgroup sees
  const int ntiles = (kend + kPfKeys - 1) / kPfKeys;
  const int wave_vis_lo = visible(min(S - 1, qw));       // fewest keys a query of the wave sees
  const int wave_vis_hi = visible(min(S - 1, qw + 31));  // most

  const size_t Lp = (size_t)a.Lp;
  const char* kv_seq = (const char*)a.kv + ((size_t)b * kHeads + h) * Lp * kKvRow * 2;
  const char* pe_seq = (const char*)a.kpe + (size_t)b * Lp * kDr * 2;

  // tile DMA: 32 KiB of [K_nope | V] rows + 8 KiB of k_pe rows, 5 loads of 1 KiB per wave
  auto issue_tile = [&](int t) {
    MLA_LDS char* dst = lds + (t % kPfRing) * kPfBufBytes;
    const char* kv_t = kv_seq + (size_t)t * kPfKeys * kKvRow * 2;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = wave * 4 + j;             // 1 KiB piece: rows 2c, 2c+1
      const int r = 2 * c + (lane >> 5), p = lane & 31;
      const int u = (p & 16) | ((p & 15) ^ pf_swz(r));
      dma16(kv_t, (uint32_t)(r * kKvRow * 2 + u * 16), lds_u32(dst + c * 1024));
    }
    const int r = 8 * wave + (lane >> 3), p = lane & 7;  // rows 8 wave .. 8 wave + 7
    dma16(pe_seq + (size_t)t * kPfKeys * kDr * 2, (uint32_t)(r * kDr * 2 + ((p ^ pf_swz_pe(r)) << 4)),
          lds_u32(dst + kPfKvBytes + wave * 1024));
  };
  for (int t = 0; t < kPfAhead && t < ntiles; ++t) issue_tile(t);

  // queries as B operands: k-steps 0..7 from q_nope, 8..11 from q_pe.  Loaded after the first
  // tiles are requested and consumed by an empty asm statement before the loop: the wait for
  // them happens here, once, and no load the compiler tracks is pending inside the loop (its
  // waits there would otherwise also drain the tile loads in flight).
  bf16x8 qf[12];
  {
    const int qc = min(qi, S - 1);
    const uint16_t* qn = (const uint16_t*)a.q_nope + (((size_t)b * S + qc) * kHeads + h) * kDh;
    const uint16_t* qp = (const uint16_t*)a.q_pe + (((size_t)b * S + qc) * kHeads + h) * kDr;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = *(const bf16x8*)(qn + ks * 16 + hf * 8);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[8 + ks] = *(const bf16x8*)(qp + ks * 16 + hf * 8);
#pragma unroll
    for (int ks = 0; ks < 12; ++ks) asm volatile("" ::"v"(qf[ks]));
  }

  // Operand addresses: a few per-lane bases, the rest immediates.  Key operand (k-step ks, key
  // block kb): row 32 kb + l32 has the swizzle of row l32, so kb only adds 32 rows.  Value
  // operand (key step kk, dv block cb): rows 16 kk + 4 hf + (lane >> 2 & 3) (+8 for the high
  // half) have swizzles independent of kk, so kk only adds 16 rows; dv columns
  // 32 cb + 16 ((lane >> 4) & 1) + 4 (lane & 3).
  int kofs[12];
  {
    const int sw_kv = pf_swz(l32), sw_pe = pf_swz_pe(l32);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) kofs[ks] = l32 * kKvRow * 2 + (((2 * ks + hf) ^ sw_kv) << 4);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kofs[8 + ks] = kPfKvBytes + l32 * kDr * 2 + (((2 * ks + hf) ^ sw_pe) << 4);
  }
  auto k_imm = [](int kb, int ks) { return kb * 32 * (ks < 8 ? kKvRow * 2 : kDr * 2); };
  int vofs[4][2];
  {
    const int vr = 4 * hf + ((lane >> 2) & 3);
    const int vc = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const int r = vr + 8 * hi, dv = cb * 32 + vc, u = 16 + (dv >> 3);
        vofs[cb][hi] = r * kKvRow * 2 + (((u & 16) | ((u & 15) ^ pf_swz(r))) << 4) + (dv & 7) * 2;
      }
  }
  auto read_v = [&](const MLA_LDS char* tile, int i) {  // operand i = 4 kk + cb
    const int kk = i >> 2, cb = i & 3, imm = kk * 16 * kKvRow * 2;
    return lds_tr_pair(tile + vofs[cb][0] + imm, tile + vofs[cb][1] + imm);
  };

  f32x16 o[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) o[cb] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f, alpha = 1.f;
  bool rescale = false;
  const float sl2 = a.scale_log2;
  f32x16 s[2];     // scores of the current tile, per key block
  bf16x8 pk[4];    // P^T operands of the tile being summed, per key step
  bf16x8 pn[4];    // P^T operands being produced for the current tile

  // Softmax of the current tile, cut into 18 stages spread over the 16 MFMA slots of the sum:
  // stage 0 masks, stage 1 takes the max, combines the lane pair and decides the rescale
  // (branch-free), stages 2..17 compute two probabilities each.
  auto sm_stage = [&](int st, int key0, bool need_mask) {
    if (st == 0) {
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = key0 + kb * 32 + (e >> 2) * 8 + hf * 4 + (e & 3);
            s[kb][e] = key < vis ? s[kb][e] : -INFINITY;
          }
      }
    } else if (st == 1) {
      float mc[4];  // four independent max3 chains over 8 scores each
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f32x16& x = s[c >> 1];
        const int e0 = (c & 1) * 8;
        mc[c] = vmax3(x[e0], x[e0 + 1], x[e0 + 2]);
        mc[c] = vmax3(mc[c], x[e0 + 3], x[e0 + 4]);
        mc[c] = vmax3(mc[c], x[e0 + 5], x[e0 + 6]);
        mc[c] = vmax2(mc[c], x[e0 + 7]);
      }
      float mt = vmax2(vmax3(mc[0], mc[1], mc[2]), mc[3]);
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
      mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * sl2;
      const bool raise = __any(mt > m_run + 8.0f);  // wave-uniform
      const float m_new = raise ? fmaxf(m_run, mt) : m_run;
      rescale = raise && m_run != -INFINITY;  // O and l hold something: bring them to m_new
      alpha = rescale ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
      l_run *= alpha;
      m_run = m_new;
    } else {
      const float msub = m_run == -INFINITY ? 0.f : m_run;  // no visible key yet: every p is 0
      const int e = (st - 2) * 2;  // 0..30: the pair e, e + 1 (one dword of a P operand)
      const int kb = e >> 4, ee = e & 15;
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][ee], sl2, -msub));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][ee + 1], sl2, -msub));
      const bf16x2 pr = {(__bf16)p0, (__bf16)p1};
      // the row sum takes the bf16 probabilities the weighted sum uses, two per dot2 instruction
      l_run = __builtin_amdgcn_fdot2_f32_bf16(pr, bf16x2{(__bf16)1.0f, (__bf16)1.0f}, l_run, false);
      pn[kb * 2 + (ee >> 3)][ee & 7] = pr[0];
      pn[kb * 2 + (ee >> 3)][(ee & 7) + 1] = pr[1];
    }
  };
  // [sum of the previous tile (operands pk) | softmax of the current tile (stages over the slots)]
  auto sum_with_softmax = [&](const MLA_LDS char* tile, int key0, bool need_mask, bool do_sm) {
    bf16x8 vr3[3];
    vr3[0] = read_v(tile, 0);
    vr3[1] = read_v(tile, 1);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i + 2 < 16) vr3[(i + 2) % 3] = read_v(tile, i + 2);
      if (do_sm) {  // stages 0, 1 at the first slot, 2..16 at slots 1..15, 17 at the last
        sm_stage(i == 0 ? 0 : i + 1, key0, need_mask);
        if (i == 0) sm_stage(1, key0, need_mask);
        if (i == 15) sm_stage(17, key0, need_mask);
      }
      __builtin_amdgcn_sched_barrier(0);
      o[i & 3] = mfma32x32x16(vr3[i % 3], pk[i >> 2], o[i & 3]);
    }
  };
  // O is brought to the reference max of the tile whose probabilities are summed next; the
  // decision was taken in that tile's softmax
  bool pending_rescale = false;
  float pending_alpha = 1.f;
  auto scale_o = [&]() {
    if (pending_rescale) {
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[cb][e] *= pending_alpha;
    }
  };

  // Before the first tile, "the sum over the previous tile" runs over a zeroed buffer with P = 0,
  // so the loop body has no first-iteration special case.
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) pk[kk] = bf16x8{};
  {
    MLA_LDS char* z = lds + (kPfRing - 1) * kPfBufBytes;
    for (int i = tid; i < kPfBufBytes / 16; i += 64 * kPfWaves) *(MLA_LDS u32x4*)(z + i * 16) = u32x4{0u, 0u, 0u, 0u};
  }

  // scores of one tile into s: the key operands stream through a ring two k-steps ahead of their
  // MFMAs
  auto compute_scores = [&](const MLA_LDS char* tile) {
    s[0] = f32x16{};
    s[1] = f32x16{};
    bf16x8 kr[3][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) kr[ks][kb] = lds_b128(tile + kofs[ks] + k_imm(kb, ks));
#pragma unroll
    for (int ks = 0; ks < 12; ++ks) {
      if (ks + 2 < 12) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) kr[(ks + 2) % 3][kb] = lds_b128(tile + kofs[ks + 2] + k_imm(kb, ks + 2));
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[kb] = mfma32x32x16(kr[ks % 3][kb], qf[ks], s[kb]);
    }
  };
  // the softmax of the scores in s on its own, for the sum that follows at once: P into pk, O
  // brought to the new reference
  auto softmax_now = [&](int key0, bool need_mask) {
#pragma unroll
    for (int st = 0; st < 18; ++st) sm_stage(st, key0, need_mask);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) pk[kk] = pn[kk];
    pending_rescale = rescale;
    pending_alpha = alpha;
    scale_o();
    pending_rescale = false;
  };

  // The per-tile barrier starts every wave's iteration together.  Waves 0-3 score the new tile
  // first (MFMA-heavy) and then sum the previous one with the new softmax riding along (VALU-heavy);
  // waves 4-7, which share the SIMDs with waves 0-3, take the phases the other way round: the
  // softmax and sum of the previous tile first, then the scores of the new one.  A SIMD then pairs
  // matrix work of one wave with vector work of the other instead of running both waves through the
  // same phase at once.  Both orders finish reading tile t - 1 before the barrier of tile t + 1,
  // after which its buffer is refilled.
  bool done = false;  // this wave's queries see no key of this tile, nor of any later one
  if (wave >= kPfWaves / 2) {
    for (int t = 0; t < ntiles; ++t) {
      pf_wait_tiles(min(ntiles - 1 - t, kPfAhead - 1));
      __syncthreads();  // tile t is in LDS; every wave is done with tile t - 2's buffer
      if (t + kPfAhead < ntiles) issue_tile(t + kPfAhead);
      if (done) continue;
      const int key0 = t * kPfKeys;
      if (t > 0) {
        softmax_now(key0 - kPfKeys, key0 > wave_vis_lo);
        sum_with_softmax(lds + ((t + kPfRing - 1) % kPfRing) * kPfBufBytes, 0, false, false);
      }
      if (key0 >= wave_vis_hi) {  // wave-uniform: no query of the wave sees this tile or later ones
        done = true;
        continue;
      }
      compute_scores(lds + (t % kPfRing) * kPfBufBytes);
    }
    if (!done && ntiles > 0) {
      const int key0 = (ntiles - 1) * kPfKeys;
      softmax_now(key0, key0 + kPfKeys > wave_vis_lo);
      sum_with_softmax(lds + ((ntiles - 1) % kPfRing) * kPfBufBytes, 0, false, false);
    }
  } else {
    for (int t = 0; t < ntiles; ++t) {
      pf_wait_tiles(min(ntiles - 1 - t, kPfAhead - 1));
      __syncthreads();  // tile t is in LDS; every wave is done with tile t - 2's buffer
      if (t + kPfAhead < ntiles) issue_tile(t + kPfAhead);
      if (done) continue;
      const int key0 = t * kPfKeys;
      const MLA_LDS char* tile = lds + (t % kPfRing) * kPfBufBytes;
      const MLA_LDS char* prev = lds + ((t + kPfRing - 1) % kPfRing) * kPfBufBytes;
      if (key0 >= wave_vis_hi) {  // wave-uniform: finish the sum over the previous tile
        scale_o();
        sum_with_softmax(prev, 0, false, false);
        done = true;
        continue;
      }
      compute_scores(tile);
      // [sum(t-1) | softmax(t)]
      scale_o();
      sum_with_softmax(prev, key0, key0 + kPfKeys > wave_vis_lo, true);
      pending_rescale = rescale;
      pending_alpha = alpha;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) pk[kk] = pn[kk];
    }
    if (!done && ntiles > 0) {
      scale_o();
      sum_with_softmax(lds + ((ntiles - 1) % kPfRing) * kPfBufBytes, 0, false, false);
    }
  }

  // normalise and store: element e of block cb is O^T[32 cb + 8 (e/4) + 4 hf + e%4][query]
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
    const float l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    if (qi < S) {
      uint16_t* dst = (uint16_t*)a.out + (((size_t)b * S + qi) * kHeads + h) * kDh;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16& d = o[cb];
          *(u32x2*)(dst + cb * 32 + g * 8 + hf * 4) =
              pack4(d[4 * g] * inv, d[4 * g + 1] * inv, d[4 * g + 2] * inv, d[4 * g + 3] * inv);
        }
      if (a.lse && hf == 0)
        a.lse[((size_t)b * S + qi) * kHeads + h] =
            l_tot > 0.f ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
    }
  }
}

hipError_t launch_prefill_attn(const PrefillArgs& a, hipStream_t stream) {
  forget_stale_error();
  const int64_t grid = (int64_t)a.B * kHeads * a.nqb;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(prefill_attn_kernel, dim3((unsigned)grid), dim3(64 * kPfWaves), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
