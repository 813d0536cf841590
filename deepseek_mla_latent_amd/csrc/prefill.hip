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
constexpr int kUpChunk = 64;                 // W rows (latent index k) per LDS chunk
constexpr int kUpMatBytes = kUpChunk * kDh * 2;  // 16 KiB: one chunk of W_UK[h] or W_UV[h]
constexpr int kUpBufBytes = 2 * kUpMatBytes;     // both matrices

constexpr int kPfQueries = 128;              // queries per attention workgroup (4 waves x 32)
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
// base plus a per-lane byte offset.  Completion is awaited with an explicit vmcnt wait.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds)
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
// K/V up-projection.  Workgroup = (sequence b, head h, 128-token tile); wave (wm, wn) computes the
// transposed product out^T[n][token] = sum_k W[k][n] c[token][k] for the 64 tokens of page wm and
// the 128 columns of matrix wn (0: W_UK -> K_nope, 1: W_UV -> V).  W^T is the A operand, read
// transposed from LDS (64-row chunks shared by the two page waves); c^T is the B operand, whose
// 8 consecutive k per lane are 16 contiguous bytes of a cache row, loaded straight from the pool.
// The accumulator layout gives each lane 4 consecutive n of one token: 8-byte bf16 stores.
//
// W chunk layout in LDS: matrix m, row r (k), 16-byte unit u stored at unit u ^ ((r & 3) << 2),
// so the 4 rows x 4 units of a transposed read fall on 16 distinct units (all 64 banks).
__global__ __launch_bounds__(256, 2) void kv_up_kernel(const uint16_t* __restrict__ pool,
                                                       const int32_t* __restrict__ block_table,
                                                       const int32_t* __restrict__ seq_lens,
                                                       const uint16_t* __restrict__ w_uk,
                                                       const uint16_t* __restrict__ w_uv, uint16_t* __restrict__ kv,
                                                       uint16_t* __restrict__ kpe, int max_pages, int tiles_per_seq) {
  __shared__ __attribute__((aligned(16))) char lds_raw[2 * kUpBufBytes];
  MLA_LDS char* lds = (MLA_LDS char*)lds_raw;

  const int id = xcd_remap(blockIdx.x, gridDim.x);  // one XCD walks all tiles of a few heads
  const int tt = id % tiles_per_seq;
  const int h = (id / tiles_per_seq) % kHeads;
  const int b = id / (tiles_per_seq * kHeads);
  const int L = seq_lens[b];
  const int npages = (L + kPage - 1) / kPage;
  if (tt * 2 >= npages) return;  // whole workgroup: no page of this tile holds a token

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int wm = wave & 1, wn = wave >> 1;
  const int page = tt * 2 + wm;
  const bool page_ok = page < npages;
  const int valid = page_ok ? min(kPage, L - page * kPage) : 0;  // tokens of this page
  const int pid = page_ok ? block_table[(size_t)b * max_pages + page] : 0;
  const uint16_t* prow = pool + (size_t)pid * kPage * kRow;
  const size_t Lp = (size_t)max_pages * kPage;

  // W chunks stream into LDS by direct-to-LDS loads: 32 pieces of 1 KiB (4 rows of one matrix)
  // per chunk, 8 per wave; LDS position p of row r receives source unit p ^ ((r & 3) << 2).
  const char* wsrc[2] = {(const char*)(w_uk + (size_t)h * kDc * kDh), (const char*)(w_uv + (size_t)h * kDc * kDh)};
  auto issue_chunk = [&](int c, int buf) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int pc = wave * 8 + j;
      const int m = pc >> 4, r = 4 * (pc & 15) + (lane >> 4), p = lane & 15;
      const int u = p ^ ((r & 3) << 2);
      dma16(wsrc[m], (uint32_t)((c * kUpChunk + r) * kDh * 2 + u * 16),
            lds_u32(lds + buf * kUpBufBytes + m * kUpMatBytes + (pc & 15) * 1024));
    }
  };

  // B operand (c^T) for k-step ks (16 latent indices) and token block tb: 16 B of the cache row.
  // Always loaded (a row of this page, or of pool page 0 for a page past the sequence) and
  // zeroed for tokens past the sequence end, so every wave issues the same number of loads.
  const bool tok_ok[2] = {l32 < valid, 32 + l32 < valid};
  auto load_c = [&](int ks, int tb) -> bf16x8 {
    const bf16x8 v = *(const bf16x8*)(prow + (size_t)(tb * 32 + l32) * kRow + ks * 16 + hf * 8);
    return tok_ok[tb] ? v : bf16x8{};
  };

  // A operand (W^T) addresses: rows k = 16 ks' + 8 hf + (lane >> 2 & 3) (+4 for the high half),
  // columns n = 32 nb + 16 ((lane >> 4) & 1) + 4 (lane & 3).
  const int tr_row = 8 * hf + ((lane >> 2) & 3);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  auto tr_off = [&](int r, int n) { return r * 256 + ((((n >> 3) ^ ((r & 3) << 2))) << 4) + (n & 7) * 2; };

  f32x16 acc[4][2];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) acc[nb][tb] = f32x16{};

  constexpr int kChunks = kDc / kUpChunk;  // 8
  bf16x8 cf[4][2], cn[4][2];
  issue_chunk(0, 0);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) cf[ks][tb] = load_c(ks, tb);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  for (int c = 0; c < kChunks; ++c) {
    // next chunk's W (into the other buffer, last read before the previous barrier) and c rows
    if (c + 1 < kChunks) {
      issue_chunk(c + 1, (c + 1) & 1);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) cn[ks][tb] = load_c((c + 1) * 4 + ks, tb);
    }
    const MLA_LDS char* wbuf = lds + (c & 1) * kUpBufBytes + wn * kUpMatBytes;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 af[4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int r = ks * 16 + tr_row, n = nb * 32 + tr_col;
        af[nb] = lds_tr_pair(wbuf + tr_off(r, n), wbuf + tr_off(r + 4, n));
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) acc[nb][tb] = mfma32x32x16(af[nb], cf[ks][tb], acc[nb][tb]);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) cf[ks][tb] = cn[ks][tb];
  }

  // Stores: element e of block (nb, tb) is out^T[32 nb + 8 (e/4) + 4 hf + e%4][32 tb + l32].
  if (page_ok) {
    uint16_t* dst = kv + (((size_t)b * kHeads + h) * Lp + (size_t)page * kPage) * kKvRow + wn * kDh;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int tok = tb * 32 + l32;
      const bool ok = tok < valid;  // rows past the sequence end are written as zeros
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16& d = acc[nb][tb];
          u32x2 v = ok ? pack4(d[4 * g], d[4 * g + 1], d[4 * g + 2], d[4 * g + 3]) : u32x2{0u, 0u};
          *(u32x2*)(dst + (size_t)tok * kKvRow + nb * 32 + g * 8 + hf * 4) = v;
        }
    }
    // the shared RoPE key: head-0 workgroups copy it densely, zeros past the sequence end
    if (h == 0 && wn == 0) {
      uint16_t* kdst = kpe + ((size_t)b * Lp + (size_t)page * kPage) * kDr;
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int q = it * 64 + lane, row = q >> 3, u = q & 7;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (row < valid) v = *(const u32x4*)(prow + (size_t)row * kRow + kDc + u * 8);
        *(u32x4*)(kdst + (size_t)row * kDr + u * 8) = v;
      }
    }
  }
}

hipError_t launch_kv_up_grid(const void* pool, const int32_t* block_table, const int32_t* seq_lens,
                             const void* w_uk, const void* w_uv, void* kv, void* kpe, int batch, int max_pages,
                             int tiles, hipStream_t stream) {
  const int64_t grid = (int64_t)batch * kHeads * tiles;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(kv_up_kernel, dim3((unsigned)grid), dim3(256), 0, stream, (const uint16_t*)pool, block_table,
                     seq_lens, (const uint16_t*)w_uk, (const uint16_t*)w_uv, (uint16_t*)kv, (uint16_t*)kpe,
                     max_pages, tiles);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------
// Causal multi-head attention over the up-projected keys.  Workgroup = (b, h, 128-query block);
// wave w owns 32 queries.  Per 64-key tile:
//   S^T (keys x queries) = [K_nope | k_pe] Q^T: 2 key blocks x 12 MFMAs, keys as the A operand
//   (ds_read_b128 rows), the wave's queries as the B operand held in registers for the whole walk;
//   online softmax per query column (the lane pair l, l^32 holds one query);
//   O^T (dv x queries) += V^T P^T: 4 dv blocks x 4 MFMAs, V^T read transposed from the same tile.
// The accumulator layout of S^T is the B-operand layout of P^T when the 16 keys of an MFMA step
// are taken in the order the accumulator holds them; the V^T reads use the same key order.
// Tile layout: key row r of [K_nope | V] (32 units of 16 B), unit u at u ^ swz(r) (low 4 bits),
// k_pe row r (8 units) at u ^ ((r >> 1) & 7): both read patterns hit 16 distinct units per
// 16 lanes.  Tiles stream in by direct-to-LDS loads, one tile ahead (two buffers).
// The running max is only raised when a tile's max exceeds it by more than 2^8 (log2 units).
__device__ __forceinline__ int pf_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int pf_swz_pe(int r) { return (r >> 1) & 7; }

__global__ __launch_bounds__(256, 2) void prefill_attn_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) char lds_raw[2 * kPfBufBytes];
  MLA_LDS char* lds = (MLA_LDS char*)lds_raw;

  const int nbh = a.B * kHeads;
  const int id = xcd_remap(blockIdx.x, gridDim.x);  // one XCD walks all query blocks of a few heads
  const int bh = id / a.nqb;
  const int qb = a.nqb - 1 - id % a.nqb;  // longest key ranges first
  if (bh >= nbh) return;
  const int b = bh / kHeads, h = bh % kHeads;
  const int L = a.seq_lens[b], S = a.S;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int q0 = qb * kPfQueries;
  const int qi = q0 + wave * 32 + l32;    // this lane's query (column)
  const int qc = min(qi, S - 1);           // padding queries behave like the last one
  auto visible = [&](int q) { return a.causal ? max(0, min(L, L - S + q + 1)) : L; };
  const int vis = visible(qc);
  const int kend = visible(min(S - 1, q0 + kPfQueries - 1));  // keys any query of the block sees
  const int ntiles = (kend + kPfKeys - 1) / kPfKeys;
  const int wave_vis = visible(min(S - 1, q0 + wave * 32));   // fewest keys a query of the wave sees

  const size_t Lp = (size_t)a.Lp;
  const char* kv_seq = (const char*)a.kv + ((size_t)b * kHeads + h) * Lp * kKvRow * 2;
  const char* pe_seq = (const char*)a.kpe + (size_t)b * Lp * kDr * 2;

  // tile DMA: 32 KiB of [K_nope | V] rows (8 loads per wave) + 8 KiB of k_pe rows (2 per wave)
  auto issue_tile = [&](int t, int buf) {
    MLA_LDS char* dst = lds + buf * kPfBufBytes;
    const char* kv_t = kv_seq + (size_t)t * kPfKeys * kKvRow * 2;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = wave * 8 + j;             // 1 KiB piece: rows 2c, 2c+1
      const int r = 2 * c + (lane >> 5), p = lane & 31;
      const int u = (p & 16) | ((p & 15) ^ pf_swz(r));
      dma16(kv_t, (uint32_t)(r * kKvRow * 2 + u * 16), lds_u32(dst + c * 1024));
    }
    const char* pe_t = pe_seq + (size_t)t * kPfKeys * kDr * 2;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = wave * 2 + j;             // rows 8c .. 8c+7
      const int r = 8 * c + (lane >> 3), p = lane & 7;
      const int u = p ^ pf_swz_pe(r);
      dma16(pe_t, (uint32_t)(r * kDr * 2 + u * 16), lds_u32(dst + kPfKvBytes + c * 1024));
    }
  };

  if (ntiles > 0) issue_tile(0, 0);

  // queries as B operands: k-steps 0..7 from q_nope, 8..11 from q_pe
  bf16x8 qf[12];
  {
    const uint16_t* qn = (const uint16_t*)a.q_nope + (((size_t)b * S + qc) * kHeads + h) * kDh;
    const uint16_t* qp = (const uint16_t*)a.q_pe + (((size_t)b * S + qc) * kHeads + h) * kDr;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = *(const bf16x8*)(qn + ks * 16 + hf * 8);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[8 + ks] = *(const bf16x8*)(qp + ks * 16 + hf * 8);
  }

  // per-lane operand offsets within a tile buffer
  int k_off[2][12];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int r = kb * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) k_off[kb][ks] = r * kKvRow * 2 + (((2 * ks + hf) ^ pf_swz(r)) << 4);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) k_off[kb][8 + ks] = kPfKvBytes + r * kDr * 2 + (((2 * ks + hf) ^ pf_swz_pe(r)) << 4);
  }
  // V^T reads: key rows 16 kk + 4 hf + (lane >> 2 & 3) (+8 for the high half), dv columns
  // 32 cb + 16 ((lane >> 4) & 1) + 4 (lane & 3)
  const int vr = 4 * hf + ((lane >> 2) & 3);
  const int vc = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  auto v_off = [&](int r, int dv) {
    const int u = 16 + (dv >> 3);
    return r * kKvRow * 2 + (((u & 16) | ((u & 15) ^ pf_swz(r))) << 4) + (dv & 7) * 2;
  };

  f32x16 o[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) o[cb] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale_log2;

  for (int t = 0; t < ntiles; ++t) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (t + 1 < ntiles) issue_tile(t + 1, (t + 1) & 1);
    const MLA_LDS char* tile = lds + (t & 1) * kPfBufBytes;

    f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < 12; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[kb] = mfma32x32x16(lds_b128(tile + k_off[kb][ks]), qf[ks], s[kb]);

    // scaled logits in log2 units; keys past this query's visible count are -inf
    const int key0 = t * kPfKeys;
    const bool need_mask = key0 + kPfKeys > wave_vis;
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float x = s[kb][e] * sl2;
        if (need_mask) {
          const int key = key0 + kb * 32 + (e >> 2) * 8 + hf * 4 + (e & 3);
          x = key < vis ? x : -INFINITY;
        }
        s[kb][e] = x;
        mt = fmaxf(mt, x);
      }
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
      mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    if (__any(mt > m_run + 8.0f)) {  // wave-uniform: raise the reference, rescale O and l
      const float m_new = fmaxf(m_run, mt);
      const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[cb][e] *= alpha;
      m_run = m_new;
    }
    const float msub = m_run == -INFINITY ? 0.f : m_run;  // no visible key yet: every p is 0
    bf16x8 pk[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = __builtin_amdgcn_exp2f(s[kb][e] - msub);
        l_run += p;
        pk[kb * 2 + (e >> 3)][e & 7] = (__bf16)p;
      }

#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int r = kk * 16 + vr;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int dv = cb * 32 + vc;
        const bf16x8 vf = lds_tr_pair(tile + v_off(r, dv), tile + v_off(r + 8, dv));
        o[cb] = mfma32x32x16(vf, pk[kk], o[cb]);
      }
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
  const int64_t grid = (int64_t)a.B * kHeads * a.nqb;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(prefill_attn_kernel, dim3((unsigned)grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
