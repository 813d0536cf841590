// The two per-head projections around the latent attention, gfx950.
//
//   absorb:   q_lat[n,h,c] = sum_d W_UK[h,c,d] q_nope[n,h,d]     (c < 512, d < 128)
//   out-proj: out[n,h,v]   = sum_c o_lat[n,h,c] W_UV[h,c,v]       (v < 128)
//
// W_UK is applied transposed to the query and W_UV after the latent average, so K and V are
// never formed: "DeepSeek-V2的推理成本如何计算？" (izhida.com), answer "专家"; "【笔记】MLA矩阵吸收分析"
// §二.2 step 2 and §三.2 step 2.  Both are batched GEMVs / thin GEMMs (M = tokens = B*S) whose
// cost is reading the 128 x 512 x 128 weight once (the same izhida answer notes that the main
// cost of the W_V product is reading W_V), so they are HBM-bound.  Each workgroup streams its
// weight slice exactly once, and every wave issues all the loads of a step before its first
// use, so a launch costs about one memory round trip plus the transfer.
#include "common.h"
#include "kernels.h"

namespace mla {

// Forces the values to be complete here: every load producing them is issued before this point,
// and the compiler cannot trickle them out one MFMA at a time.
template <typename T>
__device__ __forceinline__ void settle(const T& x) {
  asm volatile("" ::"v"(x));
}

// ---------------------------------------------------------------------------------------------
// absorb, fp32: grid (4 latent blocks of 128, 128 heads), 4 waves; wave w owns 32 latent rows
// c in [128 bx + 32 w, +32).  D(c x tokens) = W_UK[h] rows (A, straight from global) x q_nope^T
// (B) on fp32 MFMAs.  Columns of D belong to single tokens, so a token slot past the end reads a
// valid row (token 0) and its column is simply not stored.
__global__ __launch_bounds__(256) void absorb_q_f32_kernel(const void* __restrict__ q_nope,
                                                           const void* __restrict__ w_uk,
                                                           void* __restrict__ q_lat, int tokens) {
  const int h = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l32 = lane & 31, hf = lane >> 5;
  const int c_base = 128 * blockIdx.x + 32 * wave;
  const size_t wrow = ((size_t)h * kDc + c_base + l32) * kDh;
  // fp32: k step (m, j) pairs lane half hf with d = 8 m + 4 hf + j (a float4 per m).
  f32x4 aw[16];
  const f32x4* W = (const f32x4*)((const float*)w_uk + wrow + 4 * hf);
#pragma unroll
  for (int m = 0; m < 16; ++m) aw[m] = W[2 * m];
  for (int nb = 0; nb * 32 < tokens; ++nb) {
    const int n = 32 * nb + l32;
    const bool ok = n < tokens;
    const f32x4* Q = (const f32x4*)((const float*)q_nope + ((size_t)(ok ? n : 0) * kHeads + h) * kDh + 4 * hf);
    f32x4 bq[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) bq[m] = Q[2 * m];
#pragma unroll
    for (int m = 0; m < 16; ++m) settle(bq[m]);
    f32x16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
    for (int m = 0; m < 16; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = mfma32x32x2f32(aw[m][j], bq[m][j], acc);
    if (ok) {
      float* dst = (float*)q_lat + ((size_t)n * kHeads + h) * kDc + c_base + 4 * hf;
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(f32x4*)(dst + 8 * g) = f32x4{acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
    }
  }
}

// ---------------------------------------------------------------------------------------------
// absorb, bf16: grid (4 latent blocks of 128, 128 heads), 4 waves; wave w owns latent rows
// c in [128 bx + 32 w, +32).  Its W_UK rows and each 32-token block's q_nope rows reach LDS by
// 1 KiB direct-to-LDS loads (4 rows of 256 B; 16-byte unit u of row r stored at u ^ (r & 15)), so
// every global read covers whole cache lines and q_nope is read once per workgroup, not per wave.
// D(c x tokens) = W_UK[h] rows (A) x q_nope^T (B); the block's 32 x 128 outputs leave through LDS
// as whole 256-byte rows.  A token slot past the end reads token 0 and is not stored.
__global__ __launch_bounds__(256) void absorb_q_bf16_kernel(const uint16_t* __restrict__ q_nope,
                                                            const uint16_t* __restrict__ w_uk,
                                                            uint16_t* __restrict__ q_lat, int tokens) {
  __shared__ __attribute__((aligned(1024))) char w_lds[128 * 256];  // the workgroup's 128 W rows
  __shared__ __attribute__((aligned(1024))) char q_lds[32 * 256];   // one token block of q_nope
  __shared__ __attribute__((aligned(1024))) char o_lds[32 * 256];   // its 32 x 128 outputs
  const int h = blockIdx.y, cb = 128 * blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, l32 = lane & 31, hf = lane >> 5, r16 = lane >> 4, u16 = lane & 15;
  {  // this wave's 32 W rows: load i covers rows 4 i .. 4 i + 3
    const char* src = (const char*)(w_uk + ((size_t)h * kDc + cb + 32 * wave) * kDh);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 4 * i + r16;
      __builtin_amdgcn_global_load_lds((const MLA_GLOBAL void*)(src + r * 256 + ((u16 ^ (r & 15)) * 16)),
                                       (MLA_LDS void*)(w_lds + (32 * wave + 4 * i) * 256), 16, 0, 0);
    }
  }
  for (int nb = 0; nb * 32 < tokens; ++nb) {
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {  // token rows 4 j .. 4 j + 3 of the block, two loads per wave
      const int t = 4 * (2 * wave + jj) + r16;
      const int n = 32 * nb + t < tokens ? 32 * nb + t : 0;
      const char* src = (const char*)(q_nope + ((size_t)n * kHeads + h) * kDh);
      __builtin_amdgcn_global_load_lds((const MLA_GLOBAL void*)(src + ((u16 ^ (t & 15)) * 16)),
                                       (MLA_LDS void*)(q_lds + 4 * (2 * wave + jj) * 256), 16, 0, 0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's W rows and q rows have landed
    __syncthreads();                                  // every wave's q rows
    f32x16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int u = (2 * ks + hf) ^ (l32 & 15);
      const bf16x8 aw = *(const MLA_LDS bf16x8*)(w_lds + (32 * wave + l32) * 256 + u * 16);
      const bf16x8 bq = *(const MLA_LDS bf16x8*)(q_lds + l32 * 256 + u * 16);
      acc = mfma32x32x16(aw, bq, acc);
    }
    // element e: latent 32 w + (e/4)*8 + 4 hf + e%4 (of the block's 128) of token l32: 8 bytes at
    // 16-byte unit 4 w + e/4, half hf, of the token's 256-byte staging row
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const u32x2 v = {pack_bf16x2(acc[4 * g], acc[4 * g + 1]), pack_bf16x2(acc[4 * g + 2], acc[4 * g + 3])};
      *(MLA_LDS u32x2*)(o_lds + l32 * 256 + (((4 * wave + g) ^ (l32 & 15)) * 16) + hf * 8) = v;
    }
    __syncthreads();
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {  // token rows 4 j .. 4 j + 3, 16 lanes (256 B) per row
      const int t = 4 * (2 * wave + jj) + r16;
      const int n = 32 * nb + t;
      const u32x4 v = *(const MLA_LDS u32x4*)(o_lds + t * 256 + ((u16 ^ (t & 15)) * 16));
      if (n < tokens) *(u32x4*)(q_lat + ((size_t)n * kHeads + h) * kDc + cb + 8 * u16) = v;
    }
    __syncthreads();  // the block's q and output rows are read before the next block reuses them
  }
}

// ---------------------------------------------------------------------------------------------
// out-proj, bf16: one workgroup per (head h, value half vh); logical ids 2h, 2h+1 run on the
// same XCD, so the second read of o_lat[., h, .] can come from that XCD's L2.
//
// Wave w owns latent rows [128 w, +128): it copies W_UV[h][those rows][64 vh .. +64) into LDS
// and, per 32-token block, the matching o_lat slices (512 B per token, two tokens per 1 KiB
// direct-to-LDS load), so every global read is a whole 1 KiB.  Per token block it computes the
// partial D(64 values x 32 tokens) over its 128 latent rows: A = W_UV^T by transposed LDS reads,
// B = o_lat^T split into hi + lo bf16 parts (two MFMAs, so the fp32 latent input keeps about 16
// mantissa bits).  The four partials are summed through LDS.  A wave only ever reads the LDS rows
// it loaded itself, so only the sums need barriers.
constexpr int kOpRowBytes = 128;  // one latent row of the 64-value slice
// 16-byte unit u of latent row c is stored at unit u ^ op_swz(c): the transposed reads touch
// 4 consecutive rows x 64 B, which this spreads over all 64 banks.
__device__ __forceinline__ int op_swz(int c) { return ((c >> 1) & 1) << 2; }
// o_lat staging: token n's 512 B slice as 32 units of 16 B, unit u stored at u ^ (n & 15), so the
// 32 tokens' B-operand reads at one column hit 16 different bank groups (2-way at most).
constexpr int kOStageBytes = 32 * 512;  // per wave

__global__ __launch_bounds__(256, 1) void out_proj_bf16_kernel(const float* __restrict__ o_lat,
                                                               const uint16_t* __restrict__ w_uv,
                                                               uint16_t* __restrict__ out, int tokens) {
  __shared__ __attribute__((aligned(1024))) char wl_raw[kDc * kOpRowBytes];  // 64 KiB
  __shared__ __attribute__((aligned(1024))) char os_raw[4 * kOStageBytes];    // 64 KiB, then the sums
  MLA_LDS char* const wl = (MLA_LDS char*)wl_raw;
  MLA_LDS char* const os = (MLA_LDS char*)os_raw;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int h = id >> 1, vh = id & 1;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, l32 = lane & 31, hf = lane >> 5;
  const int c0 = 128 * wave;
  MLA_LDS char* const ow = os + wave * kOStageBytes;

  {  // W slice rows [c0, c0 + 128): 16 loads of 8 rows x 128 B
    const char* src = (const char*)(w_uv + (size_t)h * kDc * kDh + 64 * vh);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int c = c0 + 8 * i + (lane >> 3);
      const int u = (lane & 7) ^ op_swz(c);
      __builtin_amdgcn_global_load_lds((const MLA_GLOBAL void*)(src + (size_t)c * kDh * 2 + u * 16),
                                       (MLA_LDS void*)(wl + (c0 + 8 * i) * kOpRowBytes), 16, 0, 0);
    }
  }
  // o_lat slices of block nb: load i covers tokens 2i, 2i+1 (lane halves); a token past the end
  // reads token 0 (its column is not stored).
  auto load_o = [&](int nb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int t = 2 * i + hf;
      int n = 32 * nb + t;
      n = n < tokens ? n : 0;
      const int u = l32 ^ (t & 15);
      const char* src = (const char*)(o_lat + ((size_t)n * kHeads + h) * kDc + c0) + u * 16;
      __builtin_amdgcn_global_load_lds((const MLA_GLOBAL void*)src, (MLA_LDS void*)(ow + i * 1024), 16, 0, 0);
    }
  };

  // Transposed A read (32 values x 8 latent rows per pair): in each 16-lane group, source lane
  // s supplies latent row c + s/4 and value columns 4 (s%4) .. +3 of the group's 16 columns.
  const int r4 = (lane >> 2) & 3, g1 = (lane >> 4) & 1, q4 = lane & 3;
  const int sw = (r4 >> 1) & 1;  // op_swz of the row, as a flip of the value block bit
  const MLA_LDS char* a_base[2];
#pragma unroll
  for (int vb = 0; vb < 2; ++vb)
    a_base[vb] = wl + (c0 + 8 * hf + r4) * kOpRowBytes + 64 * (vb ^ sw) + 16 * (2 * g1 + (q4 >> 1)) + 8 * (q4 & 1);

  const int nblocks = (tokens + 31) / 32;
  for (int nb = 0; nb < nblocks; ++nb) {
    load_o(nb);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's W rows and o slices have landed
    // B operand of k step ks for lane (token l32, half hf): latent c0 + 16 ks + 8 hf + j, i.e.
    // units 4 ks + 2 hf and 4 ks + 2 hf + 1 of the token's slice.
    bf16x8 bh[8], bl[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const MLA_LDS char* row = ow + (l32 >> 1) * 1024 + (l32 & 1) * 512;
      const int u0 = (4 * ks + 2 * hf) ^ (l32 & 15);
      const f32x4 a = *(const MLA_LDS f32x4*)(row + u0 * 16);
      const f32x4 b = *(const MLA_LDS f32x4*)(row + (u0 ^ 1) * 16);
      const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
      u32x4 hw, lw;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        hw[j] = pack_bf16x2(v[2 * j], v[2 * j + 1]);
        const float r0 = v[2 * j] - __uint_as_float(hw[j] << 16);
        const float r1 = v[2 * j + 1] - __uint_as_float(hw[j] & 0xffff0000u);
        lw[j] = pack_bf16x2(r0, r1);
      }
      bh[ks] = __builtin_bit_cast(bf16x8, hw);
      bl[ks] = __builtin_bit_cast(bf16x8, lw);
    }

    f32x16 acc[2];
#pragma unroll
    for (int vb = 0; vb < 2; ++vb)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[vb][e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int vb = 0; vb < 2; ++vb) {
        const MLA_LDS char* p = a_base[vb] + ks * 16 * kOpRowBytes;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)p);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)(p + 4 * kOpRowBytes));
        const i16x8 a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        const bf16x8 av = __builtin_bit_cast(bf16x8, a8);
        acc[vb] = mfma32x32x16(av, bh[ks], acc[vb]);
        acc[vb] = mfma32x32x16(av, bl[ks], acc[vb]);
      }

    // Sum the four waves' partials in the staging area: red[((w * 2 + vb) * 16 + e) * 64 + lane];
    // element e of lane l is value 32 vb + (e/4)*8 + 4 (l/32) + e%4 of token l%32.
    __syncthreads();  // every wave has read its o slices
    MLA_LDS float* red = (MLA_LDS float*)os;
#pragma unroll
    for (int vb = 0; vb < 2; ++vb)
#pragma unroll
      for (int e = 0; e < 16; ++e) red[((wave * 2 + vb) * 16 + e) * 64 + lane] = acc[vb][e];
    __syncthreads();
    {
      const int vb = wave >> 1;
      const int n = 32 * nb + l32;
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        const int g = 2 * (wave & 1) + gg;
        float s[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = 4 * g + i;
          s[i] = red[((0 * 2 + vb) * 16 + e) * 64 + lane] + red[((1 * 2 + vb) * 16 + e) * 64 + lane] +
                 red[((2 * 2 + vb) * 16 + e) * 64 + lane] + red[((3 * 2 + vb) * 16 + e) * 64 + lane];
        }
        if (n < tokens) {
          const int v = 64 * vh + 32 * vb + 8 * g + 4 * hf;
          const u32x2 pk = {pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3])};
          *(u32x2*)(out + ((size_t)n * kHeads + h) * kDh + v) = pk;
        }
      }
    }
    __syncthreads();  // the sums are read before the next block's slices land in the area
  }
}

// ---------------------------------------------------------------------------------------------
// Split merge + out-proj in one kernel, bf16: the decode attention's split partials (o_k, lse_k)
// are merged by their log-sum-exp weights and projected by W_UV without the merged o_lat making
// a round trip through HBM (it is written only when asked for).  Merging is "【笔记】MLA矩阵吸收分析"
// §三.2 step 1 over key ranges, the projection its step 2.
//
// Workgroup = (head h, block of 16 rows), 8 waves (two per SIMD); the blocks of one head have
// consecutive logical ids (one XCD, so W_UV[h] comes from HBM once).  Wave w owns latent rows
// [64 w, +64), so each wave's loads (2 batches of 4 splits' partials and lse, 16 W loads) stay
// within the 63 the vector-memory counter tracks and go out in one round trip:
//   * its 16 KiB slice of W_UV[h] goes to LDS (direct-to-LDS, 4 rows of 256 B per load);
//   * lane l merges row l % 16 at latent 64 w + 32 ks + 8 (l / 16) + j (ks < 2, j < 8): exactly
//     the B operand of a 16x16x32 MFMA, so the merged values never leave the lane.  They are split
//     into hi + lo bf16 (two MFMAs, about 16 mantissa bits of the fp32 merge kept);
//   * D(16 values x 16 rows) for the 8 value blocks over its 64 latent rows, A = W_UV^T by
//     transposed LDS reads; the eight waves' partial sums meet in LDS.
// LDS row c of a wave's slice holds 32-byte block b (16 values) at block b ^ fsw(c) with
// fsw(c) = (c & 3) | ((c >> 3) & 1) << 2: a transposed read covers 16 rows x 32 B, which this puts
// on every bank pair exactly twice.
constexpr int kMopRows = 16;
__device__ __forceinline__ int mop_swz(int c) { return (c & 3) | (((c >> 3) & 1) << 2); }

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(512, 1) void merge_out_proj_kernel(const uint16_t* __restrict__ o_part,
                                                                const float* __restrict__ lse_part,
                                                                const uint16_t* __restrict__ w_uv,
                                                                uint16_t* __restrict__ out, float* __restrict__ o_lat,
                                                                float* __restrict__ lse, int rows, int num_splits) {
  __shared__ __attribute__((aligned(1024))) char wl_raw[kDc * kDh * 2];  // 128 KiB, then the sums
  MLA_LDS char* const wl = (MLA_LDS char*)wl_raw;
  const int nblk = (rows + kMopRows - 1) / kMopRows;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int h = id / nblk, r0 = (id % nblk) * kMopRows;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, g = lane >> 4, s16 = lane & 15;
  const int c0 = 64 * wave;
  MLA_LDS char* const ws = wl + wave * (64 * kDh * 2);  // this wave's 64 rows x 256 B

  // merge: row n = r0 + s16 (a row past the end reads row r0, which exists, and stores nothing)
  const int n = r0 + s16 < rows ? r0 + s16 : r0;
  const size_t base = (size_t)n * num_splits * kHeads + h;  // split k at base + k * kHeads
  const float* lp = lse_part + base;
  const uint16_t* op = o_part + base * kDc + c0 + 8 * g;  // + 32 ks
  // Batches of 4 splits (a split past the end repeats the last one with weight 0), two in flight.
  struct Batch {
    u32x4 x[4][2];  // [split][ks]
    float l[4];
  };
  auto load = [&](int kb, Batch& bt) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = kb + j < num_splits ? kb + j : num_splits - 1;
      bt.l[j] = kb + j < num_splits ? lp[(size_t)k * kHeads] : -INFINITY;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) bt.x[j][ks] = *(const u32x4*)(op + (size_t)k * kHeads * kDc + 32 * ks);
    }
  };
  Batch b0, b1;
  load(0, b0);
  if (4 < num_splits) load(4, b1);
  // W_UV[h] rows [c0, c0 + 64) after the first partials, so waiting for those does not wait for
  // W: load i covers local rows 4 i .. 4 i + 3 (16 lanes each)
  {
    const char* src = (const char*)(w_uv + ((size_t)h * kDc + c0) * kDh);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int c = 4 * i + g, u = s16;
      const int us = 2 * ((u >> 1) ^ mop_swz(c)) + (u & 1);
      __builtin_amdgcn_global_load_lds((const MLA_GLOBAL void*)(src + (size_t)c * kDh * 2 + us * 16),
                                       (MLA_LDS void*)(ws + i * 1024), 16, 0, 0);
    }
  }

  // Running log-sum-exp merge: weights are taken against the largest lse seen so far, and the
  // sums are rescaled when a batch raises it (an empty split has lse = -inf and weight 0).
  constexpr float kLog2e = 1.4426950408889634f;
  f32x4 acc_o[4];  // latent 32 ks + 8 g + 4 e2 + e in acc_o[2 ks + e2][e]
#pragma unroll
  for (int i = 0; i < 4; ++i) acc_o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, sum = 0.f;
  auto consume = [&](const Batch& bt) {
    const float m_new = fmaxf(fmaxf(m, fmaxf(bt.l[0], bt.l[1])), fmaxf(bt.l[2], bt.l[3]));
    const float scale = m_new > m ? (m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m - m_new) * kLog2e)) : 1.f;
    m = m_new;
    sum *= scale;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc_o[i] *= scale;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float w = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((bt.l[j] - m) * kLog2e);
      sum += w;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const u32x4 u = bt.x[j][ks];
        acc_o[2 * ks] += w * f32x4{__uint_as_float(u[0] << 16), __uint_as_float(u[0] & 0xffff0000u),
                                   __uint_as_float(u[1] << 16), __uint_as_float(u[1] & 0xffff0000u)};
        acc_o[2 * ks + 1] += w * f32x4{__uint_as_float(u[2] << 16), __uint_as_float(u[2] & 0xffff0000u),
                                       __uint_as_float(u[3] << 16), __uint_as_float(u[3] & 0xffff0000u)};
      }
    }
  };
  for (int kb = 0; kb < num_splits; kb += 8) {
    consume(b0);
    if (kb + 8 < num_splits) load(kb + 8, b0);
    if (kb + 4 < num_splits) {
      consume(b1);
      if (kb + 12 < num_splits) load(kb + 12, b1);
    }
  }
  const float inv = sum > 0.f ? 1.0f / sum : 0.f;
  const bool live = r0 + s16 < rows;
  bf16x8 bh[2], bl[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const f32x4 a = acc_o[2 * ks] * inv, b = acc_o[2 * ks + 1] * inv;
    if (o_lat && live) {
      f32x4* dst = (f32x4*)(o_lat + ((size_t)n * kHeads + h) * kDc + c0 + 32 * ks + 8 * g);
      dst[0] = a;
      dst[1] = b;
    }
    const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    u32x4 hw, lw;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      hw[j] = pack_bf16x2(v[2 * j], v[2 * j + 1]);
      const float d0 = v[2 * j] - __uint_as_float(hw[j] << 16);
      const float d1 = v[2 * j + 1] - __uint_as_float(hw[j] & 0xffff0000u);
      lw[j] = pack_bf16x2(d0, d1);
    }
    bh[ks] = __builtin_bit_cast(bf16x8, hw);
    bl[ks] = __builtin_bit_cast(bf16x8, lw);
  }
  if (lse && live && wave == 0 && g == 0) lse[(size_t)n * kHeads + h] = m == -INFINITY ? -INFINITY : m + logf(sum);

  // A operand of value block mb, k step ks: two transposed reads; source lane s of group g gives
  // local row 32 ks + 8 g + 4 t + s/4 and values 16 mb + 4 (s%4) .. +3 (t = 0, 1).
  const int fsw = (s16 >> 2) | ((g & 1) << 2);  // mop_swz of every row this lane addresses
  const MLA_LDS char* a_row = ws + (8 * g + (s16 >> 2)) * (kDh * 2) + (s16 & 3) * 8;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's W rows have landed
  f32x4 acc[8];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const MLA_LDS char* p = a_row + ks * 32 * (kDh * 2) + ((mb ^ fsw) * 32);
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)p);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)(p + 4 * (kDh * 2)));
      const i16x8 a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      const bf16x8 av = __builtin_bit_cast(bf16x8, a8);
      acc[mb] = mfma16x16x32(av, bh[ks], acc[mb]);
      acc[mb] = mfma16x16x32(av, bl[ks], acc[mb]);
    }

  // The eight waves' partial sums meet in LDS (over the W slices, once every wave is done with
  // them): red[((w * 8 + mb) * 4 + i) * 64 + lane], element i of lane l being value 16 mb + 4 g + i
  // of row s16.  Wave w then adds value block w.
  __syncthreads();
  MLA_LDS float* red = (MLA_LDS float*)wl;
#pragma unroll
  for (int mb = 0; mb < 8; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[((wave * 8 + mb) * 4 + i) * 64 + lane] = acc[mb][i];
  __syncthreads();
  {
    const int mb = wave;
    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float t = 0.f;
#pragma unroll
      for (int ww = 0; ww < 8; ++ww) t += red[((ww * 8 + mb) * 4 + i) * 64 + lane];
      sv[i] = t;
    }
    if (live) {
      const u32x2 pk = {pack_bf16x2(sv[0], sv[1]), pack_bf16x2(sv[2], sv[3])};
      *(u32x2*)(out + ((size_t)n * kHeads + h) * kDh + 16 * mb + 4 * g) = pk;
    }
  }
}

// out-proj, fp32: grid (2 value halves of 64, 128 heads), 4 waves.  The workgroup stages
// W_UV[h][:, 64 bx .. +64) in LDS, then computes D(v x tokens) = W_UV^T x o_lat^T with the fp32
// MFMA for every (32-value block, 32-token block) pair, round-robin over the waves.
__global__ __launch_bounds__(256) void out_proj_f32_kernel(const float* __restrict__ o_lat,
                                                           const float* __restrict__ w_uv, float* __restrict__ out,
                                                           int tokens) {
  __shared__ float wl[kDc * 64];  // 128 KiB
  const int h = blockIdx.y, vh = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l32 = lane & 31, hf = lane >> 5;
  {
    const float* src = w_uv + (size_t)h * kDc * kDh + 64 * vh;
    for (int u0 = 0; u0 < kDc * 16; u0 += 256 * 8) {
      f32x4 t[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int u = u0 + threadIdx.x + 256 * k;
        t[k] = *(const f32x4*)(src + (size_t)(u >> 4) * kDh + (u & 15) * 4);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int u = u0 + threadIdx.x + 256 * k;
        *(f32x4*)(wl + (u >> 4) * 64 + (u & 15) * 4) = t[k];
      }
    }
  }
  __syncthreads();

  const int ntb = (tokens + 31) / 32;
  for (int combo = wave; combo < 2 * ntb; combo += 4) {
    const int vb = combo & 1, nb = combo >> 1;
    const int n = 32 * nb + l32;
    const bool ok = n < tokens;
    const float* O = o_lat + ((size_t)(ok ? n : 0) * kHeads + h) * kDc;
    f32x16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
    // k step (m, j) pairs lane half hf with latent row c = 8 m + 4 hf + j.
    for (int m0 = 0; m0 < 64; m0 += 16) {
      f32x4 xb[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) xb[k] = *(const f32x4*)(O + 8 * (m0 + k) + 4 * hf);
#pragma unroll
      for (int k = 0; k < 16; ++k) settle(xb[k]);
#pragma unroll
      for (int k = 0; k < 16; ++k)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = 8 * (m0 + k) + 4 * hf + j;
          acc = mfma32x32x2f32(wl[c * 64 + 32 * vb + l32], xb[k][j], acc);
        }
    }
    if (ok) {  // element e: value 32 vb + (e/4)*8 + 4 hf + e%4 of token n
      float* dst = out + ((size_t)n * kHeads + h) * kDh + 64 * vh + 32 * vb + 4 * hf;
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(f32x4*)(dst + 8 * g) = f32x4{acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
    }
  }
}

hipError_t launch_absorb_q(const void* q_nope, const void* w_uk, void* q_lat, int tokens, bool bf16,
                           hipStream_t stream) {
  forget_stale_error();
  const dim3 grid(kDc / 128, kHeads);
  if (bf16)
    hipLaunchKernelGGL(absorb_q_bf16_kernel, grid, dim3(256), 0, stream, (const uint16_t*)q_nope,
                       (const uint16_t*)w_uk, (uint16_t*)q_lat, tokens);
  else
    hipLaunchKernelGGL(absorb_q_f32_kernel, grid, dim3(256), 0, stream, q_nope, w_uk, q_lat, tokens);
  return hipGetLastError();
}

hipError_t launch_merge_out_proj(const void* o_part, const float* lse_part, const void* w_uv, void* out,
                                 float* o_lat, float* lse, int rows, int num_splits, hipStream_t stream) {
  forget_stale_error();
  const int64_t grid = (int64_t)kHeads * ((rows + kMopRows - 1) / kMopRows);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(merge_out_proj_kernel, dim3((unsigned)grid), dim3(512), 0, stream, (const uint16_t*)o_part,
                     lse_part, (const uint16_t*)w_uv, (uint16_t*)out, o_lat, lse, rows, num_splits);
  return hipGetLastError();
}

hipError_t launch_out_proj(const float* o_lat, const void* w_uv, void* out, int tokens, bool bf16,
                           hipStream_t stream) {
  forget_stale_error();
  if (bf16)
    hipLaunchKernelGGL(out_proj_bf16_kernel, dim3(2 * kHeads), dim3(256), 0, stream, o_lat,
                       (const uint16_t*)w_uv, (uint16_t*)out, tokens);
  else
    hipLaunchKernelGGL(out_proj_f32_kernel, dim3(2, kHeads), dim3(256), 0, stream, o_lat, (const float*)w_uv,
                       (float*)out, tokens);
  return hipGetLastError();
}

}  // namespace mla
