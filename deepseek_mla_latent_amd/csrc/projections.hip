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

// Up to this many tokens the fp32 projections run as VALU GEMVs instead of 32-token MFMA blocks.
constexpr int kGemvTokens = 4;
static_assert(kGemvMergeTokens == kGemvTokens, "the merging GEMV takes as many rows as the plain one");

// Forces the values to be complete here: every load producing them is issued before this point,
// and the compiler cannot trickle them out one MFMA at a time.
template <typename T>
__device__ __forceinline__ void settle(const T& x) {
  asm volatile("" ::"v"(x));
}

// Largest of lanes 0-15's values (every lane gets it): a running maximum over the first row of 16
// lanes by DPP row shifts, read from its last lane.
__device__ __forceinline__ int rows16_max(int v, int lane) {
  int t = __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  if ((lane & 15) >= 1) v = t > v ? t : v;
  t = __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  if ((lane & 15) >= 2) v = t > v ? t : v;
  t = __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  if ((lane & 15) >= 4) v = t > v ? t : v;
  t = __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  if ((lane & 15) >= 8) v = t > v ? t : v;
  return __builtin_amdgcn_readlane(v, 15);
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
// absorb, fp32, at most kGemvTokens tokens: one GEMV per (token, head) on the VALU.  A 32-token
// MFMA block would be almost all padding here (31/32 of the fp32 matrix work at one token), while
// the weight stream is the same.  Grid (4 latent blocks of 128, 128 heads), 4 waves; wave w owns
// rows c in [128 bx + 32 w, +32).  Load k brings rows c0 + 2k (lanes 0-31) and c0 + 2k + 1 (lanes
// 32-63), 1 KiB contiguous, and is kept in registers for every token; lane l32 holds d in
// [4 l32, +4).  A token's 16 per-lane partial dot products are summed over the 32 lanes of each
// half by recursive halving: at lane distance 16, 8, 4, 2 each lane keeps half of its rows and adds
// its partner's partial sums of them, and distance 1 adds the last pair.  Lane l32 then holds row
// c0 + 2 (l32 / 2) + hf.
__global__ __launch_bounds__(256) void absorb_q_f32_gemv_kernel(const float* __restrict__ q_nope,
                                                                const float* __restrict__ w_uk,
                                                                float* __restrict__ q_lat, int tokens) {
  const int h = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l32 = lane & 31, hf = lane >> 5;
  const int c0 = 128 * blockIdx.x + 32 * wave;
  const f32x4* W = (const f32x4*)(w_uk + ((size_t)h * kDc + c0 + hf) * kDh + 4 * l32);
  f32x4 wr[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) wr[k] = W[k * (2 * kDh / 4)];  // row c0 + 2k + hf
  for (int n = 0; n < tokens; ++n) {
    const f32x4 qv = *(const f32x4*)(q_nope + ((size_t)n * kHeads + h) * kDh + 4 * l32);
    float p[16];
#pragma unroll
    for (int k = 0; k < 16; ++k)
      p[k] = __builtin_fmaf(wr[k][3], qv[3], __builtin_fmaf(wr[k][2], qv[2], __builtin_fmaf(wr[k][1], qv[1], wr[k][0] * qv[0])));
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) {  // partner at lane distance 2m; rows j (lower lane) or j + m
      const bool upper = (l32 & (2 * m)) != 0;
#pragma unroll
      for (int j = 0; j < m; ++j) {
        const float give = upper ? p[j] : p[j + m];
        const float keep = upper ? p[j + m] : p[j];
        p[j] = keep + __shfl_xor(give, 2 * m);
      }
    }
    const float r = p[0] + __shfl_xor(p[0], 1);
    if ((l32 & 1) == 0) q_lat[((size_t)n * kHeads + h) * kDc + c0 + l32 + hf] = r;
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
// Workgroup = (head h, a run of 16-row blocks), 8 waves (two per SIMD); a head has two workgroups
// with consecutive logical ids (one XCD, so W_UV[h] comes from HBM once), and each stages its
// W_UV[h] slices once for all of its row blocks.  Wave w owns latent rows [64 w, +64), so each
// wave's first loads (2 batches of 4 splits' partials and lse, 16 W loads) stay within the 63 the
// vector-memory counter tracks and go out in one round trip:
//   * its 16 KiB slice of W_UV[h] goes to LDS (direct-to-LDS, 4 rows of 256 B per load);
//   * lane l merges row l % 16 of the block at latent 64 w + 32 ks + 8 (l / 16) + j (ks < 2,
//     j < 8): exactly the B operand of a 16x16x32 MFMA, so the merged values never leave the lane.
//     They are split into hi + lo bf16 (two MFMAs, about 16 mantissa bits of the fp32 merge kept);
//   * D(16 values x 16 rows) for the 8 value blocks over its 64 latent rows, A = W_UV^T by
//     transposed LDS reads; the next block's first partials load meanwhile;
//   * the eight waves' partial sums meet in four 8 KiB slots in LDS, beside the W slices.
// LDS row c of a wave's slice holds 32-byte block b (16 values) at block b ^ fsw(c) with
// fsw(c) = (c & 3) | ((c >> 3) & 1) << 2: a transposed read covers 16 rows x 32 B, which this puts
// on every bank pair exactly twice.
//
// FP8 (kFp8): W_UV as the E4M3 codes mla_quantize_w_uv_fp8 writes, stored transposed (H, 128 v,
// 512 c) with one scale per 128 x 128 block, and the merged rows coded on the fly with one scale
// per 128-long latent vector, the block quantisation of the Perplexity post (sections "Слой MLA"
// and "Квантование") that out_proj_fp8_kernel applies to o_lat:
//   * wave w's slice is bytes [64 w, +64) of each of the 128 value rows (8 KiB, 16 rows x 64 B per
//     load), 16-byte unit u of value row v stored at u ^ ((v >> 2) & 3);
//   * vector kb of a row spans the latent rows of waves 2 kb and 2 kb + 1: each wave's row maxima
//     reach its partner through LDS (one barrier), then every lane codes its 16 merged values, which
//     are again the B operand of a 16x16x32 (FP8) MFMA;
//   * A = W_UV^T codes, 8 bytes read straight from a value row (no transposed read); one MFMA per
//     (ks, value block), the wave's sums scaled by the row's activation scale times the weight
//     scale of block kb before the waves' sums meet.
constexpr int kMopRows = 16;
// Direct-to-LDS load of 16 bytes per lane (lane l's bytes at LDS lds + 16 l) from a wave-uniform
// base plus a per-lane byte offset, issued from asm: with the builtin the compiler waits for every
// outstanding vector-memory load before each later LDS read it cannot prove disjoint from the
// loaded bytes, which would also retire the next row block's partials loading in the background.
// The loads are awaited explicitly (before the first row block's products).
__device__ __forceinline__ void mop_dma16(const void* base, uint32_t voff, const MLA_LDS char* lds) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  const uint64_t sbase = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
               "s"(__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds))
               : "memory");
}
__device__ __forceinline__ int mop_swz(int c) { return (c & 3) | (((c >> 3) & 1) << 2); }
__device__ __forceinline__ int mop_swz8(int v) { return (v >> 2) & 3; }

constexpr float kE4M3MaxMop = 448.0f;  // largest finite E4M3 value: a vector's maximum codes to it

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <bool kFp8>
__global__ __launch_bounds__(512, 1) void merge_out_proj_kernel(const uint16_t* __restrict__ o_part,
                                                                const float* __restrict__ lse_part,
                                                                const int32_t* __restrict__ row_plan,
                                                                const void* __restrict__ w_uv,
                                                                const float* __restrict__ w_scales,
                                                                uint16_t* __restrict__ out, float* __restrict__ o_lat,
                                                                float* __restrict__ lse, int rows, int num_splits,
                                                                int blocks_per_wg) {
  constexpr int kSliceBytes = kFp8 ? 64 * kDh : 64 * kDh * 2;  // one wave's 64 latent rows of W_UV[h]
  __shared__ __attribute__((aligned(1024))) char wl_raw[8 * kSliceBytes];  // 64 / 128 KiB: the W_UV[h] slices
  __shared__ __attribute__((aligned(1024))) char red_raw[4 * 8 * 4 * 64 * 4];  // 32 KiB: four sum slots
  __shared__ float amax_x[kFp8 ? 8 * 16 : 1];  // FP8: each wave's row maxima over its 64 latent values
  MLA_LDS char* const wl = (MLA_LDS char*)wl_raw;
  MLA_LDS f32x4* const red = (MLA_LDS f32x4*)red_raw;  // slot s: [value block][lane], 4 elements each
  const int nblk = (rows + kMopRows - 1) / kMopRows;
  const int wph = (nblk + blocks_per_wg - 1) / blocks_per_wg;  // workgroups per head
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int h = id / wph, blk0 = (id % wph) * blocks_per_wg;
  const int blk_end = blk0 + blocks_per_wg < nblk ? blk0 + blocks_per_wg : nblk;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, g = lane >> 4, s16 = lane & 15;
  const int c0 = 64 * wave;
  MLA_LDS char* const ws = wl + wave * kSliceBytes;  // this wave's slice

  // merge: row n = 16 blk + s16 (a row past the end reads row 16 blk, which exists, and stores nothing)
  auto row_of = [&](int blk) { return 16 * blk + s16 < rows ? 16 * blk + s16 : 16 * blk; };
  // The slots of row n: (first, count) from the attention's plan (first + j holds its key range j);
  // word 0 of the plan says whether every row has the fixed slots n * num_splits + j.
  const bool plan_fixed = __builtin_amdgcn_readfirstlane(row_plan[0]) != 0;
  auto plan_of = [&](int blk) {
    return plan_fixed ? int2{row_of(blk) * num_splits, num_splits} : *(const int2*)(row_plan + 4 + 2 * row_of(blk));
  };
  // The first block's plan by scalar loads (a vector load here would be waited for together with the
  // W_UV loads): whether all 16 rows keep the fixed layout, this lane's entry, the most ranges.
  auto block_plan_scalar = [&](int blk, int2& mine, int& most) -> bool {
    int e0[16], e1[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {  // all 16 loads first: one wait
      const int n = 16 * blk + q < rows ? 16 * blk + q : 16 * blk;
      e0[q] = __builtin_amdgcn_readfirstlane(row_plan[4 + 2 * n]);
      e1[q] = __builtin_amdgcn_readfirstlane(row_plan[4 + 2 * n + 1]);
    }
    int off = 0;
    most = 0;
    mine = int2{e0[0], e1[0]};
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int n = 16 * blk + q < rows ? 16 * blk + q : 16 * blk;
      off |= (e0[q] ^ (n * num_splits)) | (e1[q] ^ num_splits);
      most = e1[q] > most ? e1[q] : most;
      if (s16 == q) mine = int2{e0[q], e1[q]};
    }
    return off == 0;
  };
  // Batches of 4 splits (a split past the row's count repeats its last one with weight 0), two in
  // flight.
  struct Batch {
    u32x4 x[4][2];  // [split][ks]
    float l[4];
  };
  auto load = [&](int2 pl, int kb, Batch& bt) {
    const size_t base = (size_t)pl.x * kHeads + h;  // split k at base + k * kHeads
    const float* lp = lse_part + base;
    const uint16_t* op = o_part + base * kDc + c0 + 8 * g;  // + 32 ks
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = kb + j < pl.y ? kb + j : pl.y - 1;
      bt.l[j] = kb + j < pl.y ? lp[(size_t)k * kHeads] : -INFINITY;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) bt.x[j][ks] = *(const u32x4*)(op + (size_t)k * kHeads * kDc + 32 * ks);
    }
  };
  // The first block's partials go out for the fixed layout (row * num_splits, num_splits) before its
  // plan is read; they are issued again below in the rare case that the plan differs (a ragged batch).
  const int2 pl_fixed = {row_of(blk0) * num_splits, num_splits};
  Batch b0, b1;
  load(pl_fixed, 0, b0);
  if (4 < num_splits) load(pl_fixed, 4, b1);
  // W_UV[h] rows [c0, c0 + 64) after the first partials, so waiting for those does not wait for
  // W: load i covers local rows 4 i .. 4 i + 3 (16 lanes each).  Staged once for every row block of
  // the workgroup.
  if constexpr (kFp8) {  // load i: value rows 16 i .. 16 i + 15 (lane l: row 16 i + l / 4, LDS unit l % 4)
    const uint8_t* src = (const uint8_t*)w_uv + (size_t)h * kDh * kDc + c0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int v = 16 * i + (lane >> 2);
      const int u = (lane & 3) ^ mop_swz8(v);
      mop_dma16(src, (uint32_t)(v * kDc + u * 16), ws + i * 1024);
    }
  } else {
    const char* src = (const char*)((const uint16_t*)w_uv + ((size_t)h * kDc + c0) * kDh);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int c = 4 * i + g, u = s16;
      const int us = 2 * ((u >> 1) ^ mop_swz(c)) + (u & 1);
      mop_dma16(src, (uint32_t)(c * kDh * 2 + us * 16), ws + i * 1024);
    }
  }
  // the plan of the first block; the most ranges of its 16 rows bounds the merge loop
  int2 pl = pl_fixed;
  int nsp = num_splits;
  if (!plan_fixed && !block_plan_scalar(blk0, pl, nsp)) {
    load(pl, 0, b0);
    if (4 < nsp) load(pl, 4, b1);
  }
  int2 pl_next = blk0 + 1 < blk_end ? plan_of(blk0 + 1) : pl;
  const float sw = kFp8 ? w_scales[h * 4 + (wave >> 1)] : 1.f;  // FP8: weight scale of block kb = w / 2
  // A operand of value block mb, k step ks: two transposed reads; source lane s of group g gives
  // local row 32 ks + 8 g + 4 t + s/4 and values 16 mb + 4 (s%4) .. +3 (t = 0, 1).
  const int fsw = (s16 >> 2) | ((g & 1) << 2);  // mop_swz of every row this lane addresses
  const MLA_LDS char* a_row = ws + (8 * g + (s16 >> 2)) * (kDh * 2) + (s16 & 3) * 8;
  constexpr float kLog2e = 1.4426950408889634f;

  for (int blk = blk0; blk < blk_end; ++blk) {
    const int n = row_of(blk);
    const bool live = 16 * blk + s16 < rows;
    // Running log-sum-exp merge: weights are taken against the largest lse seen so far, and the
    // sums are rescaled when a batch raises it (an empty split has lse = -inf and weight 0).
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
    for (int kb = 0; kb < nsp; kb += 8) {
      consume(b0);
      if (kb + 8 < nsp) load(pl, kb + 8, b0);
      if (kb + 4 < nsp) {
        consume(b1);
        if (kb + 12 < nsp) load(pl, kb + 12, b1);
      }
    }
    const float inv = sum > 0.f ? 1.0f / sum : 0.f;
    float ov[2][8];  // the merged row: latent 64 w + 32 ks + 8 g + j
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const f32x4 a = acc_o[2 * ks] * inv, b = acc_o[2 * ks + 1] * inv;
      if (o_lat && live) {
        f32x4* dst = (f32x4*)(o_lat + ((size_t)n * kHeads + h) * kDc + c0 + 32 * ks + 8 * g);
        dst[0] = a;
        dst[1] = b;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) ov[ks][j] = a[j], ov[ks][4 + j] = b[j];
    }
    bf16x8 bh[2], bl[2];  // bf16: hi + lo parts
    uint32_t bc[2][2];    // FP8: codes (8 per ks)
    float s_row = 1.f;    // FP8: activation scale of this lane's row times the weight scale
    if constexpr (kFp8) {
      float m8 = 0.f;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int j = 0; j < 8; ++j) m8 = fmaxf(m8, fabsf(ov[ks][j]));
      m8 = fmaxf(m8, __shfl_xor(m8, 16));
      m8 = fmaxf(m8, __shfl_xor(m8, 32));
      if (g == 0) amax_x[wave * 16 + s16] = m8;
      __syncthreads();
      const float amax = fmaxf(m8, amax_x[(wave ^ 1) * 16 + s16]);
      const float f = amax > 0.f ? kE4M3MaxMop / amax : 0.f;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          int word = __builtin_amdgcn_cvt_pk_fp8_f32(ov[ks][4 * i] * f, ov[ks][4 * i + 1] * f, 0, false);
          word = __builtin_amdgcn_cvt_pk_fp8_f32(ov[ks][4 * i + 2] * f, ov[ks][4 * i + 3] * f, word, true);
          bc[ks][i] = f > 0.f ? (uint32_t)word : 0u;
        }
      s_row = (amax / kE4M3MaxMop) * sw;
    } else {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32x4 hw, lw;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          hw[j] = pack_bf16x2(ov[ks][2 * j], ov[ks][2 * j + 1]);
          const float d0 = ov[ks][2 * j] - __uint_as_float(hw[j] << 16);
          const float d1 = ov[ks][2 * j + 1] - __uint_as_float(hw[j] & 0xffff0000u);
          lw[j] = pack_bf16x2(d0, d1);
        }
        bh[ks] = __builtin_bit_cast(bf16x8, hw);
        bl[ks] = __builtin_bit_cast(bf16x8, lw);
      }
    }
    if (lse && live && wave == 0 && g == 0) lse[(size_t)n * kHeads + h] = m == -INFINITY ? -INFINITY : m + logf(sum);

    if (blk == blk0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's W rows have landed
    // the next row block's first partials stream in during this block's products and sums (its plan
    // was loaded a block ahead)
    if (blk + 1 < blk_end) {
      pl = pl_next;
      nsp = plan_fixed ? num_splits : rows16_max(pl.y, lane);
      load(pl, 0, b0);
      if (4 < nsp) load(pl, 4, b1);
      // from the table, unconditionally (past the end: the last block's entry again, unused), so
      // that nothing uses the loaded entry before the next row block
      pl_next = *(const int2*)(row_plan + 4 + 2 * row_of(blk + 2 < blk_end ? blk + 2 : blk_end - 1));
    }
    f32x4 acc[8];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (kFp8) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const long b = (long)(((uint64_t)bc[ks][1] << 32) | bc[ks][0]);
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) {  // A: value row 16 mb + s16, latent bytes 32 ks + 8 g .. +7
          const int v = 16 * mb + s16, u = 2 * ks + (g >> 1);
          const long a = *(const MLA_LDS long*)(ws + v * 64 + ((u ^ mop_swz8(v)) * 16) + (g & 1) * 8);
          acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, acc[mb], 0, 0, 0);
        }
      }
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) acc[mb] *= s_row;
    } else {
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
    }

    // The eight waves' partial sums (over their latent rows) meet in the four sum slots: waves 4-7
    // put theirs in slots 0-3, waves 0-3 add them and put the pair sums back, then wave w adds value
    // block w over the four slots.  Element i of lane l is value 16 mb + 4 g + i of row s16.
    auto slot = [&](int sl, int mb) -> MLA_LDS f32x4& { return red[(sl * 8 + mb) * 64 + lane]; };
    if (wave >= 4) {
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) slot(wave - 4, mb) = acc[mb];
    }
    __syncthreads();
    if (wave < 4) {
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) slot(wave, mb) = acc[mb] + slot(wave, mb);
    }
    __syncthreads();
    {
      const int mb = wave;
      const f32x4 sv = (slot(0, mb) + slot(1, mb)) + (slot(2, mb) + slot(3, mb));
      if (live) {
        const u32x2 pk = {pack_bf16x2(sv[0], sv[1]), pack_bf16x2(sv[2], sv[3])};
        *(u32x2*)(out + ((size_t)n * kHeads + h) * kDh + 16 * mb + 4 * g) = pk;
      }
    }
    __syncthreads();  // the slots are free for the next row block
  }
}

// out-proj, fp32, at most kGemvTokens tokens: one GEMV per (token, head) on the VALU (a 32-token
// MFMA block would be almost all padding).  Grid (2 value halves of 64, 128 heads), 4 waves; wave
// w owns latent rows [128 w, +128), and lane group r4 = lane / 16 the 32 rows 128 w + 32 r4 + i,
// whose 64 values of this half (256 B each, lane l16 holding values 4 l16 .. +3) stay in registers
// for every token.  Per token a lane adds up its 32 rows weighted by o_lat (read once per lane
// group); the four lane groups are summed by shuffles and the four waves through LDS, in a fixed
// order.
__global__ __launch_bounds__(256) void out_proj_f32_gemv_kernel(const float* __restrict__ o_lat,
                                                                const float* __restrict__ w_uv,
                                                                float* __restrict__ out, int tokens) {
  __shared__ f32x4 part[4 * kGemvTokens * 16];  // [wave][token][l16]
  const int h = blockIdx.y, vh = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l16 = lane & 15, r4 = lane >> 4;
  const int c0 = 128 * wave + 32 * r4;
  const f32x4* W = (const f32x4*)(w_uv + ((size_t)h * kDc + c0) * kDh + 64 * vh + 4 * l16);
  f32x4 wr[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) wr[i] = W[i * (kDh / 4)];  // row c0 + i
  for (int n = 0; n < tokens; ++n) {
    const f32x4* O = (const f32x4*)(o_lat + ((size_t)n * kHeads + h) * kDc + c0);
    f32x4 ov[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) ov[i] = O[i];
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float o = ov[i >> 2][i & 3];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(o, wr[i][e], acc[e]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[e] += __shfl_xor(acc[e], 16);
      acc[e] += __shfl_xor(acc[e], 32);
    }
    if (r4 == 0) part[(wave * kGemvTokens + n) * 16 + l16] = acc;
  }
  __syncthreads();
  const int n = lane >> 4;  // wave 0: lane 16 n + l16 sums token n's values 4 l16 .. +3
  if (wave == 0 && n < tokens) {
    f32x4 v = part[n * 16 + l16];
#pragma unroll
    for (int w = 1; w < 4; ++w) v += part[(w * kGemvTokens + n) * 16 + l16];
    *(f32x4*)(out + ((size_t)n * kHeads + h) * kDh + 64 * vh + 4 * l16) = v;
  }
}

// Split merge + out-proj, fp32, at most kGemvTokens query rows: out_proj_f32_gemv_kernel's grid,
// waves and dot products, with o_lat formed in the kernel from the attention's fp32 split partials
// instead of read from memory (the separate lse_merge_kernel launch is saved; at one query row it
// is much of a step's fixed cost).  Row n's ranges are slots first .. first + count - 1 of the row
// table (first = n * num_splits, count = num_splits when word 0 says every row keeps those).
// The merge comes first and uses all 256 threads: thread t takes latent columns 2t, 2t + 1 of
// head h and loads them from eight splits at a time together with their lse values, so the
// partials of a row arrive in one round trip beside the W_UV rows; o = sum_k w_k o_k / sum_k w_k,
// w_k = e^(lse_k - max_k lse_k) (all splits empty: o = 0, lse = -inf), the merge of
// "【笔记】MLA矩阵吸收分析" §三.2 step 1 over key ranges, with the maximum taken per batch of eight.  The merged
// rows go to LDS for the dot products; the workgroups of value half 0 also write o_lat and lse
// when asked for.
__global__ __launch_bounds__(256) void merge_out_proj_f32_gemv_kernel(const float* __restrict__ o_part,
                                                                      const float* __restrict__ lse_part,
                                                                      const int32_t* __restrict__ row_plan,
                                                                      const float* __restrict__ w_uv,
                                                                      float* __restrict__ out, float* __restrict__ o_lat,
                                                                      float* __restrict__ lse, int tokens,
                                                                      int num_splits) {
  __shared__ f32x4 part[4 * kGemvTokens * 16];              // [wave][token][l16]
  __shared__ __attribute__((aligned(16))) float om[kGemvTokens * kDc];  // merged rows
  const int h = blockIdx.y, vh = blockIdx.x;
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63, l16 = lane & 15, r4 = lane >> 4;
  const int c0 = 128 * wave + 32 * r4;
  const f32x4* W = (const f32x4*)(w_uv + ((size_t)h * kDc + c0) * kDh + 64 * vh + 4 * l16);
  f32x4 wr[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) wr[i] = W[i * (kDh / 4)];  // row c0 + i
  const bool fixed = __builtin_amdgcn_readfirstlane(row_plan[0]) != 0;
  constexpr float kLog2e = 1.4426950408889634f;
  for (int n = 0; n < tokens; ++n) {
    const int first = fixed ? n * num_splits : __builtin_amdgcn_readfirstlane(row_plan[4 + 2 * n]);
    const int cnt = fixed ? num_splits : __builtin_amdgcn_readfirstlane(row_plan[4 + 2 * n + 1]);
    const float* lp = lse_part + (size_t)first * kHeads + h;  // split k at lp[k * kHeads]
    const float* op = o_part + ((size_t)first * kHeads + h) * kDc + 2 * t;  // split k at op[k * kHeads * kDc]
    // eight splits' lse values and partials in flight at once; the running maximum is raised per
    // batch (the sums rescaled with it), so a row's loads need no round trip before them
    float m = -INFINITY, a0 = 0.f, a1 = 0.f, sum = 0.f;
    for (int kb = 0; kb < cnt; kb += 8) {
      float l[8];
      float2 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int k = kb + j < cnt ? kb + j : cnt - 1;
        l[j] = lp[(size_t)k * kHeads];
        v[j] = *(const float2*)(op + (size_t)k * kHeads * kDc);
      }
      float mb = m;
#pragma unroll
      for (int j = 0; j < 8; ++j) mb = kb + j < cnt ? fmaxf(mb, l[j]) : mb;
      const float sc = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m - mb) * kLog2e);
      a0 *= sc;
      a1 *= sc;
      sum *= sc;
      m = mb;
      const float m_ref = m == -INFINITY ? 0.f : m;  // all splits so far empty: every weight is 0
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float w = kb + j < cnt ? __builtin_amdgcn_exp2f((l[j] - m_ref) * kLog2e) : 0.f;
        sum += w;
        a0 = __builtin_fmaf(w, v[j].x, a0);
        a1 = __builtin_fmaf(w, v[j].y, a1);
      }
    }
    const float inv = sum > 0.f ? 1.0f / sum : 0.f;
    const float2 o2 = {a0 * inv, a1 * inv};
    *(float2*)(om + n * kDc + 2 * t) = o2;
    if (vh == 0) {
      if (o_lat) *(float2*)(o_lat + ((size_t)n * kHeads + h) * kDc + 2 * t) = o2;
      if (lse && t == 0) lse[(size_t)n * kHeads + h] = m == -INFINITY ? -INFINITY : m + logf(sum);
    }
  }
  __syncthreads();  // the merged rows are in LDS
  for (int n = 0; n < tokens; ++n) {
    const f32x4* O = (const f32x4*)(om + n * kDc + c0);
    f32x4 ov[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) ov[i] = O[i];
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float o = ov[i >> 2][i & 3];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(o, wr[i][e], acc[e]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[e] += __shfl_xor(acc[e], 16);
      acc[e] += __shfl_xor(acc[e], 32);
    }
    if (r4 == 0) part[(wave * kGemvTokens + n) * 16 + l16] = acc;
  }
  __syncthreads();
  const int n = lane >> 4;  // wave 0: lane 16 n + l16 sums token n's values 4 l16 .. +3
  if (wave == 0 && n < tokens) {
    f32x4 v = part[n * 16 + l16];
#pragma unroll
    for (int w = 1; w < 4; ++w) v += part[(w * kGemvTokens + n) * 16 + l16];
    *(f32x4*)(out + ((size_t)n * kHeads + h) * kDh + 64 * vh + 4 * l16) = v;
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
  if (ntb == 1) {
    // One token block: two (value block) items for four waves, so each item is split over two
    // waves by latent half (rows [256 kh, +256)); the halves' sums meet in LDS, added in order.
    __shared__ f32x4 half_sums[2 * 4 * 64];  // [value block][element group][lane] of latent half 1
    const int vb = wave & 1, kh = wave >> 1;
    const int n = l32;
    const bool ok = n < tokens;
    const float* O = o_lat + ((size_t)(ok ? n : 0) * kHeads + h) * kDc;
    f32x16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
    for (int m0 = 32 * kh; m0 < 32 * kh + 32; m0 += 16) {
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
    if (kh == 1) {
#pragma unroll
      for (int g = 0; g < 4; ++g)
        half_sums[(vb * 4 + g) * 64 + lane] = f32x4{acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
    }
    __syncthreads();
    if (kh == 0 && ok) {  // element e: value 32 vb + (e/4)*8 + 4 hf + e%4 of token n
      float* dst = out + ((size_t)n * kHeads + h) * kDh + 64 * vh + 32 * vb + 4 * hf;
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(f32x4*)(dst + 8 * g) =
            f32x4{acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]} + half_sums[(vb * 4 + g) * 64 + lane];
    }
    return;
  }
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
  else if (tokens <= kGemvTokens)
    hipLaunchKernelGGL(absorb_q_f32_gemv_kernel, grid, dim3(256), 0, stream, (const float*)q_nope,
                       (const float*)w_uk, (float*)q_lat, tokens);
  else
    hipLaunchKernelGGL(absorb_q_f32_kernel, grid, dim3(256), 0, stream, q_nope, w_uk, q_lat, tokens);
  return hipGetLastError();
}

hipError_t launch_merge_out_proj(const void* o_part, const float* lse_part, const int32_t* row_plan, const void* w_uv,
                                 bool w_fp8, void* out, float* o_lat, float* lse, int rows, int num_splits,
                                 int slots, hipStream_t stream) {
  (void)slots;  // the merge reads each row's slots from row_plan
  forget_stale_error();
  // two workgroups per head (one per CU at 128 heads), each over a run of 16-row blocks, so a
  // workgroup stages its W_UV[h] slices once for all of its rows
  const int nblk = (rows + kMopRows - 1) / kMopRows;
  const int wph = nblk < 2 ? nblk : 2;
  if (wph == 0) return hipSuccess;
  const int bpw = (nblk + wph - 1) / wph;
  const int64_t grid = (int64_t)kHeads * ((nblk + bpw - 1) / bpw);
  if (w_fp8) {
    const float* scales = (const float*)((const uint8_t*)w_uv + (size_t)kHeads * kDc * kDh);
    hipLaunchKernelGGL(merge_out_proj_kernel<true>, dim3((unsigned)grid), dim3(512), 0, stream,
                       (const uint16_t*)o_part, lse_part, row_plan, w_uv, scales, (uint16_t*)out, o_lat, lse, rows, num_splits,
                       bpw);
  } else {
    hipLaunchKernelGGL(merge_out_proj_kernel<false>, dim3((unsigned)grid), dim3(512), 0, stream,
                       (const uint16_t*)o_part, lse_part, row_plan, w_uv, (const float*)nullptr, (uint16_t*)out, o_lat, lse,
                       rows, num_splits, bpw);
  }
  return hipGetLastError();
}

hipError_t launch_merge_out_proj_f32(const float* o_part, const float* lse_part, const int32_t* row_plan,
                                     const float* w_uv, float* out, float* o_lat, float* lse, int tokens, int num_splits,
                                     int slots, hipStream_t stream) {
  (void)slots;  // the merge reads each row's slots from row_plan
  forget_stale_error();
  if (tokens <= 0) return hipSuccess;
  if (tokens > kGemvTokens) return hipErrorInvalidValue;
  hipLaunchKernelGGL(merge_out_proj_f32_gemv_kernel, dim3(2, kHeads), dim3(256), 0, stream, o_part, lse_part, row_plan,
                     w_uv, out, o_lat, lse, tokens, num_splits);
  return hipGetLastError();
}

hipError_t launch_out_proj(const float* o_lat, const void* w_uv, void* out, int tokens, bool bf16,
                           hipStream_t stream) {
  forget_stale_error();
  if (bf16)
    hipLaunchKernelGGL(out_proj_bf16_kernel, dim3(2 * kHeads), dim3(256), 0, stream, o_lat,
                       (const uint16_t*)w_uv, (uint16_t*)out, tokens);
  else if (tokens <= kGemvTokens)
    hipLaunchKernelGGL(out_proj_f32_gemv_kernel, dim3(2, kHeads), dim3(256), 0, stream, o_lat, (const float*)w_uv,
                       (float*)out, tokens);
  else
    hipLaunchKernelGGL(out_proj_f32_kernel, dim3(2, kHeads), dim3(256), 0, stream, o_lat, (const float*)w_uv,
                       (float*)out, tokens);
  return hipGetLastError();
}

}  // namespace mla
