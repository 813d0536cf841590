// The two per-head projections around the latent attention, gfx950.
//
//   absorb:   q_lat[n,h,c] = sum_d W_UK[h,c,d] q_nope[n,h,d]     (c < 512, d < 128)
//   out-proj: out[n,h,v]   = sum_c o_lat[n,h,c] W_UV[h,c,v]       (v < 128)
//
// W_UK is applied transposed to the query and W_UV after the latent average, so K and V are
// never formed: "DeepSeek-V2的推理成本如何计算？" (izhida.com), answer "专家"; "【笔记】MLA矩阵吸收分析"
// §二.2 step 2 and §三.2 step 2.  Both are batched GEMVs / thin GEMMs (M = tokens = B*S) whose
// cost is reading the 128 x 512 x 128 weight once (the same izhida answer notes that the main
// cost of the W_V product is reading W_V), so they are HBM-bound: every workgroup streams its
// weight slice exactly once and loops over the token blocks with it held in registers / LDS.
#include "common.h"
#include "kernels.h"

namespace mla {

// ---------------------------------------------------------------------------------------------
// absorb: grid (4 latent blocks of 128, 128 heads), 4 waves; wave w owns 32 latent rows
// c in [128 bx + 32 w, +32).  D(c x tokens) = W_UK[h] rows (A, straight from global) x q_nope^T (B).
template <bool BF16>
__global__ __launch_bounds__(256) void absorb_q_kernel(const void* __restrict__ q_nope,
                                                       const void* __restrict__ w_uk, void* __restrict__ q_lat,
                                                       int tokens) {
  const int h = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l32 = lane & 31, hf = lane >> 5;
  const int c_base = 128 * blockIdx.x + 32 * wave;
  const size_t wrow = ((size_t)h * kDc + c_base + l32) * kDh;
  if constexpr (BF16) {
    // A: lane holds W[c_base + l32][16 ks + 8 hf .. +7]
    bf16x8 aw[8];
    const bf16x8* W = (const bf16x8*)((const uint16_t*)w_uk + wrow + 8 * hf);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) aw[ks] = W[2 * ks];
    for (int nb = 0; nb * 32 < tokens; ++nb) {
      const int n = 32 * nb + l32;
      const bool ok = n < tokens;
      const bf16x8* Q = (const bf16x8*)((const uint16_t*)q_nope + ((size_t)(ok ? n : 0) * kHeads + h) * kDh + 8 * hf);
      f32x16 acc;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        bf16x8 bq = Q[2 * ks];
        if (!ok) bq = bf16x8{};
        acc = mfma32x32x16(aw[ks], bq, acc);
      }
      if (ok) {  // element e: latent c_base + (e/4)*8 + 4 hf + e%4 of token n
        uint16_t* dst = (uint16_t*)q_lat + ((size_t)n * kHeads + h) * kDc + c_base + 4 * hf;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          uint2 v = {pack_bf16x2(acc[4 * g], acc[4 * g + 1]), pack_bf16x2(acc[4 * g + 2], acc[4 * g + 3])};
          *(uint2*)(dst + 8 * g) = v;
        }
      }
    }
  } else {
    // fp32: k step (m, j) pairs lane half hf with d = 8 m + 4 hf + j (a float4 per m).
    f32x4 aw[16];
    const f32x4* W = (const f32x4*)((const float*)w_uk + wrow + 4 * hf);
#pragma unroll
    for (int m = 0; m < 16; ++m) aw[m] = W[2 * m];
    for (int nb = 0; nb * 32 < tokens; ++nb) {
      const int n = 32 * nb + l32;
      const bool ok = n < tokens;
      const f32x4* Q = (const f32x4*)((const float*)q_nope + ((size_t)(ok ? n : 0) * kHeads + h) * kDh + 4 * hf);
      f32x16 acc;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        f32x4 bq = Q[2 * m];
        if (!ok) bq = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = mfma32x32x2f32(aw[m][j], bq[j], acc);
      }
      if (ok) {
        float* dst = (float*)q_lat + ((size_t)n * kHeads + h) * kDc + c_base + 4 * hf;
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *(f32x4*)(dst + 8 * g) = f32x4{acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// out-proj: grid (2 value halves of 64, 128 heads), 4 waves.  The workgroup stages
// W_UV[h][:, 64 bx .. +64) (all 512 latent rows) in LDS once, then computes
// D(v x tokens) = W_UV^T (A, transposed LDS read) x o_lat^T (B, from global) for every
// (32-value block, 32-token block) pair, round-robin over the waves.  bf16: o_lat is split into
// hi + lo bf16 parts (two MFMAs) so the fp32 latent output loses no precision worth noting.
template <bool BF16>
__global__ __launch_bounds__(256) void out_proj_kernel(const float* __restrict__ o_lat,
                                                       const void* __restrict__ w_uv, void* __restrict__ out,
                                                       int tokens) {
  constexpr int kEl = BF16 ? 2 : 4;
  constexpr int kRowBytes = 64 * kEl;  // one latent row of the staged slice
  __shared__ __attribute__((aligned(16))) char wl_raw[kDc * kRowBytes];
  MLA_LDS char* wl = (MLA_LDS char*)wl_raw;
  const int h = blockIdx.y, vh = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l32 = lane & 31, hf = lane >> 5;

  {  // stage: row c of the slice is 64 values at W_UV[h][c][64 vh]
    const char* src = (const char*)w_uv + ((size_t)h * kDc * kDh + 64 * vh) * kEl;
    constexpr int kUnitsPerRow = kRowBytes / 16;
    for (int u = threadIdx.x; u < kDc * kUnitsPerRow; u += 256) {
      const int c = u / kUnitsPerRow, k = u % kUnitsPerRow;
      *(MLA_LDS u32x4*)(wl + c * kRowBytes + k * 16) = *(const u32x4*)(src + (size_t)c * kDh * kEl + k * 16);
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
    if constexpr (BF16) {
      // A lane l: value column 32 vb + l%32, latent rows 16 ks + 8 hf + j.  Transposed read:
      // source lane s of each 16-lane group supplies latent row (s/4) (+4 for the second read)
      // and value columns 4 (s%4) .. +3 of the group's 16-column half.
      const int r4 = (lane >> 2) & 3;
      const int col = 32 * vb + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll 4
      for (int ks = 0; ks < 32; ++ks) {
        const int c = 16 * ks + 8 * hf + r4;
        i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)(wl + c * kRowBytes + col * 2));
        i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)(wl + (c + 4) * kRowBytes + col * 2));
        i16x8 a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        const bf16x8 av = __builtin_bit_cast(bf16x8, a8);
        const f32x4 x0 = ok ? *(const f32x4*)(O + 16 * ks + 8 * hf) : f32x4{0.f, 0.f, 0.f, 0.f};
        const f32x4 x1 = ok ? *(const f32x4*)(O + 16 * ks + 8 * hf + 4) : f32x4{0.f, 0.f, 0.f, 0.f};
        const float x[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint16_t h0 = f32_to_bf16(x[2 * j]), h1 = f32_to_bf16(x[2 * j + 1]);
          hw[j] = uint32_t(h0) | (uint32_t(h1) << 16);
          lw[j] = pack_bf16x2(x[2 * j] - bf16_to_f32(h0), x[2 * j + 1] - bf16_to_f32(h1));
        }
        const u32x4 hv = {hw[0], hw[1], hw[2], hw[3]}, lv = {lw[0], lw[1], lw[2], lw[3]};
        acc = mfma32x32x16(av, __builtin_bit_cast(bf16x8, hv), acc);
        acc = mfma32x32x16(av, __builtin_bit_cast(bf16x8, lv), acc);
      }
    } else {
      // fp32: k step (m, j) pairs lane half hf with latent row c = 8 m + 4 hf + j.
      const MLA_LDS float* wf = (const MLA_LDS float*)wl;
#pragma unroll 2
      for (int m = 0; m < 64; ++m) {
        const f32x4 xb = ok ? *(const f32x4*)(O + 8 * m + 4 * hf) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = 8 * m + 4 * hf + j;
          acc = mfma32x32x2f32(wf[c * 64 + 32 * vb + l32], xb[j], acc);
        }
      }
    }
    if (ok) {  // element e: value 32 vb + (e/4)*8 + 4 hf + e%4 of token n
      const int v0 = 64 * vh + 32 * vb + 4 * hf;
      if constexpr (BF16) {
        uint16_t* dst = (uint16_t*)out + ((size_t)n * kHeads + h) * kDh + v0;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          uint2 v = {pack_bf16x2(acc[4 * g], acc[4 * g + 1]), pack_bf16x2(acc[4 * g + 2], acc[4 * g + 3])};
          *(uint2*)(dst + 8 * g) = v;
        }
      } else {
        float* dst = (float*)out + ((size_t)n * kHeads + h) * kDh + v0;
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *(f32x4*)(dst + 8 * g) = f32x4{acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
      }
    }
  }
}

hipError_t launch_absorb_q(const void* q_nope, const void* w_uk, void* q_lat, int tokens, bool bf16,
                           hipStream_t stream) {
  const dim3 grid(kDc / 128, kHeads);
  if (bf16)
    hipLaunchKernelGGL(absorb_q_kernel<true>, grid, dim3(256), 0, stream, q_nope, w_uk, q_lat, tokens);
  else
    hipLaunchKernelGGL(absorb_q_kernel<false>, grid, dim3(256), 0, stream, q_nope, w_uk, q_lat, tokens);
  return hipGetLastError();
}

hipError_t launch_out_proj(const float* o_lat, const void* w_uv, void* out, int tokens, bool bf16,
                           hipStream_t stream) {
  const dim3 grid(2, kHeads);
  if (bf16)
    hipLaunchKernelGGL(out_proj_kernel<true>, grid, dim3(256), 0, stream, o_lat, w_uv, out, tokens);
  else
    hipLaunchKernelGGL(out_proj_kernel<false>, grid, dim3(256), 0, stream, o_lat, w_uv, out, tokens);
  return hipGetLastError();
}

}  // namespace mla
