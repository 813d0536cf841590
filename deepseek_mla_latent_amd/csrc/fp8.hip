// FP8 block-quantised per-head products (k_b_proj / v_b_proj), gfx950.
//
// The Perplexity post ("Lower latency and higher throughput with multi-node DeepSeek deployment")
// runs the W_UK and W_UV products as an FP8 block-quantised batched matmul (section "Слой MLA") with
// the scheme of section "Квантование": weights quantised statically, one scale per 128 x 128 block;
// activations quantised on the fly, one scale per 128-element vector along the reduction
// dimension.  Format E4M3 (bias 7, 3 mantissa bits, no infinities, largest finite 448); a block's
// scale is amax / 448 in fp32; a value is coded as x * (448 / amax) (one fp32 division per block,
// fp32 products) rounded to the nearest E4M3 value, ties to even, by the hardware conversion.
//
//   quantize_weight_fp8_kernel  W (H, 512, 128) bf16 -> codes + scales (H, 4); W_UV's codes are
//                               stored transposed, (H, 128 v, 512 c), so both products read
//                               8 consecutive k per lane from one row.
//   absorb_q_fp8_kernel         q_lat = W_UK q_nope per head: K = 128 (one block per token/head)
//   out_proj_fp8_kernel         out = W_UV^T o_lat per head: K = 512 (four blocks per token/head)
// One workgroup (8 waves) per head.  Per block of 32 tokens the workgroup first codes the
// activations once, cooperatively, into LDS (codes + per-vector scales); then each wave runs its
// 32x32x16 FP8 MFMAs with fp32 accumulation, the weight codes (loaded once per workgroup) as the
// A operand and the activation codes from LDS as the B operand; results go out through an LDS
// tile as whole rows.  Each block's sum is scaled by its activation
// scale (per token: a lane holds one token) times its weight scale.  Lane halves split each
// 128-long k block: half hf holds k in [64 hf, 64 hf + 64), 8 per MFMA step, the same order for
// the A and B operands.
#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

constexpr float kE4M3Max = 448.0f;

// N values -> N codes (N/4 words, 4 codes per word, little-endian) of x * factor.  The conversion
// is the hardware's (v_cvt_pk_fp8_f32: OCP E4M3, round to nearest even, subnormals kept), two
// values per instruction.  |x * factor| <= 448 (1 + 2^-23) by construction, which rounds to at
// most 448, so no value reaches the overflow encoding.  An all-zero block (factor 0) has codes 0
// (a -0.0 input would otherwise give the code of -0).
template <int N>
__device__ __forceinline__ void code_n(const float (&x)[N], float factor, uint32_t (&w)[N / 4]) {
#pragma unroll
  for (int i = 0; i < N / 4; ++i) {
    int word = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * i] * factor, x[4 * i + 1] * factor, 0, false);
    word = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * i + 2] * factor, x[4 * i + 3] * factor, word, true);
    w[i] = factor > 0.f ? (uint32_t)word : 0u;
  }
}
__device__ __forceinline__ float code_factor(float amax) { return amax > 0.f ? kE4M3Max / amax : 0.f; }

__device__ __forceinline__ f32x16 mfma_fp8(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, const f32x16& c) {
  const long a = (long)(((uint64_t)a1 << 32) | a0), b = (long)(((uint64_t)b1 << 32) | b0);
  return __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(a, b, c, 0, 0, 0);
}

}  // namespace

// ------------------------------------------------------------------------------------------------
// One workgroup (256 threads) per (head, 128-row block of the 512 latent rows): thread t holds
// row r = t / 2, columns 64 (t % 2) .. +63 of the block.  amax over the block, then codes.
__global__ __launch_bounds__(256) void quantize_weight_fp8_kernel(const uint16_t* __restrict__ w,
                                                                  uint8_t* __restrict__ codes,
                                                                  float* __restrict__ scales, int transpose) {
  __shared__ float red[4];
  __shared__ __attribute__((aligned(16))) uint8_t tile[128 * 128];
  const int h = blockIdx.y, cb = blockIdx.x, t = threadIdx.x;
  const int r = t >> 1, c0 = 64 * (t & 1);
  const uint16_t* src = w + ((size_t)h * kDc + cb * 128 + r) * kDh + c0;
  float x[64];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const u32x4 v = *(const u32x4*)(src + u * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[8 * u + 2 * j] = __uint_as_float(v[j] << 16);
      x[8 * u + 2 * j + 1] = __uint_as_float(v[j] & 0xffff0000u);
    }
  }
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 64; ++i) m = fmaxf(m, fabsf(x[i]));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((t & 63) == 0) red[t >> 6] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float scale = amax / kE4M3Max;
  uint32_t wd[16];
  code_n<64>(x, code_factor(amax), wd);
  if (t == 0) scales[h * 4 + cb] = scale;
  if (!transpose) {  // codes (H, 512, 128), row-major like W
    uint8_t* dst = codes + ((size_t)h * kDc + cb * 128 + r) * kDh + c0;
#pragma unroll
    for (int u = 0; u < 4; ++u) *(u32x4*)(dst + 16 * u) = u32x4{wd[4 * u], wd[4 * u + 1], wd[4 * u + 2], wd[4 * u + 3]};
    return;
  }
  // transposed: codes (H, 128, 512): row v, columns c; through LDS
#pragma unroll
  for (int u = 0; u < 16; ++u) *(uint32_t*)(tile + r * 128 + c0 + 4 * u) = wd[u];
  __syncthreads();
  const int v = t >> 1, k0 = 64 * (t & 1);  // this thread writes row v, latent rows k0 .. +63 of the block
  uint32_t out[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) word |= (uint32_t)tile[(k0 + 4 * i + j) * 128 + v] << (8 * j);
    out[i] = word;
  }
  uint8_t* dst = codes + ((size_t)h * kDh + v) * kDc + cb * 128 + k0;
#pragma unroll
  for (int u = 0; u < 4; ++u) *(u32x4*)(dst + 16 * u) = u32x4{out[4 * u], out[4 * u + 1], out[4 * u + 2], out[4 * u + 3]};
}

// ------------------------------------------------------------------------------------------------
// Activation coding into LDS.  A block of 32 tokens, V vectors of 128 per token: groups of P
// consecutive values, 128 / P groups per vector; thread tid takes groups tid, tid + NT, ...
// (NT = workgroup size).  A vector's groups sit in consecutive lanes, so its amax is a few lane
// shuffles.  All of a thread's loads are issued before any coding.  Codes row j holds token j's
// vectors back to back; 16-byte unit u of a 128-byte vector of row j sits at u ^ (j & 7), so the
// 16 tokens a B-operand read spans hit distinct units.  Rows past `tokens` code the last token.
template <int V>  // vectors (of 128) per token
struct ActCodes {
  uint8_t codes[32 * V * 128];
  float scale[32 * V];
};

__device__ __forceinline__ int act_off(int j, int vec, int V, int byte) {  // byte within the 128-byte vector
  return (j * V + vec) * 128 + ((((byte >> 4) ^ (j & 7))) << 4) + (byte & 15);
}

template <int V, int P, int NT, bool BF16>
__device__ __forceinline__ void code_tokens(const void* src, size_t token_stride, int n0, int tokens, int tid,
                                            ActCodes<V>& st) {
  constexpr int kParts = 128 / P, kPasses = 32 * V * kParts / NT;
  static_assert(kPasses * NT == 32 * V * kParts, "whole passes");
  float x[kPasses][P];
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int g = pass * NT + tid, vecid = g / kParts, part = g % kParts;
    const int j = vecid / V, vec = vecid % V;
    const int n = min(n0 + j, tokens - 1);
    if (BF16) {
      const uint16_t* p = (const uint16_t*)src + n * token_stride + vec * 128 + part * P;
#pragma unroll
      for (int u = 0; u < P / 8; ++u) {
        const u32x4 a = *(const u32x4*)(p + 8 * u);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          x[pass][8 * u + 2 * k] = __uint_as_float(a[k] << 16);
          x[pass][8 * u + 2 * k + 1] = __uint_as_float(a[k] & 0xffff0000u);
        }
      }
    } else {
      const float* p = (const float*)src + n * token_stride + vec * 128 + part * P;
#pragma unroll
      for (int u = 0; u < P / 4; ++u) {
        const f32x4 q = *(const f32x4*)(p + 4 * u);
        x[pass][4 * u] = q[0], x[pass][4 * u + 1] = q[1], x[pass][4 * u + 2] = q[2], x[pass][4 * u + 3] = q[3];
      }
    }
  }
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int g = pass * NT + tid, vecid = g / kParts, part = g % kParts;
    const int j = vecid / V, vec = vecid % V;
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < P; ++i) m = fmaxf(m, fabsf(x[pass][i]));
#pragma unroll
    for (int off = 1; off < kParts; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
    uint32_t w[P / 4];
    code_n<P>(x[pass], code_factor(m), w);
    if (P == 16)
      *(u32x4*)&st.codes[act_off(j, vec, V, part * P)] = u32x4{w[0], w[1], w[2], w[3]};
    else
      *(u32x2*)&st.codes[act_off(j, vec, V, part * P)] = u32x2{w[0], w[1]};
    if (part == 0) st.scale[vecid] = m / kE4M3Max;
  }
}

// B operand of k-step ks (vector vec) for this lane's token l32 and k half hf: 8 bytes
__device__ __forceinline__ uint64_t act_b(const uint8_t* codes, int l32, int hf, int vec, int V, int ks) {
  return *(const uint64_t*)&codes[act_off(l32, vec, V, 64 * hf + 8 * ks)];
}

// 8 bytes of output for token row `row` at byte `byte` of a staged tile of 16-byte units with
// `units` units per row; unit u of row r sits at u ^ (r % units), so the 32 rows one
// MFMA-fragment store spans hit distinct units.
__device__ __forceinline__ int out_off(int row, int byte, int units) {
  return row * units * 16 + ((((byte >> 4) ^ (row & (units - 1)))) << 4) + (byte & 15);
}

// fragment (32 x 32 D, this lane's column = token l32) -> bf16 into the staged tile at rows' byte
// offset `byte0` (+ 16 g + 8 hf per 4-row group g), times `s`
__device__ __forceinline__ void stage_fragment(uint8_t* tile, int units, int l32, int hf, int byte0,
                                               const f32x16& acc, float s) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    u32x2 v;
    v[0] = pack_bf16x2(acc[4 * g] * s, acc[4 * g + 1] * s);
    v[1] = pack_bf16x2(acc[4 * g + 2] * s, acc[4 * g + 3] * s);
    *(u32x2*)&tile[out_off(l32, byte0 + 16 * g + 8 * hf, units)] = v;
  }
}

// staged tile (32 token rows of `units` 16-byte units) -> global rows dst + n * stride (bytes)
template <int NT>
__device__ __forceinline__ void store_tile(const uint8_t* tile, int units, uint8_t* dst, size_t stride, int n0,
                                           int tokens, int tid) {
#pragma unroll
  for (int k = tid; k < 32 * units; k += NT) {
    const int row = k / units, u = k % units;
    if (n0 + row < tokens)
      *(u32x4*)(dst + (size_t)(n0 + row) * stride + 16 * u) = *(const u32x4*)&tile[out_off(row, 16 * u, units)];
  }
}

// absorb: grid (4 latent blocks of 128 rows, 128 heads), 4 waves: a workgroup's rows are exactly
// one 128 x 128 weight block (one weight scale), and 512 workgroups keep every compute unit
// streaming (8 KiB of codes per head and block half: 16 KiB per workgroup).  Wave w owns latent
// rows cb + 32 w + l32.  Its 32 code rows (128 B each) reach LDS by four 1 KiB direct-to-LDS
// loads, whole cache lines, with 16-byte unit u of row r stored at u ^ (r & 7); the A operand of
// step ks is 8 bytes of that row.  Per block of 32 tokens the workgroup codes q_nope[., h, :] once
// into LDS (one scale per token: K = 128 is one block), each wave runs 8 FP8 MFMAs, and the bf16
// results leave through an LDS tile as whole 256-byte rows.
__global__ __launch_bounds__(256) void absorb_q_fp8_kernel(const uint16_t* __restrict__ q_nope,
                                                           const uint8_t* __restrict__ codes,
                                                           const float* __restrict__ scales,
                                                           uint16_t* __restrict__ q_lat, int tokens) {
  __shared__ __attribute__((aligned(1024))) uint8_t w_lds[128 * 128];
  __shared__ __attribute__((aligned(16))) ActCodes<1> st;
  __shared__ __attribute__((aligned(16))) uint8_t tile[32 * 256];
  const int h = blockIdx.y, cb = blockIdx.x, tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  {  // load i: rows 8 i .. 8 i + 7 of the wave's 32 (lane l: row 8 i + l / 8, LDS unit l % 8)
    const uint8_t* src = codes + ((size_t)h * kDc + 128 * cb + 32 * wave) * kDh;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 8 * i + (lane >> 3);
      const int u = (lane & 7) ^ (r & 7);
      __builtin_amdgcn_global_load_lds((const MLA_GLOBAL void*)(src + r * 128 + u * 16),
                                       (MLA_LDS void*)(w_lds + (32 * wave + 8 * i) * 128), 16, 0, 0);
    }
  }
  const float sw = scales[h * 4 + cb];
  const int r = 32 * wave + l32;  // this lane's code row (A operand row)
  for (int n0 = 0; n0 < tokens; n0 += 32) {
    __syncthreads();  // the previous block's codes and staged rows are consumed
    code_tokens<1, 8, 256, true>(q_nope + (size_t)h * kDh, (size_t)kHeads * kDh, n0, tokens, tid, st);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's code rows have landed
    __syncthreads();
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {  // k = 64 hf + 8 ks .. +7: unit 4 hf + ks / 2, half ks % 2
      const int u = (4 * hf + (ks >> 1)) ^ (r & 7);
      const u32x2 a = *(const u32x2*)&w_lds[r * 128 + u * 16 + (ks & 1) * 8];
      const uint64_t b = act_b(st.codes, l32, hf, 0, 1, ks);
      acc = mfma_fp8(a[0], a[1], (uint32_t)b, (uint32_t)(b >> 32), acc);
    }
    stage_fragment(tile, 256 / 16, l32, hf, 2 * 32 * wave, acc, st.scale[l32] * sw);
    __syncthreads();
    store_tile<256>(tile, 256 / 16, (uint8_t*)(q_lat + (size_t)h * kDc + 128 * cb), (size_t)kHeads * kDc * 2, n0,
                    tokens, tid);
  }
}

// out-proj: one workgroup per head, 8 waves; wave w owns value rows v = 32 (w & 3) + l32 and the
// latent blocks kb = 2 (w >> 2), +1.  A = W_UV^T codes of row v (the lane's k half of each of its
// two latent blocks: 2 x 64 bytes, loaded once).  Each latent block's MFMA sum is scaled by
// s_o[n][kb] * s_w[h][kb]; waves 4..7 hand their fp32 sums to waves 0..3 through LDS, which add
// them (blocks 0+1, then 2+3) and stage the bf16 rows (256 bytes per token) for whole-row stores.
__global__ __launch_bounds__(512) void out_proj_fp8_kernel(const float* __restrict__ o_lat,
                                                           const uint8_t* __restrict__ codes,
                                                           const float* __restrict__ scales,
                                                           uint16_t* __restrict__ out, int tokens) {
  __shared__ __attribute__((aligned(16))) ActCodes<4> st;
  __shared__ __attribute__((aligned(16))) float red[4][16][64];
  __shared__ __attribute__((aligned(16))) uint8_t tile[32 * kDh * 2];
  const int h = blockIdx.x, tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int vb = wave & 3, kh = wave >> 2;
  const int lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int v = vb * 32 + l32;
  uint32_t aw[2][16];
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2) {
    const uint8_t* src = codes + ((size_t)h * kDh + v) * kDc + (2 * kh + k2) * 128 + 64 * hf;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const u32x4 q = *(const u32x4*)(src + 16 * u);
      aw[k2][4 * u] = q[0], aw[k2][4 * u + 1] = q[1], aw[k2][4 * u + 2] = q[2], aw[k2][4 * u + 3] = q[3];
    }
  }
  const float sw0 = scales[h * 4 + 2 * kh], sw1 = scales[h * 4 + 2 * kh + 1];
  for (int n0 = 0; n0 < tokens; n0 += 32) {
    __syncthreads();
    code_tokens<4, 16, 512, false>(o_lat + (size_t)h * kDc, (size_t)kHeads * kDc, n0, tokens, tid, st);
    __syncthreads();
    f32x16 acc = {};
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const int kb = 2 * kh + k2;
      f32x16 part = {};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const uint64_t b = act_b(st.codes, l32, hf, kb, 4, ks);
        part = mfma_fp8(aw[k2][2 * ks], aw[k2][2 * ks + 1], (uint32_t)b, (uint32_t)(b >> 32), part);
      }
      const float s = st.scale[l32 * 4 + kb] * (k2 ? sw1 : sw0);
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] += part[e] * s;
    }
    if (kh == 1) {
#pragma unroll
      for (int e = 0; e < 16; ++e) red[vb][e][lane] = acc[e];
    }
    __syncthreads();
    if (kh == 0) {
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] += red[vb][e][lane];
      stage_fragment(tile, kDh * 2 / 16, l32, hf, 2 * vb * 32, acc, 1.0f);
    }
    __syncthreads();
    store_tile<512>(tile, kDh * 2 / 16, (uint8_t*)(out + (size_t)h * kDh), (size_t)kHeads * kDh * 2, n0, tokens,
                    tid);
  }
}

hipError_t launch_quantize_weight_fp8(const void* w, void* packed, bool transpose, hipStream_t stream) {
  forget_stale_error();
  uint8_t* codes = (uint8_t*)packed;
  float* scales = (float*)(codes + (size_t)kHeads * kDc * kDh);
  hipLaunchKernelGGL(quantize_weight_fp8_kernel, dim3(4, kHeads), dim3(256), 0, stream, (const uint16_t*)w, codes,
                     scales, transpose ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_absorb_q_fp8(const void* q_nope, const void* packed, void* q_lat, int tokens, hipStream_t stream) {
  forget_stale_error();
  if (tokens == 0) return hipSuccess;
  const uint8_t* codes = (const uint8_t*)packed;
  const float* scales = (const float*)(codes + (size_t)kHeads * kDc * kDh);
  hipLaunchKernelGGL(absorb_q_fp8_kernel, dim3(4, kHeads), dim3(256), 0, stream, (const uint16_t*)q_nope, codes,
                     scales, (uint16_t*)q_lat, tokens);
  return hipGetLastError();
}

hipError_t launch_out_proj_fp8(const float* o_lat, const void* packed, void* out, int tokens, hipStream_t stream) {
  forget_stale_error();
  if (tokens == 0) return hipSuccess;
  const uint8_t* codes = (const uint8_t*)packed;
  const float* scales = (const float*)(codes + (size_t)kHeads * kDc * kDh);
  hipLaunchKernelGGL(out_proj_fp8_kernel, dim3(kHeads), dim3(512), 0, stream, o_lat, codes, scales, (uint16_t*)out,
                     tokens);
  return hipGetLastError();
}

}  // namespace mla
