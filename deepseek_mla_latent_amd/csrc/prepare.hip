// The step before the path, gfx950: the fused a-projection as a plain bf16 linear layer, and
// rotary position embedding with AppendKV into the paged cache.
//
// The Perplexity post ("Lower latency and higher throughput with multi-node DeepSeek deployment")
// lists InputNorm, QKVProj, AppendKV, BMM as the stage before attention (section "Наложение
// вычислений и взаимодействия") and fuses q_a_proj and kv_a_proj into one projection (section
// "Слой MLA"); the absorption note ("【笔记】MLA矩阵吸收分析", §二.1) gives the compressed widths
// (q_lora_rank, kv_lora_rank).
//
//   linear_kernel       y = x W (bf16 in, fp32 accumulation) on 32x32x16 bf16 MFMAs; split over K
//                       when the grid would otherwise not fill the chip, with a deterministic
//                       reduction of the fp32 partials (linear_reduce_kernel).
//   rope_append_kernel  per new token: rotate q_pe of every head and k_pe (RoFormer's rotation of
//                       consecutive pairs), and write [c_KV | rotated k_pe] into its cache slot.
#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

__device__ __forceinline__ bf16x8 lds_b128(const MLA_LDS char* p) { return *(const MLA_LDS bf16x8*)p; }
__device__ __forceinline__ uint32_t lds_u32_(const MLA_LDS char* p) { return (uint32_t)(uintptr_t)p; }

// Transposed 16-bit read: within each group of 16 lanes, lane i names the 8-byte piece
// (row i/4, columns 4(i%4) .. +3) of a 4 x 16 block and receives column i of that block.
__device__ __forceinline__ bf16x8 lds_tr_pair(const MLA_LDS char* lo, const MLA_LDS char* hi) {
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)lo);
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)hi);
  const i16x8 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, r);
}

}  // namespace

// ------------------------------------------------------------------------------------------------
// y (M x N) = x (M x K) W (K x N), row-major bf16.  Workgroup = 2 waves = 64 output columns x
// 32·MB rows x one K range; wave w owns columns 32 w .. +31 and all MB row blocks.  The product is
// taken transposed, y^T = W^T x^T: W^T is the A operand (read transposed from LDS), x^T the B
// operand (8 consecutive k of one row per lane: a ds_read_b128).  K advances in chunks of 64
// streamed into a ring of kLinRing LDS buffers by direct-to-LDS loads, kLinRing - 1 chunks ahead
// (for a few rows the layer is a weight stream, and the ring keeps enough of it in flight).
//   W chunk: 64 rows (k) x 128 B; unit u of row r at u ^ (((r >> 1) & 1) << 2), so the 4 rows x
//            64 B of a transposed read land in the four 64-byte quarters of the 256-byte bank row;
//   x chunk: 32·MB rows x 128 B; unit u of row m at u ^ ((m >> 1) & 7).
// Accumulators: element e of block mb is y^T[32 wave + 8 (e/4) + 4 hf + e%4][32 mb + l32], so a
// lane holds 4 consecutive columns of one row.
constexpr int kLinRing = 6;

__device__ __forceinline__ void lin_dma16(const void* sbase, uint32_t voff, uint32_t lds) {
  const uint64_t a = (uint64_t)(uintptr_t)sbase;
  const uint64_t base = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base),
               "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

template <int MB>
__device__ __forceinline__ void lin_wait(int younger) {  // at most `younger` chunks (2 + 2 MB loads each) in flight
  constexpr int per = 4 + 2 * MB;  // this wave's loads per chunk
  switch (younger) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(per) : "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * per) : "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * per) : "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * per) : "memory"); break;
  }
}

template <int MB>
__global__ __launch_bounds__(128) void linear_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                                                     uint16_t* __restrict__ y, float* __restrict__ partial, int M,
                                                     int K, int N, int k_per_split) {
  constexpr int kChunk = 64;
  constexpr int kWBytes = kChunk * 64 * 2;       // 8 KiB
  constexpr int kXBytes = 32 * MB * kChunk * 2;  // 4 KiB per row block
  constexpr int kBuf = kWBytes + kXBytes;
  __shared__ __attribute__((aligned(16))) char lds_raw[kLinRing * kBuf];
  MLA_LDS char* lds = (MLA_LDS char*)lds_raw;

  const int nblocks = N / 64, mblocks = (M + 32 * MB - 1) / (32 * MB);
  // consecutive logical ids share an XCD (and its L2): neighbouring column blocks of one K range
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int nb = bid % nblocks;
  const int mblk = (bid / nblocks) % mblocks;
  const int split = bid / (nblocks * mblocks);
  const int n0 = nb * 64, m0 = mblk * 32 * MB;
  const int k0 = split * k_per_split, k1 = min(K, k0 + k_per_split);
  const int nchunks = (k1 - k0) / kChunk;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hf = lane >> 5;

  // chunk c: W rows k0 + 64c .. +63 (columns n0 .. n0 + 63) in 8 pieces of 8 rows, x rows
  // m0 .. m0 + 32·MB - 1 (clamped to M - 1: their results are not stored) in 4·MB pieces
  auto issue_chunk = [&](int c) {
    MLA_LDS char* wb = lds + (c % kLinRing) * kBuf;
    MLA_LDS char* xb = wb + kWBytes;
    const int kc = k0 + c * kChunk;
    const char* wbase = (const char*)(w + (size_t)kc * N + n0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int pc = wave * 4 + j, r = 8 * pc + (lane >> 3), p = lane & 7;
      lin_dma16(wbase, (uint32_t)(r * N * 2 + ((p ^ (((r >> 1) & 1) << 2)) << 4)), lds_u32_(wb + pc * 1024));
    }
    const char* xbase = (const char*)(x + kc);
#pragma unroll
    for (int j = 0; j < 2 * MB; ++j) {
      const int pc = wave * 2 * MB + j, r = 8 * pc + (lane >> 3), p = lane & 7;
      const int m = min(m0 + r, M - 1);
      lin_dma16(xbase, (uint32_t)((size_t)m * K * 2 + ((p ^ ((r >> 1) & 7)) << 4)), lds_u32_(xb + pc * 1024));
    }
  };

  // A operand (W^T): rows k = 16 ks + 8 hf + (lane >> 2 & 3) (+4), columns n = 32 wave +
  // 16 ((lane >> 4) & 1) + 4 (lane & 3)
  const int tr_row = 8 * hf + ((lane >> 2) & 3);
  const int tr_col = 32 * wave + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  auto w_off = [&](int r) { return r * 128 + ((((tr_col >> 3) ^ (((r >> 1) & 1) << 2))) << 4) + (tr_col & 7) * 2; };

  f32x16 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x16{};
  for (int c = 0; c < kLinRing - 1 && c < nchunks; ++c) issue_chunk(c);
  auto consume = [&](int c) {
    __syncthreads();  // chunk c is in LDS; every wave is done with chunk c - 1's buffer
    if (c + kLinRing - 1 < nchunks) issue_chunk(c + kLinRing - 1);
    const MLA_LDS char* wb = lds + (c % kLinRing) * kBuf;
    const MLA_LDS char* xb = wb + kWBytes;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int r = ks * 16 + tr_row;
      const bf16x8 af = lds_tr_pair(wb + w_off(r), wb + w_off(r + 4));
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int m = mb * 32 + l32;
        const bf16x8 bf = lds_b128(xb + m * 128 + (((2 * ks + hf) ^ ((m >> 1) & 7)) << 4));
        acc[mb] = mfma32x32x16(af, bf, acc[mb]);
      }
    }
  };
  // Steady state: kLinRing - 2 younger chunks stay in flight, a constant wait (a wait chosen per
  // chunk by a switch put a chain of compares and branches into every iteration: 4% slower).
  int c = 0;
  for (; c + kLinRing - 2 < nchunks; ++c) {
    lin_wait<MB>(kLinRing - 2);
    consume(c);
  }
  for (; c < nchunks; ++c) {  // the last kLinRing - 2 chunks
    lin_wait<MB>(nchunks - 1 - c);
    consume(c);
  }

  // element e of block mb: column n0 + 32 wave + 8 (e/4) + 4 hf + e%4, row m0 + 32 mb + l32
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = m0 + mb * 32 + l32;
    if (m >= M) continue;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int n = n0 + 32 * wave + 8 * g + 4 * hf;
      const f32x16& d = acc[mb];
      if (partial) {
        f32x4 v = {d[4 * g], d[4 * g + 1], d[4 * g + 2], d[4 * g + 3]};
        *(f32x4*)(partial + ((size_t)split * M + m) * N + n) = v;
      } else {
        u32x2 v;
        v[0] = pack_bf16x2(d[4 * g], d[4 * g + 1]);
        v[1] = pack_bf16x2(d[4 * g + 2], d[4 * g + 3]);
        *(u32x2*)(y + (size_t)m * N + n) = v;
      }
    }
  }
}

// y = sum over the K splits of the fp32 partials (in split order), rounded once to bf16.
__global__ __launch_bounds__(256) void linear_reduce_kernel(const float* __restrict__ partial,
                                                            uint16_t* __restrict__ y, int MN4, int splits) {
  const int i = blockIdx.x * 256 + threadIdx.x;  // group of 4 elements
  if (i >= MN4) return;
  f32x4 s = *(const f32x4*)(partial + (size_t)i * 4);
  for (int k = 1; k < splits; ++k) {
    const f32x4 v = *(const f32x4*)(partial + ((size_t)k * MN4 + i) * 4);
    s += v;
  }
  u32x2 o;
  o[0] = pack_bf16x2(s[0], s[1]);
  o[1] = pack_bf16x2(s[2], s[3]);
  *(u32x2*)(y + (size_t)i * 4) = o;
}

hipError_t launch_linear(const void* x, const void* w, void* y, float* partial, int M, int K, int N, int splits,
                         hipStream_t stream) {
  forget_stale_error();
  const int mb = M >= 512 ? 4 : 1;
  const int mblocks = (M + 32 * mb - 1) / (32 * mb);
  const int64_t grid = (int64_t)mblocks * (N / 64) * splits;
  if (grid == 0) return hipSuccess;
  float* part = splits > 1 ? partial : nullptr;
  if (mb == 4)
    hipLaunchKernelGGL(linear_kernel<4>, dim3((unsigned)grid), dim3(128), 0, stream, (const uint16_t*)x,
                       (const uint16_t*)w, (uint16_t*)y, part, M, K, N, K / splits);
  else
    hipLaunchKernelGGL(linear_kernel<1>, dim3((unsigned)grid), dim3(128), 0, stream, (const uint16_t*)x,
                       (const uint16_t*)w, (uint16_t*)y, part, M, K, N, K / splits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  const int mn4 = M * N / 4;
  hipLaunchKernelGGL(linear_reduce_kernel, dim3((unsigned)((mn4 + 255) / 256)), dim3(256), 0, stream, partial,
                     (uint16_t*)y, mn4, splits);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------
// base^(-2j/64) for the 32 pairs, formed on the host in fp64 and passed by value
struct InvFreq {
  double v[32];
};

// One workgroup (128 threads) per new token (b, i) at position pos = L_b - S + i:
//   the 32 rotation angles pos * base^(-2j/64) are formed and reduced modulo 2 pi in fp64 (exact
//   enough for positions in the hundreds of thousands), their cos / sin taken in fp32 and kept in LDS;
//   q_pe[b,i,h,:] of every head is rotated (thread h), k_pe from the kv_a row likewise (thread 0..31
//   one pair each), and [c_KV | rotated k_pe] is written to page block_table[b][pos / 64], slot
//   pos % 64.  A token at a negative position (L_b < S) is rotated but not written.
__global__ __launch_bounds__(128) void rope_append_kernel(uint16_t* __restrict__ q_pe, const uint16_t* __restrict__ kv_a,
                                                          int kv_stride, uint16_t* __restrict__ pool,
                                                          const int32_t* __restrict__ block_table,
                                                          const int32_t* __restrict__ seq_lens, int S,
                                                          int max_pages, InvFreq inv_freq_arg, Bounds bounds) {
  __shared__ float cs[32], sn[32];
  __shared__ __attribute__((aligned(16))) uint16_t krot[kDr];
  const int token = blockIdx.x, b = token / S, i = token % S;
  const int tid = threadIdx.x;
  const uint16_t* src = kv_a + (size_t)token * kv_stride;
  uint16_t* q = q_pe + ((size_t)token * kHeads + tid) * kDr;
  // every load is issued before any result is needed: the position and page, this head's q_pe
  // (thread = head), a 16-byte piece of c_KV (threads 0..63) and a k_pe pair (threads 0..31)
  const int pos = checked_len(bounds, seq_lens[b]) - S + i;
  const int page = pos >= 0 ? block_table[(size_t)b * max_pages + pos / kPage] : 0;
  u32x4 qv[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) qv[u] = *(const u32x4*)(q + u * 8);
  u32x4 cv = {0u, 0u, 0u, 0u};
  if (tid < kDc / 8) cv = *(const u32x4*)(src + tid * 8);
  uint32_t kp = 0;
  if (tid < 32) kp = *(const uint32_t*)(src + kDc + 2 * tid);
  if (tid < 32) {
    // angle in fp64, reduced to [-pi, pi] in fp64, then an fp32 sine / cosine of the remainder
    const double th = (double)pos * inv_freq_arg.v[tid];
    const double r = th - 6.283185307179586 * rint(th * 0.15915494309189535);
    float s, c;
    sincosf((float)r, &s, &c);
    cs[tid] = c;
    sn[tid] = s;
    const float x0 = __uint_as_float(kp << 16), x1 = __uint_as_float(kp & 0xffff0000u);
    *(uint32_t*)&krot[2 * tid] = pack_bf16x2(x0 * c - x1 * s, x0 * s + x1 * c);
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 8; ++u) {  // q_pe of head tid, 4 pairs per 16 bytes
    u32x4 v = qv[u];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int p = u * 4 + j;
      const float x0 = __uint_as_float(v[j] << 16), x1 = __uint_as_float(v[j] & 0xffff0000u);
      v[j] = pack_bf16x2(x0 * cs[p] - x1 * sn[p], x0 * sn[p] + x1 * cs[p]);
    }
    *(u32x4*)(q + u * 8) = v;
  }
  if (pos < 0 || !page_ok(bounds, page)) return;  // no slot (or, checked, an unusable page): no write
  uint16_t* dst = pool + ((size_t)page * kPage + pos % kPage) * kRow;
  if (tid < kDc / 8) *(u32x4*)(dst + tid * 8) = cv;  // c_KV: a copy
  else if (tid < kDc / 8 + kDr / 8)
    *(u32x4*)(dst + kDc + (tid - kDc / 8) * 8) = *(const u32x4*)(krot + (tid - kDc / 8) * 8);
}

hipError_t launch_rope_append(void* q_pe, const void* kv_a, int kv_stride, void* pool, const int32_t* block_table,
                              const int32_t* seq_lens, int B, int S, int max_pages, double base, const Bounds& bounds,
                              hipStream_t stream) {
  forget_stale_error();
  const int64_t grid = (int64_t)B * S;
  if (grid == 0) return hipSuccess;
  InvFreq f;
  for (int j = 0; j < 32; ++j) f.v[j] = pow(base, -2.0 * j / kDr);
  hipLaunchKernelGGL(rope_append_kernel, dim3((unsigned)grid), dim3(128), 0, stream, (uint16_t*)q_pe,
                     (const uint16_t*)kv_a, kv_stride, (uint16_t*)pool, block_table, seq_lens, S, max_pages, f, bounds);
  return hipGetLastError();
}

}  // namespace mla
