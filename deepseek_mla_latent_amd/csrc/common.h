// Shared device-side definitions for the gfx950 MLA decode kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace mla {

// Launch helpers read the launch's status from the thread's last-error slot right after the
// launch.  An error that an earlier, unrelated runtime call left there (the caller's own, or a
// framework's) would then be reported as this launch's, so the slot is cleared first.
inline void forget_stale_error() { (void)hipGetLastError(); }

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define MLA_LDS __attribute__((address_space(3)))
#define MLA_GLOBAL __attribute__((address_space(1)))

// D(32x32) += A(32x16) * B(16x32), bf16 in, fp32 accumulate.
// Lane l holds A[l%32][8*(l/32) .. +7], B[8*(l/32) .. +7][l%32];
// D element i of lane l is D[(i/4)*8 + (l/32)*4 + i%4][l%32].
__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// D(32x32) += A(32x2) * B(2x32), fp32. Lane l holds A[l%32][l/32], B[l/32][l%32]; D as above.
__device__ __forceinline__ f32x16 mfma32x32x2f32(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// bf16 <-> fp32.  The narrowing casts compile to v_cvt_pk_bf16_f32 (round to nearest even).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup w -> XCD w % 8), each XCD
// with its own L2. Renumber so that consecutive logical ids run on the same XCD: logical ids
// [0, n0) go to XCD 0, the next block to XCD 1, ... A bijection on [0, n).
__device__ __forceinline__ int xcd_remap(int w, int n) {
  const int q = n >> 3, r = n & 7;
  const int xcd = w & 7, local = w >> 3;
  return xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

// Table checks of the bounds-checked build (see Bounds in kernels.h); without MLA_DEBUG_BOUNDS
// they compile to nothing.  The flag and the count go out as vector atomics.
#ifdef MLA_DEBUG_BOUNDS
__device__ __forceinline__ void bounds_report(const Bounds& bd, uint32_t what) {
  atomicOr(bd.err, what);
  atomicAdd(bd.err + 1, 1u);
}
// seq_lens entry L, clamped into [0, max_seq_len]
__device__ __forceinline__ int checked_len(const Bounds& bd, int L) {
  if (L < 0 || L > bd.max_seq_len) {
    bounds_report(bd, kBoundsBadSeqLen);
    L = L < 0 ? 0 : bd.max_seq_len;
  }
  return L;
}
// whether page id pid may be used (num_pages 0: any non-negative id)
__device__ __forceinline__ bool page_ok(const Bounds& bd, int pid) {
  const uint32_t lim = bd.num_pages > 0 ? (uint32_t)bd.num_pages : 0x80000000u;
  if ((uint32_t)pid < lim) return true;
  bounds_report(bd, kBoundsBadPage);
  return false;
}
// a page id to read from: pid, or page 0 when it is out of range
__device__ __forceinline__ int checked_page(const Bounds& bd, int pid) { return page_ok(bd, pid) ? pid : 0; }
#else
__device__ __forceinline__ int checked_len(const Bounds&, int L) { return L; }
__device__ __forceinline__ bool page_ok(const Bounds&, int) { return true; }
__device__ __forceinline__ int checked_page(const Bounds&, int pid) { return pid; }
#endif

}  // namespace mla
