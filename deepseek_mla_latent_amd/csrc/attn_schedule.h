// LDS ring schedule of the bf16 decode-attention kernel, shared by the kernel and the host (where
// mla_debug_attn_schedule exposes it so a CPU test can walk it).
//
// A workgroup walks its key range in ntiles tiles of 32 tokens.  Tile t lives in ring buffer
// t % kNumBufs.  The prologue loads tiles 0-2; iteration t (0 <= t < ntiles) then scores tile t+1,
// takes the weighted sum of tile t, and issues the direct-to-LDS loads of tile t+3 into buffer
// (t+3) % 4, the one tile t-1 used.  A workgroup barrier closes iteration t only while tiles remain
// to publish (t + 2 < ntiles); it is what orders the loads of iteration t+1 after every wave's
// reads of tile t.
//
// Past the last tile the loads of an iteration still issue (a branch per load inside the MFMA
// stream measured slower than the load) and carry bytes nobody reads; they must still never land
// in a buffer another wave may be reading.  Iterations ntiles-3 and ntiles-2 write buffer
// (t+3) % 4 = tile t-1's, which the barrier closing iteration t-1 (t + 1 < ntiles) already freed.
// The last iteration has no such barrier behind it (tile t-1 = ntiles-2 may still be summed by a
// slower wave), so its loads go to buffer (t+2) % 4 instead: tile t-2's, freed by the barrier that
// closed iteration t-2, or a buffer no tile ever used when t < 2.
#pragma once

namespace mla {

constexpr int kNumBufs = 4;  // LDS tile buffers in the ring

// Whether a workgroup barrier closes iteration t.
__host__ __device__ constexpr bool attn_barrier_after(int t, int ntiles) { return t + 2 < ntiles; }

// Ring buffer that the loads issued in iteration t write.
__host__ __device__ constexpr int attn_dma_buffer(int t, int ntiles) {
  return (t + 1 < ntiles ? t + 3 : t + 2) % kNumBufs;
}

}  // namespace mla
