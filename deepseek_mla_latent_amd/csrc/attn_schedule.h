// LDS ring schedule of the bf16 decode-attention kernel, shared by the kernel and the host (where
// mla_debug_attn_schedule exposes it so a CPU test can walk it).
//
// A workgroup walks its key range in ntiles tiles of 32 tokens.  A tile is stored in two parts: its
// 32 latent rows (c_KV, 32 KiB) in ring A and its 32 RoPE-key rows (k_pe, 4 KiB) in ring B.  Each of
// the four waves computes the scores of its own 32 heads, and holds the weighted sum of every head
// over its own quarter of the latent columns, so the probabilities of a tile pass between the waves
// through a third ring, P.
//
// Iteration u (0 <= u < ntiles), between the barriers Z(u-1) and Z(u):
//   * scores of tile u (reads ring A and ring B of tile u); the loads of tile u + 2 are issued;
//   * weighted sum of tile u - 1 (reads ring A of tile u - 1 and ring P of tile u - 1), with the
//     softmax of tile u running in the gaps of its MFMA chain;
//   * the probabilities of tile u (and the rescale words that go with them) are written to ring P;
//     every wave then waits for its loads of tile u + 1 and meets the others at Z(u).
// The prologue loads tiles 0 and 1 and publishes tile 0 with a barrier; after Z(ntiles - 1) the
// weighted sum of the last tile runs.
//
// Why the rings are as deep as they are:
//   * ring A, 4 buffers: tile j is read in iterations j and j + 1, so its buffer is free only after
//     Z(j + 1); tile u + 2 therefore goes where tile u - 2 was, freed by Z(u - 1) at the start of
//     iteration u;
//   * ring B, 3 buffers: the k_pe rows of tile j are read only in iteration j, so tile u + 2 may go
//     where tile u - 1 was, freed by Z(u - 1);
//   * ring P, 2 buffers: the probabilities of tile u are written in iteration u and read in
//     iteration u + 1; the next write into the same buffer is in iteration u + 2, after Z(u + 1).
// Loads past the last tile still issue (a branch per load inside the MFMA stream measured slower
// than the load); they carry no data anyone reads and go to the buffers the ring assigns to their
// tile index, which by the argument above nobody is reading.
#pragma once

namespace mla {

constexpr int kNumBufsA = 4;  // latent parts of tiles
constexpr int kNumBufsB = 3;  // RoPE-key parts of tiles
constexpr int kNumBufsP = 2;  // probabilities of a tile
constexpr int kLoadAhead = 2;  // iteration u issues the loads of tile u + kLoadAhead

__host__ __device__ constexpr int attn_a_buffer(int tile) { return tile % kNumBufsA; }
__host__ __device__ constexpr int attn_b_buffer(int tile) { return tile % kNumBufsB; }
__host__ __device__ constexpr int attn_p_buffer(int tile) { return tile % kNumBufsP; }

}  // namespace mla
