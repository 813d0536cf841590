"""Seeded synthetic inputs for absorbed MLA decode.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic.  Both the CPU oracle (through the tests) and the HIP
path consume what it returns, so the two sides always see bit-identical
inputs.

Shapes follow the decode problem as the pages state it:

* the per-head query split into a no-RoPE part ``q_nope`` (d_h = 128) and a
  RoPE part ``q_pe`` (d_R = 64), for 128 heads — "DeepSeek-V2的推理成本如何计算？"
  (izhida.com), answer "DeepSeek" (MAC count 128×(512+64+512)) and answer
  "专家" (RoPE as a shared-key MQA term);
* the latent cache row ``[c_KV (512) | k_pe (64)]`` = 576 elements per token,
  one per layer, shared by all heads — same answer "专家" (576 per layer) and
  "Lower latency and higher throughput with multi-node DeepSeek deployment"
  (Perplexity), section "Одноузловое против многоузлового" (70,272 B/token);
* per-head up-projections W_UK and W_UV, stored (heads, d_c, d_h) row-major,
  the (k, h, d) and (k, h, v) tensors of "【笔记】MLA矩阵吸收分析" §二.1 and §三.1
  with the head axis moved to the front;
* a paged cache addressed through a block table ("flexible page table",
  Perplexity post, section "Слой MLA"), 64 tokens per page.

Draw order for one workload (one ``numpy.random.default_rng(seed)``):
cache lengths → page permutation → q_nope → q_pe → W_UK → W_UV → cache pool.
Values are fp32 standard normals; weights are scaled to variance 1/d_c; bf16
workloads round every tensor to bf16 with round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple

import numpy as np

HEADS = 128
KV_LORA_RANK = 512  # d_c
ROPE_DIM = 64  # d_R
HEAD_DIM = 128  # d_h (no-RoPE query/key part and value head dim)
PAGE_SIZE = 64
ROW = KV_LORA_RANK + ROPE_DIM  # 576 elements per cached token

BF16_NAN_BITS = np.uint16(0x7FC0)
_POOL_CHUNK_PAGES = 256  # fixed chunking of the pool draw (keeps the stream reproducible)


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """One synthetic decode batch.

    ``cache_len`` is L, the tokens stored per sequence *including* the
    ``q_len`` tokens appended this step (AppendKV runs before attention in the
    Perplexity post's stage list, section "Наложение вычислений и
    взаимодействия").  ``ragged`` replaces it with an inclusive uniform range.
    """

    name: str
    batch: int
    q_len: int
    cache_len: Optional[int]
    dtype: str  # "f32" or "bf16"
    paged: bool  # True: block table is a random permutation of the pool
    ragged: Optional[Tuple[int, int]] = None
    heads: int = HEADS
    kv_lora_rank: int = KV_LORA_RANK
    rope_dim: int = ROPE_DIM
    head_dim: int = HEAD_DIM
    page_size: int = PAGE_SIZE

    @property
    def softmax_scale(self) -> float:
        # 1/sqrt(d_h + d_R) on the whole logit (no-RoPE + RoPE parts).
        return 1.0 / math.sqrt(self.head_dim + self.rope_dim)


# The five decode workloads: tiny fp32 check, DeepSeek-V2-shaped batch 32 at 4K,
# ragged paged batch 128, MTP verify (2 query tokens, causal), long context.
WORKLOADS = {
    "tiny_fp32": DecodeWorkload("tiny_fp32", batch=1, q_len=1, cache_len=512, dtype="f32", paged=False),
    "b32_t4096": DecodeWorkload("b32_t4096", batch=32, q_len=1, cache_len=4096, dtype="bf16", paged=False),
    "ragged_b128": DecodeWorkload("ragged_b128", batch=128, q_len=1, cache_len=None, dtype="bf16",
                                  paged=True, ragged=(1024, 8192)),
    "mtp_b64_s2_t16384": DecodeWorkload("mtp_b64_s2_t16384", batch=64, q_len=2, cache_len=16384 + 2,
                                        dtype="bf16", paged=True),
    "long_b4_t131072": DecodeWorkload("long_b4_t131072", batch=4, q_len=1, cache_len=131072, dtype="bf16",
                                      paged=False),
}
WORKLOAD_SEEDS = {name: i + 1 for i, name in enumerate(WORKLOADS)}

# Prefill of a whole prompt in multi-head form: one 4096-token prompt (the 4K context of the
# DeepSeek-V2 cost estimate), every token a query (S = L), causal, paged cache.
PREFILL_WORKLOADS = {
    "prefill_b1_s4096": DecodeWorkload("prefill_b1_s4096", batch=1, q_len=4096, cache_len=4096, dtype="bf16",
                                       paged=True),
}
WORKLOAD_SEEDS.update({name: 101 + i for i, name in enumerate(PREFILL_WORKLOADS)})

# Tree-masked verify: each of 32 sequences (4096 committed tokens) verifies an 8-node draft tree
# (``draft_trees``, at most 3 children per node) cached after them, so L = 4096 + 8.
TREE_WORKLOADS = {
    "tree_b32_s8_t4096": DecodeWorkload("tree_b32_s8_t4096", batch=32, q_len=8, cache_len=4096 + 8, dtype="bf16",
                                        paged=True),
}
WORKLOAD_SEEDS.update({name: 201 + i for i, name in enumerate(TREE_WORKLOADS)})
TREE_SEEDS = {name: 301 + i for i, name in enumerate(TREE_WORKLOADS)}  # of the draft trees


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round-to-nearest-even; NaN stays NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    bias = ((u >> np.uint64(16)) & np.uint64(1)) + np.uint64(0x7FFF)
    out = ((u + bias) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_NAN_BITS
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class DecodeInputs:
    """Host copy of one batch.  bf16 tensors are uint16 bit patterns."""

    workload: DecodeWorkload
    seq_lens: np.ndarray  # (B,) int32, L_b
    block_table: np.ndarray  # (B, max_pages) int32, -1 in unused slots
    pool: np.ndarray  # (P, page, 576)
    q_nope: np.ndarray  # (B, S, H, d_h)
    q_pe: np.ndarray  # (B, S, H, d_R)
    w_uk: np.ndarray  # (H, d_c, d_h)
    w_uv: np.ndarray  # (H, d_c, d_h)

    @property
    def is_bf16(self) -> bool:
        return self.workload.dtype == "bf16"

    def f32(self, name: str) -> np.ndarray:
        """Tensor ``name`` as exact fp32 values."""
        a = getattr(self, name)
        return bf16_bits_to_f32(a) if self.is_bf16 else a

    @property
    def num_pages(self) -> int:
        return int(self.pool.shape[0])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.seq_lens.size else 0

    def sequence_rows(self, b: int) -> np.ndarray:
        """The L_b cached rows of sequence b in logical order (fp32 values)."""
        L = int(self.seq_lens[b])
        ps = self.workload.page_size
        npg = -(-L // ps)
        pages = self.block_table[b, :npg]
        rows = self.pool[pages].reshape(npg * ps, -1)[:L]
        return bf16_bits_to_f32(rows) if self.is_bf16 else rows


def _cast(x: np.ndarray, dtype: str) -> np.ndarray:
    return round_to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def generate(w: DecodeWorkload, seed: int, *, poison_unused: bool = False,
             seq_lens: Optional[np.ndarray] = None) -> DecodeInputs:
    """Draw one batch for workload ``w`` from ``default_rng(seed)``.

    ``poison_unused`` fills every pool slot that holds no cached token (the
    tail of each sequence's last page, and pages no sequence owns) with NaN,
    so a kernel that reads them shows it.  ``seq_lens`` overrides the cache
    lengths (used for edge cases); it is then not drawn.
    """
    rng = np.random.default_rng(seed)
    B, S, H, ps = w.batch, w.q_len, w.heads, w.page_size
    if seq_lens is not None:
        lens = np.asarray(seq_lens, dtype=np.int32).reshape(B)
    elif w.ragged is not None:
        lo, hi = w.ragged
        lens = rng.integers(lo, hi + 1, size=B).astype(np.int32)
    else:
        lens = np.full(B, w.cache_len, dtype=np.int32)
    pages_per_seq = (lens.astype(np.int64) + ps - 1) // ps
    total_pages = int(pages_per_seq.sum())
    max_pages = int(pages_per_seq.max()) if B else 0
    if w.paged:
        order = rng.permutation(total_pages).astype(np.int32)
    else:
        order = np.arange(total_pages, dtype=np.int32)
    bt = np.full((B, max(max_pages, 1)), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        n = int(pages_per_seq[b])
        bt[b, :n] = order[off:off + n]
        off += n

    f32 = np.float32
    q_nope = rng.standard_normal((B, S, H, w.head_dim), dtype=f32)
    q_pe = rng.standard_normal((B, S, H, w.rope_dim), dtype=f32)
    wscale = f32(1.0 / math.sqrt(w.kv_lora_rank))
    w_uk = rng.standard_normal((H, w.kv_lora_rank, w.head_dim), dtype=f32) * wscale
    w_uv = rng.standard_normal((H, w.kv_lora_rank, w.head_dim), dtype=f32) * wscale

    row = w.kv_lora_rank + w.rope_dim
    pool_dtype = np.uint16 if w.dtype == "bf16" else np.float32
    pool = np.empty((max(total_pages, 1), ps, row), dtype=pool_dtype)
    if total_pages == 0:
        pool[:] = BF16_NAN_BITS if w.dtype == "bf16" else np.nan
    for p0 in range(0, total_pages, _POOL_CHUNK_PAGES):
        p1 = min(total_pages, p0 + _POOL_CHUNK_PAGES)
        pool[p0:p1] = _cast(rng.standard_normal((p1 - p0, ps, row), dtype=f32), w.dtype)

    if poison_unused:
        nan = BF16_NAN_BITS if w.dtype == "bf16" else np.float32(np.nan)
        used = np.zeros(pool.shape[:2], dtype=bool)
        for b in range(B):
            L = int(lens[b])
            for j in range(int(pages_per_seq[b])):
                used[bt[b, j], :max(0, min(ps, L - j * ps))] = True
        pool[~used] = nan

    return DecodeInputs(w, lens, bt, pool, _cast(q_nope, w.dtype), _cast(q_pe, w.dtype),
                        _cast(w_uk, w.dtype), _cast(w_uv, w.dtype))


def generate_named(name: str, *, poison_unused: bool = False) -> DecodeInputs:
    """The batch for one of the named workloads (decode, prefill or tree verify), with its fixed seed."""
    w = {**WORKLOADS, **PREFILL_WORKLOADS, **TREE_WORKLOADS}[name]
    return generate(w, WORKLOAD_SEEDS[name], poison_unused=poison_unused)


def small_workload(batch: int, q_len: int, cache_len=None, *, dtype: str = "bf16", paged: bool = True,
                   ragged=None, name: str = "small") -> DecodeWorkload:
    """A reduced-size workload with the real head dims (for parity at oracle-friendly sizes)."""
    return DecodeWorkload(name, batch=batch, q_len=q_len, cache_len=cache_len, dtype=dtype, paged=paged,
                          ragged=ragged)


def generate_latent(w: DecodeWorkload, seed: int):
    """Stand-alone inputs for the attention and output-projection calls.

    Returns (q_lat, o_lat): q_lat (B,S,H,d_c) with the variance an absorbed query has
    (d_h · 1/d_c = 1/4), rounded to the workload dtype; o_lat (B,S,H,d_c) fp32 N(0,1),
    the latent output the projection consumes.  Drawn from ``default_rng(seed)``.
    """
    rng = np.random.default_rng(seed)
    shape = (w.batch, w.q_len, w.heads, w.kv_lora_rank)
    q_lat = rng.standard_normal(shape, dtype=np.float32) * np.float32(math.sqrt(w.head_dim / w.kv_lora_rank))
    o_lat = rng.standard_normal(shape, dtype=np.float32)
    return _cast(q_lat, w.dtype), o_lat


def draft_trees(batch: int, size: int, seed: int, *, max_children: int = 3) -> np.ndarray:
    """Seeded draft trees for tree-masked verify: (batch, size) int32 parent indices.

    Node 0 is the root (parent -1, a child of the last committed token); every later node j picks
    its parent uniformly among the earlier nodes that still have fewer than ``max_children``
    children, so parents always come before children (the order the nodes are cached in).  The
    shape follows EAGLE-style speculation trees (a few candidates per level), which the Perplexity
    post names as planned work (section "Будущая работа").
    """
    rng = np.random.default_rng(seed)
    parents = np.full((batch, size), -1, dtype=np.int32)
    for b in range(batch):
        children = np.zeros(size, dtype=np.int64)
        for j in range(1, size):
            open_nodes = np.flatnonzero(children[:j] < max_children)
            p = int(rng.choice(open_nodes))
            parents[b, j] = p
            children[p] += 1
    return parents
