"""Algorithmic bytes and FLOPs of the three decode calls, and MI355X roofline times.

"Algorithmic" means what the method itself must move and compute: every cached row read once,
weights read once, inputs read and outputs written once.  Implementation overhead (split-K
partials, LDS re-reads, redundant loads) is excluded on purpose, so achieved/peak is an honest
fraction of the hardware limit.

* absorb_q:  W_UK + q_nope + q_lat;  2·T·H·d_c·d_h FLOPs (T = B·S tokens)
* decode_attn: cache L_b·(d_c+d_R)·e for every sequence, q_lat + q_pe, block-table entries of the
  used pages + lengths (int32), o_lat + lse written in fp32;  2·H·(d_c + d_R + d_c) FLOPs per
  visible (query, key) pair — twice the per-token multiply-accumulate count of the izhida answer
  "DeepSeek" ("DeepSeek-V2的推理成本如何计算？": 128×(512+64+512) per cached token).
* out_proj:  W_UV + o_lat (fp32) + out;  2·T·H·d_c·d_h FLOPs.

Prefill in multi-head form (two calls):

* prefill_kv_up: latent rows and k_pe read once, W_UK + W_UV, [K_nope | V] of every cached token
  and head plus the dense k_pe written;  2·L·H·d_c·2d_h FLOPs (L = all cached tokens).
* prefill_attn: q_nope + q_pe, [K_nope | V] + k_pe read once, out + lse written;
  2·H·(d_h + d_R + d_h) FLOPs per visible (query, key) pair.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Sequence

HBM_PEAK_BYTES_S = 8.0e12  # MI355X HBM3E
MFMA_PEAK_FLOPS = {"bf16": 2.5e15, "f32": 157.3e12}  # dense MFMA


@dataclass
class CallCost:
    name: str
    bytes: int
    flops: int

    def roof_seconds(self, dtype: str) -> float:
        return max(self.bytes / HBM_PEAK_BYTES_S, self.flops / MFMA_PEAK_FLOPS[dtype])

    def bound(self, dtype: str) -> str:
        return "hbm" if self.bytes / HBM_PEAK_BYTES_S >= self.flops / MFMA_PEAK_FLOPS[dtype] else "mfma"


def _tree_visible_new_keys(parents, L: int) -> list:
    """Per node of a draft tree: how many of the new keys it sees (itself and its ancestors, those at
    positions >= 0), walking parent links."""
    S = len(parents)
    out = []
    for i in range(S):
        n, j = 0, i
        while j >= 0:
            n += 1 if L - S + j >= 0 else 0
            p = int(parents[j])
            j = p if p < j else -1
        out.append(n)
    return out


def visible_pairs(seq_lens: Sequence[int], q_len: int, causal: bool = True, tree=None) -> int:
    """(query, key) pairs the attention scores: causal / full rule, or a draft tree's mask
    (``tree``: (B, S) parents)."""
    pairs = 0
    for b, L in enumerate(seq_lens):
        L = int(L)
        if tree is not None:
            pairs += q_len * max(0, L - q_len) + sum(_tree_visible_new_keys(tree[b], L))
            continue
        for i in range(q_len):
            n = L - q_len + i + 1 if causal else L
            pairs += max(0, min(L, n))
    return pairs


def path_costs(seq_lens: Sequence[int], q_len: int, dtype: str, *, heads: int = 128, d_c: int = 512,
               d_r: int = 64, d_h: int = 128, page: int = 64, causal: bool = True, fp8_projections: bool = False,
               tree=None, fused: bool = False):
    """Algorithmic bytes and FLOPs of each call of one decode step.  With ``fused`` the attention
    and the out-projection are one call (mla_decode_attn_out_proj, or its FP8 form, without the
    optional latent outputs): its bytes are the attention's reads plus W_UV and the output."""
    e = 2 if dtype == "bf16" else 4
    ew = 1 if fp8_projections else e  # weight element bytes (FP8 codes; scales added below)
    wsc = heads * (d_c // 128) * 4 if fp8_projections else 0
    B = len(seq_lens)
    T = B * q_len
    absorb = CallCost("mla_absorb_q", heads * d_c * d_h * ew + wsc + T * heads * (d_h + d_c) * e,
                      2 * T * heads * d_c * d_h)
    cache = sum(int(L) for L in seq_lens) * (d_c + d_r) * e
    tables = sum(-(-int(L) // page) for L in seq_lens) * 4 + B * 4
    attn = CallCost("mla_decode_attn",
                    cache + T * heads * (d_c + d_r) * e + tables + T * heads * (d_c + 1) * 4,
                    2 * heads * (d_c + d_r + d_c) * visible_pairs(seq_lens, q_len, causal, tree))
    if tree is not None:
        attn = CallCost(attn.name, attn.bytes + T * 4, attn.flops)  # plus the parent table
    out = CallCost("mla_out_proj", heads * d_c * d_h * ew + wsc + T * heads * d_c * 4 + T * heads * d_h * e,
                   2 * T * heads * d_c * d_h)
    if fused:
        reads = attn.bytes - T * heads * (d_c + 1) * 4  # no o_lat / lse written
        name = "mla_decode_attn_out_proj_fp8" if fp8_projections else "mla_decode_attn_out_proj"
        return [absorb, CallCost(name, reads + heads * d_c * d_h * ew + wsc + T * heads * d_h * e,
                                 attn.flops + out.flops)]
    return [absorb, attn, out]


def prefill_costs(seq_lens: Sequence[int], q_len: int, dtype: str = "bf16", *, heads: int = 128, d_c: int = 512,
                  d_r: int = 64, d_h: int = 128, causal: bool = True):
    e = 2 if dtype == "bf16" else 4
    L = sum(int(n) for n in seq_lens)
    T = len(seq_lens) * q_len
    up = CallCost("mla_prefill_kv_up",
                  L * (d_c + d_r) * e + 2 * heads * d_c * d_h * e + L * heads * 2 * d_h * e + L * d_r * e,
                  2 * L * heads * d_c * 2 * d_h)
    attn = CallCost("mla_prefill_attn",
                    T * heads * (d_h + d_r) * e + L * heads * 2 * d_h * e + L * d_r * e + T * heads * (d_h * e + 4),
                    2 * heads * (d_h + d_r + d_h) * visible_pairs(seq_lens, q_len, causal))
    return [up, attn]
