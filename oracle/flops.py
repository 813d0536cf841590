"""FLOP and byte counts of the MLA decode path — TEST INFRASTRUCTURE (see ``oracle/__init__``).

Convention ("【笔记】MLA矩阵吸收分析" §一.1): FLOPs of a tensor product are
counted with a bias add, so each output element costs 2 × (contracted extent)
and a step costs 2 × the product of the extents of every index it touches.
The note's §一.2 applies it to the two orders of a matrix chain, and §二 / §三
to three computation orders of each MLA absorption.  Each order below is the
note's list of steps, each step named by the indices it touches; the total is
the sum of the steps.  Index letters are the note's: b batch, s query tokens,
t cached tokens, h heads, d no-RoPE head dim, k latent rank (kv_lora_rank),
q query latent rank (q_lora_rank), v value head dim, e model dim.
"""
from __future__ import annotations

from fractions import Fraction
from math import prod


def step_flops(indices: str, **ext: int) -> int:
    """2 × product of the extents of every distinct index a step touches (§一.1 convention)."""
    return 2 * prod(ext[c] for c in sorted(set(indices)))


def linear_flops(B: int, S: int, D: int, O: int, *, bias: bool) -> int:
    """nn.Linear on (B,S,D) with a (D,O) weight (§一.1).

    Each of the B·S·O outputs takes D multiplies and D-1 adds, plus one add for
    the bias when there is one.
    """
    per_element = D + (D - 1) + (1 if bias else 0)
    return B * S * O * per_element


# §一.2: (m,n) x (n,p) x (p,q) in the two association orders.
CHAIN_ORDERS = {
    1: ("mnp", "mpq"),  # (A B) C : A·B first, then ·C
    2: ("npq", "mnq"),  # A (B C) : B·C first, then A·
}

# §二 (first absorption, W_UK): steps of each order.
FIRST_ABSORPTION = {
    # 1: W_UQ c^Q -> (b,s,h,d); W_UK c^KV -> (b,t,h,d); scores over d -> (b,h,s,t)
    1: ("bsqhd", "btkhd", "bhstd"),
    # 2: W_UQ c^Q -> (b,s,h,d); absorb W_UK into the query -> (b,s,h,k); scores over k
    2: ("bsqhd", "bshkd", "bhstk"),
    # 3: pre-multiply W_UQ^T W_UK -> (h,q,k); apply to c^Q -> (b,s,h,k); scores over k
    3: ("hqkd", "bshkq", "bhstk"),
}

# §三 (second absorption, W_UV and W_O): steps of each order.
SECOND_ABSORPTION = {
    # 1: W_UV c^KV -> (b,t,h,v); score · V -> (b,h,s,v); W_O -> (b,h,s,e)
    1: ("bthvk", "bhsvt", "bhsev"),
    # 2: score · c^KV -> (b,h,s,k); W_UV -> (b,h,s,v); W_O -> (b,h,s,e)
    2: ("bhskt", "bhsvk", "bhsev"),
    # 3: pre-multiply W_O W_UV -> (h,k,e); score · c^KV -> (b,h,s,k); apply -> (b,h,s,e)
    3: ("hkev", "bhskt", "bhsek"),
}


def chain_flops(order: int, m: int, n: int, p: int, q: int) -> int:
    return sum(step_flops(st, m=m, n=n, p=p, q=q) for st in CHAIN_ORDERS[order])


def first_absorption_flops(order: int, *, b: int, s: int, t: int, h: int, d: int, k: int, q: int) -> int:
    return sum(step_flops(st, b=b, s=s, t=t, h=h, d=d, k=k, q=q) for st in FIRST_ABSORPTION[order])


def second_absorption_flops(order: int, *, b: int, s: int, t: int, h: int, v: int, k: int, e: int) -> int:
    return sum(step_flops(st, b=b, s=s, t=t, h=h, v=v, k=k, e=e) for st in SECOND_ABSORPTION[order])


def decode_attention_macs(*, heads: int, kv_lora_rank: int, rope_dim: int, context: int) -> int:
    """Multiply-accumulates of one decode token's attention in one layer.

    "DeepSeek-V2的推理成本如何计算？" answer "DeepSeek": per head, a 512-d latent
    inner product and a 64-d RoPE inner product for the score, and a weighted
    sum over the 512-d latent for the output, for every cached token.
    """
    return heads * (kv_lora_rank + rope_dim + kv_lora_rank) * context


def projection_weight_elements(*, n_h: int, d_h: int, d_c: int, d_cq: int, d: int, materialised: bool) -> int:
    """Parameter elements of the four attention projections (izhida answer "DeepSeek", 3rd paragraph).

    Materialised: W_Q·W_K^T as (n_h, d_c', d_c) and W_V·W_O as (n_h, d_c, d).
    Not materialised: W_Q (n_h, d_c', d_h), W_K and W_V (n_h, d_c, d_h), W_O (n_h, d_h, d).
    """
    if materialised:
        return n_h * d_cq * d_c + n_h * d_c * d
    return n_h * d_cq * d_h + 2 * n_h * d_c * d_h + n_h * d_h * d


def latent_cache_bytes_per_token(*, layers: int, kv_lora_rank: int, rope_dim: int, elem_bytes: int) -> int:
    """Cached bytes per token over all layers: one [c_KV | k_pe] row per layer.

    Perplexity post, section "Одноузловое против многоузлового" (70,272 B per
    token for DeepSeek-V3/R1); izhida answer "专家" (576 per layer).
    """
    return layers * (kv_lora_rank + rope_dim) * elem_bytes


def mla_to_gqa_cache_ratio(*, kv_lora_rank: int, rope_dim: int, groups: int, head_dim: int) -> Fraction:
    """Per-layer cache of MLA against GQA with ``groups`` KV heads (K and V each)."""
    return Fraction(kv_lora_rank + rope_dim, 2 * groups * head_dim)


# ---------------------------------------------------------------------------------------------
# Algorithmic work of the three library calls (what the method must move and compute; no
# implementation overhead such as split partials).  e = element bytes of the input dtype.

def absorb_q_cost(*, tokens: int, heads: int, d_c: int, d_h: int, e: int):
    """(bytes, flops): read W_UK and q_nope, write q_lat; 2·tokens·h·d_c·d_h flops."""
    nbytes = heads * d_c * d_h * e + tokens * heads * d_h * e + tokens * heads * d_c * e
    return nbytes, step_flops("nhcd", n=tokens, h=heads, c=d_c, d=d_h)


def decode_attn_cost(*, seq_lens, q_len: int, heads: int, d_c: int, d_r: int, e: int, causal: bool = True):
    """(bytes, flops) of the attention call.

    Bytes: every cached row once (L_b·(d_c+d_R)·e), q_lat and q_pe read, block
    table and lengths read (int32), o_lat and lse written in fp32.  FLOPs:
    2·h·(d_c + d_R + d_c) per visible (query, key) pair.
    """
    B = len(seq_lens)
    page = 64
    cache = sum(int(L) for L in seq_lens) * (d_c + d_r) * e
    q = B * q_len * heads * (d_c + d_r) * e
    table = sum(-(-int(L) // page) for L in seq_lens) * 4 + B * 4
    outs = B * q_len * heads * (d_c + 1) * 4
    pairs = 0
    for L in seq_lens:
        for i in range(q_len):
            n = int(L) - q_len + i + 1 if causal else int(L)
            pairs += max(0, min(int(L), n))
    return cache + q + table + outs, 2 * heads * (d_c + d_r + d_c) * pairs


def out_proj_cost(*, tokens: int, heads: int, d_c: int, d_h: int, e: int):
    """(bytes, flops): read W_UV and o_lat (fp32), write out; 2·tokens·h·d_c·d_h flops."""
    nbytes = heads * d_c * d_h * e + tokens * heads * d_c * 4 + tokens * heads * d_h * e
    return nbytes, step_flops("nhcd", n=tokens, h=heads, c=d_c, d=d_h)
