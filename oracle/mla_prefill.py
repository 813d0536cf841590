"""fp64 CPU reference of MLA prefill in multi-head form — TEST INFRASTRUCTURE (see ``oracle/__init__``).

The pages give the order-1 route ("【笔记】MLA矩阵吸收分析", §二.1 and §三.1) and say when it wins:
with as many query tokens as keys (t = s, training and prefill) order 1 costs fewer FLOPs than the
absorbed order (§二.4.1).  The Perplexity post ("Lower latency and higher throughput with
multi-node DeepSeek deployment", section "Будущая работа") plans exactly that for its prefill:
project the latent into K/V space first, then compute in MHA form.  Its two steps:

* ``kv_up_reference`` — K_nope = C W_UK[h] and V = C W_UV[h] per head for every cached token
  (§二.1 step 2, shape (b,t,h,d); §三.1 step 1, shape (b,t,h,v)), plus the shared RoPE key.
* ``mha_attention_reference`` — per head, scores of the query against [K_nope | k_pe] (the RoPE
  part is a key shared by every head whose score is added: izhida answer "专家"), exact softmax
  over the visible keys, and the weighted sum of V (§二.1 step 3, §三.1 step 2).

The same readings as the decode reference apply (scale is a parameter, natural-log lse, rotated
q_pe / k_pe, query i of S sees the first L - S + i + 1 keys when causal, empty set -> 0 / -inf).
"""
from __future__ import annotations

import numpy as np

from oracle.mla_decode import _softmax_stats, gather_rows, visible_keys


def kv_up_reference(pool, block_table, seq_lens, w_uk, w_uv, *, page_size: int = 64, heads=None):
    """Up-projected keys and values of every cached token, fp64.

    Returns K (B,H,Lmax,d_h), V (B,H,Lmax,d_h) and kpe (B,Lmax,d_R); rows at or past seq_lens[b]
    are NaN (they hold no token).  ``heads`` limits the heads computed (the others stay NaN).
    """
    seq_lens = np.asarray(seq_lens)
    B = len(seq_lens)
    H, Dc, Dh = w_uk.shape
    Dr = pool.shape[-1] - Dc
    Lmax = int(seq_lens.max()) if B else 0
    K = np.full((B, H, Lmax, Dh), np.nan)
    V = np.full((B, H, Lmax, w_uv.shape[2]), np.nan)
    kpe = np.full((B, Lmax, Dr), np.nan)
    for b in range(B):
        L = int(seq_lens[b])
        rows = gather_rows(pool, block_table[b], L, page_size)
        C = rows[:, :Dc]
        kpe[b, :L] = rows[:, Dc:]
        for h in (range(H) if heads is None else heads):
            K[b, h, :L] = C @ np.asarray(w_uk[h], dtype=np.float64)
            V[b, h, :L] = C @ np.asarray(w_uv[h], dtype=np.float64)
    return K, V, kpe


def mha_attention_reference(q_nope, q_pe, K, V, kpe, seq_lens, *, softmax_scale: float, causal: bool = True,
                            heads=None):
    """Per-head attention over given keys and values, fp64.

    q_nope (B,S,H,d_h), q_pe (B,S,H,d_R), K / V (B,H,>=L,d_h), kpe (B,>=L,d_R).
    Logit of query i, head h, key j: scale * (q_nope . K[b,h,j] + q_pe . kpe[b,j]).
    Returns out (B,S,H,d_v) and lse (B,S,H); heads outside ``heads`` stay NaN.
    """
    q_nope = np.asarray(q_nope, dtype=np.float64)
    q_pe = np.asarray(q_pe, dtype=np.float64)
    B, S, H, _ = q_nope.shape
    out = np.full((B, S, H, V.shape[-1]), np.nan)
    lse = np.full((B, S, H), np.nan)
    for b in range(B):
        L = int(seq_lens[b])
        R = np.asarray(kpe[b, :L], dtype=np.float64)
        for h in (range(H) if heads is None else heads):
            Kh = np.asarray(K[b, h, :L], dtype=np.float64)
            Vh = np.asarray(V[b, h, :L], dtype=np.float64)
            for i in range(S):
                n = visible_keys(L, S, i, causal)
                z = softmax_scale * (Kh[:n] @ q_nope[b, i, h] + R[:n] @ q_pe[b, i, h])
                p, lse[b, i, h] = _softmax_stats(z)
                out[b, i, h] = p @ Vh[:n] if n else 0.0
    return {"out": out, "lse": lse}
