"""fp64 CPU reference of MLA decode — TEST INFRASTRUCTURE (see ``oracle/__init__``).

What the path computes, as the pages state it:

* Attention scores per head are the no-RoPE part ``q_nope·k_nope`` with
  ``k_nope = W_UK^T c_KV`` plus a RoPE part ``q_pe·k_pe`` whose key ``k_pe`` is
  shared by all heads (a "RoPE MQA" score added to the MLA score) —
  "DeepSeek-V2的推理成本如何计算？" (izhida.com), answer "专家".
* The output per head is ``W_UV^T`` applied to the attention-weighted sum of
  the latent; equivalently the weighted sum of ``v = W_UV^T c_KV`` — same
  answer, and "【笔记】MLA矩阵吸收分析" §三.1 (order 1) / §三.2 (order 2).
* The non-absorbed route ("order 1": up-project K and V per head, then plain
  multi-head attention) is §二.1 and §三.1 of the same note.  This module
  follows it for the end-to-end reference, so it shares no arithmetic with the
  absorbed GPU route; agreement of the two orders is the identity the note and
  the izhida answer rest on.

Readings where the pages are silent (each listed in the design notes):
softmax scale is a caller parameter (1/sqrt(d_h + d_R) for the workloads),
natural-exp softmax, ``lse`` in natural-log units of the scaled logits;
q_pe / k_pe arrive already rotated; with S query tokens and L cached tokens
(the S new ones included) query i sees keys j < L - S + i + 1 when causal;
an empty key set gives o_lat = 0, out = 0, lse = -inf.

Tree-masked verify (the Perplexity post, section "Будущая работа": EAGLE-style speculation
predicts several tokens arranged as a tree): the S new tokens are the nodes of a draft tree,
cached at positions L - S .. L - 1 in an order where every parent precedes its children;
``parents[j]`` in [-1, j) names node j's parent (-1: a child of the last committed token).
Query i sees the committed keys 0 .. L - S - 1 and the new keys of its ancestors and itself
(a reading: the pages give no mask; a chain of parents j - 1 is the causal case).
"""
from __future__ import annotations

from typing import Iterable, Optional

import numpy as np


def gather_rows(pool: np.ndarray, block_table_row: np.ndarray, length: int, page_size: int) -> np.ndarray:
    """Paged addressing: token j of a sequence is ``pool[bt[j // page], j % page]``.

    The Perplexity post ("Lower latency and higher throughput with multi-node
    DeepSeek deployment", section "Слой MLA") runs MLA over a paged cache with
    a flexible page table; this is that lookup, one page at a time.
    """
    rows = np.empty((length, pool.shape[-1]), dtype=np.float64)
    for j0 in range(0, length, page_size):  # one page at a time: tokens j0 .. j0+count-1
        count = min(page_size, length - j0)
        rows[j0:j0 + count] = pool[int(block_table_row[j0 // page_size]), :count]
    return rows


def visible_keys(L: int, S: int, i: int, causal: bool) -> int:
    """Keys visible to query token i of S, with L tokens cached (S new ones included)."""
    n = L - S + i + 1 if causal else L
    return max(0, min(L, n))


def tree_ancestors(parents) -> np.ndarray:
    """A[i, j] is true iff node j is node i or one of its ancestors, walking parent links."""
    parents = np.asarray(parents, dtype=np.int64)
    S = parents.shape[0]
    A = np.zeros((S, S), dtype=bool)
    for i in range(S):
        j = i
        while j >= 0:
            A[i, j] = True
            p = int(parents[j])
            if not -1 <= p < j:
                raise ValueError(f"parent of node {j} is {p}: must be in [-1, {j})")
            j = p
    return A


def visible_key_index(L: int, S: int, i: int, causal: bool, ancestors: Optional[np.ndarray] = None):
    """The keys query token i of S sees, as an index into the sequence's rows.  Without a tree:
    the first ``visible_keys`` ones (a slice, so rows are views, not copies).  With a tree
    (``ancestors`` from ``tree_ancestors``): an index array of the committed keys and the new keys
    of node i's ancestors and itself."""
    if ancestors is None:
        return slice(0, visible_keys(L, S, i, causal))
    base = L - S
    new = [base + j for j in range(S) if ancestors[i, j] and base + j >= 0]
    return np.concatenate([np.arange(max(base, 0)), np.asarray(new, dtype=np.int64)]).astype(np.int64)


def _softmax_stats(z: np.ndarray):
    """Exact two-pass softmax of one logit row: (p, lse)."""
    if z.size == 0:
        return z, -np.inf
    m = np.max(z)
    w = np.exp(z - m)
    lsum = np.sum(w)
    return w / lsum, m + np.log(lsum)


def mla_decode_nonabsorbed(q_nope, q_pe, w_uk, w_uv, pool, block_table, seq_lens, *, softmax_scale: float,
                           page_size: int = 64, causal: bool = True,
                           seqs: Optional[Iterable[int]] = None, heads: Optional[Iterable[int]] = None,
                           return_probs: bool = False, tree=None):
    """Reference decode, non-absorbed order, fp64.

    Shapes: q_nope (B,S,H,d_h), q_pe (B,S,H,d_R), w_uk / w_uv (H,d_c,d_h),
    pool (P,page,d_c+d_R), block_table (B,max_pages), seq_lens (B,).

    For each sequence b and head h (the "order 1" steps of the absorption note,
    §二.1 and §三.1): K = C_b W_UK[h], V = C_b W_UV[h]; logits
    z_j = scale·(q_nope·K_j + q_pe·R_j) for the visible keys; exact softmax;
    out = Σ p_j V_j.  ``o_lat`` = Σ p_j C_j is the latent-space output the
    attention call returns (same p).  Entries outside ``seqs``×``heads`` stay
    NaN.  ``tree`` (B,S) parent indices switch to the tree mask (``causal`` is
    then ignored).  Returns a dict with o_lat (B,S,H,d_c), lse (B,S,H),
    out (B,S,H,d_h) and, if asked, probs[(b,i,h)] = p.
    """
    q_nope = np.asarray(q_nope, dtype=np.float64)
    q_pe = np.asarray(q_pe, dtype=np.float64)
    B, S, H, Dh = q_nope.shape
    Dc = w_uk.shape[1]
    Dv = w_uv.shape[2]
    o_lat = np.full((B, S, H, Dc), np.nan)
    lse = np.full((B, S, H), np.nan)
    out = np.full((B, S, H, Dv), np.nan)
    probs = {}
    seqs = range(B) if seqs is None else list(seqs)
    heads = range(H) if heads is None else list(heads)
    for b in seqs:
        L = int(seq_lens[b])
        rows = gather_rows(pool, block_table[b], L, page_size)
        C, R = rows[:, :Dc], rows[:, Dc:]
        anc = None if tree is None else tree_ancestors(tree[b])
        for h in heads:
            K = C @ np.asarray(w_uk[h], dtype=np.float64)  # (L, d_h)  k_nope of every cached token
            V = C @ np.asarray(w_uv[h], dtype=np.float64)  # (L, d_h)  v of every cached token
            for i in range(S):
                idx = visible_key_index(L, S, i, causal, anc)
                n = idx.stop if isinstance(idx, slice) else idx.size
                z = softmax_scale * (K[idx] @ q_nope[b, i, h] + R[idx] @ q_pe[b, i, h])
                p, lse[b, i, h] = _softmax_stats(z)
                out[b, i, h] = p @ V[idx] if n else 0.0
                o_lat[b, i, h] = p @ C[idx] if n else 0.0
                if return_probs:
                    probs[(b, i, h)] = p
    res = {"o_lat": o_lat, "lse": lse, "out": out}
    if return_probs:
        res["probs"] = probs
    return res


def absorb_q_reference(q_nope, w_uk):
    """q_lat[b,s,h,c] = Σ_d W_UK[h,c,d]·q_nope[b,s,h,d] (W_UK applied transposed to q).

    izhida answer "专家": apply W_K transposed to q so K is never computed;
    "【笔记】MLA矩阵吸收分析" §二.2, step 2 (shape (b,s,h,k)).
    """
    q = np.asarray(q_nope, dtype=np.float64)
    w = np.asarray(w_uk, dtype=np.float64)
    B, S, H, Dh = q.shape
    out = np.empty((B, S, H, w.shape[1]))
    for h in range(H):
        out[:, :, h, :] = q[:, :, h, :] @ w[h].T
    return out


def out_proj_reference(o_lat, w_uv):
    """out[b,s,h,v] = Σ_c o_lat[b,s,h,c]·W_UV[h,c,v] (W_UV applied after attention).

    izhida answer "专家": apply W_V after the latent attention-weighted average;
    "【笔记】MLA矩阵吸收分析" §三.2, step 2 (shape (b,h,s,v)).
    """
    o = np.asarray(o_lat, dtype=np.float64)
    w = np.asarray(w_uv, dtype=np.float64)
    B, S, H, Dc = o.shape
    out = np.empty((B, S, H, w.shape[2]))
    for h in range(H):
        out[:, :, h, :] = o[:, :, h, :] @ w[h]
    return out


def latent_attention_reference(q_lat, q_pe, pool, block_table, seq_lens, *, softmax_scale: float,
                               page_size: int = 64, causal: bool = True,
                               seqs: Optional[Iterable[int]] = None, tree=None):
    """What the attention call computes from an already-absorbed query, fp64.

    Logit of head h against cached token j: scale·(q_lat·c_j + q_pe·k_pe_j),
    the latent c_j serving as the key and (below) as the value of every head
    — izhida answer "DeepSeek" (each head takes a weighted sum over the
    512-d latent; the RoPE inner product is 64-d) and answer "专家".  ``tree``
    as in ``mla_decode_nonabsorbed``.  Returns o_lat (B,S,H,d_c) = Σ_j p_j c_j
    and lse (B,S,H).
    """
    q_lat = np.asarray(q_lat, dtype=np.float64)
    q_pe = np.asarray(q_pe, dtype=np.float64)
    B, S, H, Dc = q_lat.shape
    o_lat = np.full((B, S, H, Dc), np.nan)
    lse = np.full((B, S, H), np.nan)
    for b in (range(B) if seqs is None else seqs):
        L = int(seq_lens[b])
        rows = gather_rows(pool, block_table[b], L, page_size)
        C, R = rows[:, :Dc], rows[:, Dc:]
        anc = None if tree is None else tree_ancestors(tree[b])
        for i in range(S):
            idx = visible_key_index(L, S, i, causal, anc)
            n = idx.stop if isinstance(idx, slice) else idx.size
            Z = softmax_scale * (C[idx] @ q_lat[b, i].T + R[idx] @ q_pe[b, i].T)  # (n, H): one column per head
            for h in range(H):
                p, lse[b, i, h] = _softmax_stats(Z[:, h])
                o_lat[b, i, h] = p @ C[idx] if n else 0.0
    return {"o_lat": o_lat, "lse": lse}


def softmax_mass(q_lat, q_pe, pool, block_table, seq_lens, lse, rows, *, softmax_scale: float,
                 page_size: int = 64, causal: bool = True, tree=None):
    """For each (b, i, h) in ``rows``: the sum over the keys that query sees of exp(z_j - lse[b,i,h]),
    with z_j = scale·(q_lat·c_j + q_pe·k_pe_j) computed here in fp64.

    The attention output is an attention-weighted average (izhida answer "专家"), so its weights
    e^{z_j - lse} sum to one exactly when ``lse`` is the log of their normaliser.  Handed an lse
    from elsewhere, this returns how far its weights are from summing to one.  Rows whose key set
    is empty give NaN (no weights; lse is -inf there).  ``tree`` as in ``mla_decode_nonabsorbed``.
    """
    q_lat = np.asarray(q_lat, dtype=np.float64)
    q_pe = np.asarray(q_pe, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    B, S, H, Dc = q_lat.shape
    mass = np.full(len(rows), np.nan)
    by_seq = {}
    for k, (b, i, h) in enumerate(rows):
        by_seq.setdefault(int(b), []).append((k, int(i), int(h)))
    for b, items in by_seq.items():
        L = int(seq_lens[b])
        data = gather_rows(pool, block_table[b], L, page_size)
        C, R = data[:, :Dc], data[:, Dc:]
        anc = None if tree is None else tree_ancestors(tree[b])
        for k, i, h in items:
            idx = visible_key_index(L, S, i, causal, anc)
            n = idx.stop if isinstance(idx, slice) else idx.size
            if n == 0:
                continue
            z = softmax_scale * (C[idx] @ q_lat[b, i, h] + R[idx] @ q_pe[b, i, h])
            mass[k] = np.sum(np.exp(z - lse[b, i, h]))
    return mass


def o_proj_reference(out, w_o):
    """y[b,s,e] = sum over heads h and value dims v of out[b,s,h,v] W_O[h,v,e], fp64.

    The output projection after the path: "【笔记】MLA矩阵吸收分析" §三.1 / §三.2, step 3 (W_O of shape
    (n_heads x v_head_dim, dim) -> (h, v, e)), summed over the heads as the FLOP count 2bhsev of
    the same steps implies.  ``w_o`` is (H, d_v, e).
    """
    o = np.asarray(out, dtype=np.float64)
    B, S, H, V = o.shape
    w = np.asarray(w_o, dtype=np.float64).reshape(H * V, -1)
    return (o.reshape(B * S, H * V) @ w).reshape(B, S, -1)
