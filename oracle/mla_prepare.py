"""fp64 CPU reference of the step that produces the path's inputs — TEST INFRASTRUCTURE (see
``oracle/__init__``).

The Perplexity post ("Lower latency and higher throughput with multi-node DeepSeek deployment")
lists the stage before attention as InputNorm, QKVProj, AppendKV, BMM (section "Наложение
вычислений и взаимодействия") and fuses q_a_proj and kv_a_proj into one projection qkv_a_proj
(section "Слой MLA").  The absorption note ("【笔记】MLA矩阵吸收分析", §二.1) names the shapes: the
hidden state is compressed to c^Q (q_lora_rank) and c^KV (kv_lora_rank).  Three definitions:

* ``linear_reference``      y = x W: the fused a-projection (and any other plain projection, such
                            as W_UQ, in the same form);
* ``rope_reference``        rotary position embedding of a 64-wide vector at a position;
* ``append_kv_reference``   the new tokens' [c_KV | rotated k_pe] rows written into the paged cache.

Readings (the pages are silent; each is listed in the design notes): the fused projection's
output is [c^Q | c^KV | k_pe before rotation] in that order; the normalisations between the
projection and the cache (InputNorm and the latent norms) are outside; RoPE is the rotation of
Su et al. (RoFormer): consecutive pairs (2i, 2i+1) of the vector turn by the angle
pos * base^(-2i/d), base 10000; the S new tokens of a sequence with L cached tokens (the S
included) sit at positions L - S .. L - 1.
"""
from __future__ import annotations

import numpy as np


def linear_reference(x, w):
    """y[t, n] = sum_k x[t, k] w[k, n] in fp64 (a library matmul as the one step)."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64)


def rope_angles(pos, dim: int = 64, base: float = 10000.0):
    """theta[..., i] = pos * base^(-2i/dim) for i < dim/2."""
    inv = base ** (-np.arange(0, dim, 2, dtype=np.float64) / dim)
    return np.asarray(pos, dtype=np.float64)[..., None] * inv


def rope_reference(x, pos, base: float = 10000.0):
    """Rotate each consecutive pair (x[2i], x[2i+1]) of the last axis by pos * base^(-2i/d).

    ``pos`` broadcasts against x's leading axes (one position per vector)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    th = rope_angles(pos, d, base)
    c, s = np.cos(th), np.sin(th)
    while c.ndim < x.ndim:  # positions given for leading axes only: broadcast over the rest
        c, s = c[..., None, :], s[..., None, :]
    c = np.broadcast_to(c, x.shape[:-1] + (d // 2,))
    s = np.broadcast_to(s, x.shape[:-1] + (d // 2,))
    even, odd = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = even * c - odd * s
    out[..., 1::2] = even * s + odd * c
    return out


def new_token_positions(seq_lens, q_len: int):
    """Positions (B, S) of the S new tokens: L_b - S + i."""
    L = np.asarray(seq_lens, dtype=np.int64)
    return L[:, None] - q_len + np.arange(q_len)[None, :]


def append_kv_reference(pool, block_table, seq_lens, c_kv, k_pe_rot, *, page_size: int = 64):
    """A copy of ``pool`` with token pos of sequence b, for each new token (b, i), set to
    [c_kv[b, i] | k_pe_rot[b, i]] at page block_table[b][pos // page], slot pos % page.
    Tokens at negative positions (a sequence shorter than S) are not written."""
    out = np.array(pool, dtype=np.float64, copy=True)
    B, S = c_kv.shape[:2]
    pos = new_token_positions(seq_lens, S)
    for b in range(B):
        for i in range(S):
            p = int(pos[b, i])
            if p < 0:
                continue
            page = int(block_table[b, p // page_size])
            out[page, p % page_size, :c_kv.shape[-1]] = c_kv[b, i]
            out[page, p % page_size, c_kv.shape[-1]:] = k_pe_rot[b, i]
    return out
