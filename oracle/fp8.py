"""FP8 block quantisation and the two per-head products in FP8 — TEST INFRASTRUCTURE (see
``oracle/__init__``).

The Perplexity post ("Lower latency and higher throughput with multi-node DeepSeek deployment")
describes the scheme (section "Квантование"): weights are quantised statically with one scale per
128 x 128 block, activations on the fly with one scale per 128-element vector along the reduction
dimension K (an (M, K) x (K, N) product needs (M x ceil(K/128)) activation scales and
(ceil(K/128) x ceil(N/128)) weight scales); its k_b_proj / v_b_proj products (W_UK and W_UV) run
as an FP8 block-quantised batched matmul (section "Слой MLA").

Readings (the pages name the scheme, not the format or the rounding; each listed in the design
notes): FP8 is E4M3 (4 exponent bits, bias 7, 3 mantissa bits, no infinities, largest finite
448); a block's scale is amax / 448 computed in fp32; a value x is coded as x * (448 / amax)
(the factor an fp32 division, the product an fp32 multiplication) rounded to the nearest E4M3
value, ties to even; an all-zero block has codes 0.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
BLOCK = 128


def e4m3_round(v):
    """Nearest E4M3 value (ties to even) of fp32 values with |v| <= 464, as float32.

    Normal numbers 2^e (1 + m/8) have spacing 2^(e-3); below 2^-6 the spacing is 2^-9.
    Rounding to that spacing is exact in fp32 (a power-of-two scaling and np.rint)."""
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v).astype(np.float64)
    e = np.frexp(np.where(a > 0, a, 1.0))[1] - 1.0  # a = 2^e * [1, 2)
    spacing = np.where(a >= 2.0 ** -6, 2.0 ** (e - 3), 2.0 ** -9)
    q = np.rint(v.astype(np.float64) / spacing) * spacing
    return np.clip(q, -E4M3_MAX, E4M3_MAX).astype(np.float32)


def e4m3_encode(q):
    """8-bit codes of exactly representable E4M3 values."""
    q = np.asarray(q, dtype=np.float64)
    sign = (np.signbit(q)).astype(np.uint8) << 7
    a = np.abs(q)
    normal = a >= 2.0 ** -6
    e = np.frexp(np.where(normal, a, 1.0))[1] - 1.0
    exp_field = np.where(normal, e + 7, 0).astype(np.uint8)
    man = np.where(normal, (a / 2.0 ** e - 1.0) * 8.0, a / 2.0 ** -9)
    assert np.all(man == np.rint(man)), "value not representable"
    return sign | (exp_field << 3) | man.astype(np.uint8)


def e4m3_decode(code):
    """Value of 8-bit E4M3 codes (NaN for S.1111.111)."""
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    s = np.where(c >> 7, -1.0, 1.0)
    E, M = (c >> 3) & 15, c & 7
    v = np.where(E == 0, M * 2.0 ** -9, (1.0 + M / 8.0) * 2.0 ** (E - 7.0))
    v = np.where((E == 15) & (M == 7), np.nan, v)
    return s * v


def quantize(x, axis_blocks):
    """Block quantisation: ``x`` (fp32) is cut into blocks whose extent along each axis is given
    by ``axis_blocks`` (None = the whole axis); returns (code values, scales per block) with
    x ~= code value * scale of its block."""
    x = np.asarray(x, dtype=np.float32)
    shape = x.shape
    bs = [shape[i] if b is None else b for i, b in enumerate(axis_blocks)]
    nb = [shape[i] // bs[i] for i in range(len(shape))]
    # (n0, b0, n1, b1, ...)
    xr = x.reshape([v for i in range(len(shape)) for v in (nb[i], bs[i])])
    red = tuple(2 * i + 1 for i in range(len(shape)))
    amax = np.max(np.abs(xr), axis=red, keepdims=True).astype(np.float32)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    factor = (np.float32(E4M3_MAX) / np.where(amax > 0, amax, np.float32(1.0))).astype(np.float32)
    codes = e4m3_round((xr * factor).astype(np.float32))  # an fp32 product, then E4M3 rounding
    codes = np.where(amax > 0, codes, np.float32(0.0))
    return codes.reshape(shape), np.squeeze(scale, axis=red).astype(np.float32)


def absorb_q_fp8_reference(q_nope, w_uk):
    """q_lat[n,h,c] = sum_d W_UK[h,c,d] q_nope[n,h,d] with both operands block quantised.

    Reduction K = d (128: one block).  Weight W_UK[h] (c x d): blocks of 128 c x 128 d.
    Activation q_nope[n,h,:]: one vector of 128.  Products of the codes are summed per block in
    fp64 and multiplied by the two scales.  Returns (q_lat, weight codes, weight scales)."""
    q = np.asarray(q_nope, dtype=np.float32)
    B, S, H, D = q.shape
    wq, ws = quantize(w_uk, (1, BLOCK, BLOCK))  # ws: (H, C/128, 1): per head, 128 x 128 blocks
    qq, qs = quantize(q.reshape(B * S, H, D), (1, 1, BLOCK))  # qs: (T, H, 1)
    C = w_uk.shape[1]
    out = np.empty((B * S, H, C))
    for h in range(H):
        acc = qq[:, h, :].astype(np.float64) @ wq[h].astype(np.float64).T  # (T, C)
        scale = qs[:, h, 0][:, None].astype(np.float64) * np.repeat(ws[h, :, 0], BLOCK)[None, :].astype(np.float64)
        out[:, h, :] = acc * scale
    return out.reshape(B, S, H, C), wq, ws


def out_proj_fp8_reference(o_lat, w_uv):
    """out[n,h,v] = sum_c o_lat[n,h,c] W_UV[h,c,v] with both operands block quantised.

    Reduction K = c (512: four blocks).  Weight W_UV[h] (c x v): blocks of 128 c x 128 v.
    Activation o_lat[n,h,:]: four vectors of 128 along c.  Each block's sum of code products
    is multiplied by its activation and weight scale, then the blocks are added."""
    o = np.asarray(o_lat, dtype=np.float32)
    B, S, H, C = o.shape
    wq, ws = quantize(w_uv, (1, BLOCK, BLOCK))  # ws: (H, C/128, V/128)
    oq, os_ = quantize(o.reshape(B * S, H, C), (1, 1, BLOCK))  # os_: (T, H, C/128)
    V = w_uv.shape[2]
    out = np.zeros((B * S, H, V))
    for h in range(H):
        for kb in range(C // BLOCK):
            sl = slice(kb * BLOCK, (kb + 1) * BLOCK)
            acc = oq[:, h, sl].astype(np.float64) @ wq[h, sl, :].astype(np.float64)  # (T, V)
            out[:, h, :] += acc * (os_[:, h, kb][:, None].astype(np.float64) * np.float64(ws[h, kb, 0]))
    return out.reshape(B, S, H, V), wq, ws
