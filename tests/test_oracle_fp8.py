"""Pins of the FP8 block-quantisation oracle.

* E4M3 rounding equals torch's float8_e4m3fn conversion (a library routine) on a dense grid,
  random values and every tie; the 254 finite codes decode to torch's values and encode back;
* quantisation: the block maximum maps to +-448, every value is within half a spacing;
* with operands built from E4M3 values and block maxima of 448 * 2^k (so every scale is a power of
  two and every code exact), both FP8 products equal the exact fp64 products (closed form), with
  different scales per block so a scale applied to the wrong block fails;
* on N(0,1) data the FP8 products stay within a few percent of the unquantised ones;
* a planted block size of 64 breaks the exact-product pin.
"""
import numpy as np
import pytest
import torch

from oracle import fp8
from oracle import mla_decode as dec


def _torch_e4m3(v):
    return torch.from_numpy(np.asarray(v, dtype=np.float32)).to(torch.float8_e4m3fn).float().numpy()


def test_rounding_matches_torch():
    grid = np.linspace(-464, 464, 200001, dtype=np.float32)
    small = np.linspace(-0.05, 0.05, 100001, dtype=np.float32)
    rnd = np.random.default_rng(1).standard_normal(100000).astype(np.float32) * 50
    values = fp8.e4m3_decode(np.arange(256, dtype=np.uint8))
    finite = values[np.isfinite(values)]
    s = np.sort(np.unique(finite))
    ties = ((s[1:] + s[:-1]) / 2).astype(np.float32)  # exact midpoints (all representable in fp32)
    for v in (grid, small, rnd, ties, finite.astype(np.float32)):
        np.testing.assert_array_equal(fp8.e4m3_round(v), _torch_e4m3(v))


def test_codes_decode_and_encode():
    codes = np.arange(256, dtype=np.uint8)
    vals = fp8.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    np.testing.assert_array_equal(np.isnan(vals), np.isnan(ref))
    fin = ~np.isnan(vals)
    np.testing.assert_array_equal(vals[fin], ref[fin])
    assert np.nanmax(vals) == 448.0 and np.sum(np.isnan(vals)) == 2
    keep = fin & ~((codes == 128))  # -0 encodes as +0's magnitude with the sign bit: compare values
    np.testing.assert_array_equal(fp8.e4m3_decode(fp8.e4m3_encode(vals[keep])), vals[keep])


def test_quantize_properties():
    x = np.random.default_rng(2).standard_normal((256, 384)).astype(np.float32)
    q, s = fp8.quantize(x, (128, 128))
    assert s.shape == (2, 3)
    for i in range(2):
        for j in range(3):
            blk = x[128 * i:128 * (i + 1), 128 * j:128 * (j + 1)]
            qb = q[128 * i:128 * (i + 1), 128 * j:128 * (j + 1)]
            assert np.max(np.abs(qb)) == 448.0
            a = np.abs(blk / s[i, j]).astype(np.float64)
            e = np.frexp(np.maximum(a, 2.0 ** -6))[1] - 1.0
            assert np.all(np.abs(blk / s[i, j] - qb) <= 2.0 ** (e - 4) + 1e-12)
    z, zs = fp8.quantize(np.zeros((128, 128), np.float32), (128, 128))
    assert np.all(z == 0) and np.all(zs == 0)


def _exact_operands(rng, shape, blocks, exps):
    """E4M3 values with each block's maximum |value| = 448 * 2^k (k from `exps`, one per block)."""
    vals = fp8.e4m3_decode(np.arange(256, dtype=np.uint8))
    vals = vals[np.isfinite(vals)]
    x = rng.choice(vals, size=shape).astype(np.float64)
    it = iter(exps)
    idx = [range(0, shape[i], blocks[i] or shape[i]) for i in range(len(shape))]
    for start in np.ndindex(*[len(r) for r in idx]):
        sl = tuple(slice(idx[i][start[i]], idx[i][start[i]] + (blocks[i] or shape[i])) for i in range(len(shape)))
        k = next(it)
        blk = x[sl]
        blk.flat[0] = 448.0
        x[sl] = blk * 2.0 ** k
    return x.astype(np.float32)


def test_exact_products_with_power_of_two_scales():
    rng = np.random.default_rng(3)
    H = 2
    w_uk = _exact_operands(rng, (H, 512, 128), (1, 128, 128), [-12, -9, -10, -11, -8, -13, -9, -10])
    w_uv = _exact_operands(rng, (H, 512, 128), (1, 128, 128), [-9, -11, -10, -12, -13, -8, -10, -9])
    q = _exact_operands(rng, (3 * H, 128), (1, 128), [-3, -5, -4, -6, -2, -7]).reshape(3, 1, H, 128)
    o = _exact_operands(rng, (3 * H, 512), (1, 128), list(rng.integers(-8, -2, size=3 * H * 4))).reshape(3, 1, H, 512)
    got, _, _ = fp8.absorb_q_fp8_reference(q, w_uk)
    np.testing.assert_array_equal(got, dec.absorb_q_reference(q, w_uk))
    got, _, _ = fp8.out_proj_fp8_reference(o, w_uv)
    np.testing.assert_array_equal(got, dec.out_proj_reference(o, w_uv))


def test_quantised_products_track_the_unquantised_ones():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((4, 1, 8, 128)).astype(np.float32)
    o = rng.standard_normal((4, 1, 8, 512)).astype(np.float32)
    w = (rng.standard_normal((8, 512, 128)) / np.sqrt(512)).astype(np.float32)
    for got, want in ((fp8.absorb_q_fp8_reference(q, w)[0], dec.absorb_q_reference(q, w)),
                      (fp8.out_proj_fp8_reference(o, w)[0], dec.out_proj_reference(o, w))):
        err = np.max(np.abs(got - want)) / np.max(np.abs(want))
        assert 1e-4 < err < 0.05


def test_planted_block_size_is_caught(monkeypatch):
    rng = np.random.default_rng(5)
    w_uk = _exact_operands(rng, (1, 512, 128), (1, 128, 128), [-12, -9, -10, -11])
    q = _exact_operands(rng, (2, 128), (1, 128), [-3, -5]).reshape(2, 1, 1, 128)
    monkeypatch.setattr(fp8, "BLOCK", 64)
    got, _, _ = fp8.absorb_q_fp8_reference(q, w_uk)
    assert not np.array_equal(got, dec.absorb_q_reference(q, w_uk))
