"""Pins of the fp64 oracle of the step before the path (projection, RoPE, AppendKV).

* the projection equals torch.matmul in fp64 (a library routine); a transposed weight fails;
* RoPE (RoFormer's rotation, a reading: the pages give no formula) against an independent
  formulation: each pair as a complex number times e^{i theta} (numpy complex arithmetic); the
  closed forms of a hand-worked 4-wide example; position 0 is the identity; norms are kept;
  rotations compose (pos m then n = pos m + n); scores depend on positions only through their
  difference;
* AppendKV: reading the sequences back through the page table returns the new rows at the last S
  positions, every other slot of the pool is unchanged bit for bit, and tokens at negative
  positions (L < S) are not written.
"""
import math

import numpy as np
import pytest
import torch

from oracle import mla_decode as dec
from oracle import mla_prepare as ref


def test_linear_is_matmul():
    rng = np.random.default_rng(1)
    x, w = rng.standard_normal((5, 7)), rng.standard_normal((7, 3))
    np.testing.assert_allclose(ref.linear_reference(x, w), (torch.from_numpy(x) @ torch.from_numpy(w)).numpy(),
                               rtol=1e-13, atol=1e-13)
    with pytest.raises(ValueError):
        ref.linear_reference(x, w.T)


def test_rope_against_complex_rotation():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, 4, 64))
    pos = np.array([0, 5, 4095])
    got = ref.rope_reference(x, pos)
    z = x[..., 0::2] + 1j * x[..., 1::2]
    freq = 10000.0 ** (-np.arange(32) * 2.0 / 64.0)
    want = z * np.exp(1j * pos[:, None, None] * freq)
    np.testing.assert_allclose(got[..., 0::2], want.real, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(got[..., 1::2], want.imag, rtol=1e-12, atol=1e-12)


def test_rope_hand_worked_example():
    """d = 4, base 10000: pair 0 turns by pos, pair 1 by pos / 100 (10000^(2/4) = 100)."""
    x = np.array([1.0, 0.0, 1.0, 0.0])
    got = ref.rope_reference(x, 1.0)
    np.testing.assert_allclose(got, [math.cos(1), math.sin(1), math.cos(0.01), math.sin(0.01)], rtol=0, atol=1e-15)
    got = ref.rope_reference(np.array([0.0, 2.0]), math.pi / 2)  # d = 2: one pair, angle = pos
    np.testing.assert_allclose(got, [-2.0, 0.0], atol=1e-15)


def test_rope_invariants():
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    np.testing.assert_array_equal(ref.rope_reference(q, 0), q)
    r = ref.rope_reference(q, 1234)
    np.testing.assert_allclose(np.hypot(r[0::2], r[1::2]), np.hypot(q[0::2], q[1::2]), rtol=1e-12)
    np.testing.assert_allclose(ref.rope_reference(ref.rope_reference(q, 300), 77), ref.rope_reference(q, 377),
                               rtol=1e-10, atol=1e-10)
    s1 = ref.rope_reference(q, 900) @ ref.rope_reference(k, 100)
    s2 = ref.rope_reference(q, 5800) @ ref.rope_reference(k, 5000)
    assert abs(s1 - s2) < 1e-9


def _paged(seed, lens, page=4, row=6):
    rng = np.random.default_rng(seed)
    npg = [-(-int(L) // page) for L in lens]
    P = sum(npg) + 2  # two spare pages no sequence owns
    order = rng.permutation(P)
    bt = np.full((len(lens), max(npg)), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(npg):
        bt[b, :n] = order[off:off + n]
        off += n
    return rng.standard_normal((P, page, row)), bt


def test_append_writes_the_last_positions_only():
    lens = np.array([9, 4, 13])
    S = 3
    pool, bt = _paged(4, lens)
    rng = np.random.default_rng(5)
    c, k = rng.standard_normal((3, S, 4)), rng.standard_normal((3, S, 2))
    out = ref.append_kv_reference(pool, bt, lens, c, k, page_size=4)
    touched = np.zeros(pool.shape[:2], dtype=bool)
    for b, L in enumerate(lens):
        rows = dec.gather_rows(out, bt[b], int(L), 4)
        np.testing.assert_array_equal(rows[L - S:, :4], c[b])
        np.testing.assert_array_equal(rows[L - S:, 4:], k[b])
        for j in range(L - S, L):
            touched[bt[b, j // 4], j % 4] = True
    np.testing.assert_array_equal(out[~touched], pool[~touched])


def test_append_skips_negative_positions():
    lens = np.array([2])
    pool, bt = _paged(6, lens)
    c, k = np.ones((1, 3, 4)), np.ones((1, 3, 2))
    out = ref.append_kv_reference(pool, bt, lens, c, k, page_size=4)
    rows = dec.gather_rows(out, bt[0], 2, 4)
    np.testing.assert_array_equal(rows, np.ones((2, 6)))  # tokens 1 and 2 of 3 land at positions 0, 1
    mask = np.ones(pool.shape[:2], dtype=bool)
    mask[bt[0, 0], :2] = False
    np.testing.assert_array_equal(out[mask], pool[mask])


def test_planted_mistake_is_caught(monkeypatch):
    """A frequency exponent without the factor 2, put into the oracle, fails the hand-worked pin."""
    good = ref.rope_angles
    monkeypatch.setattr(ref, "rope_angles",
                        lambda pos, dim=64, base=10000.0: good(pos, dim, base) ** 0 * np.asarray(pos, dtype=np.float64)[..., None]
                        * base ** (-np.arange(0, dim, 2, dtype=np.float64) / (2 * dim)))
    got = ref.rope_reference(np.array([1.0, 0.0, 1.0, 0.0]), 1.0)
    assert not np.allclose(got, [math.cos(1), math.sin(1), math.cos(0.01), math.sin(0.01)], atol=1e-6)
