"""The seeded input generator: reproducibility, bf16 rounding, page-table structure, sizes."""
import numpy as np
import pytest
import torch

from deepseek_mla_latent_amd import inputs as gen


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1e-40, np.inf, -np.inf], np.float32)])
    # exact ties: halfway between two bf16 values, both parities of the kept LSB
    ties = (np.arange(1, 200, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties])
    ours = gen.round_to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, theirs)
    back = gen.bf16_bits_to_f32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())
    assert gen.round_to_bf16_bits(np.array([np.nan], np.float32))[0] == 0x7FC0


def test_reproducible_and_seed_dependent():
    w = gen.small_workload(3, 2, ragged=(10, 300), dtype="bf16", paged=True)
    a, b, c = gen.generate(w, 5), gen.generate(w, 5), gen.generate(w, 6)
    for name in ("seq_lens", "block_table", "pool", "q_nope", "q_pe", "w_uk", "w_uv"):
        np.testing.assert_array_equal(getattr(a, name), getattr(b, name))
    assert not np.array_equal(a.q_nope, c.q_nope)


def test_block_table_is_a_bijection_onto_the_pool():
    w = gen.small_workload(7, 1, ragged=(1, 500), dtype="bf16", paged=True)
    x = gen.generate(w, 3)
    pages = -(-x.seq_lens.astype(int) // 64)
    used = np.concatenate([x.block_table[b, :pages[b]] for b in range(7)])
    assert sorted(used.tolist()) == list(range(x.num_pages))
    assert np.all(x.block_table[np.arange(x.block_table.shape[1])[None, :] >= pages[:, None]] == -1)
    assert not np.array_equal(used, np.arange(x.num_pages))  # actually permuted


def test_contiguous_is_identity_table():
    w = gen.small_workload(3, 1, cache_len=200, dtype="bf16", paged=False)
    x = gen.generate(w, 1)
    assert np.array_equal(x.block_table.reshape(-1), np.arange(12))


def test_poison_marks_exactly_the_unused_slots():
    w = gen.small_workload(3, 1, ragged=(1, 200), dtype="bf16", paged=True)
    x = gen.generate(w, 4, poison_unused=True)
    f = x.f32("pool")
    for b in range(3):
        rows = x.sequence_rows(b)
        assert np.all(np.isfinite(rows))
    finite_rows = np.isfinite(f).all(-1).sum()
    assert finite_rows == int(x.seq_lens.sum())
    assert np.isnan(f).all(-1).sum() == f.shape[0] * 64 - int(x.seq_lens.sum())


def test_weight_and_value_statistics():
    w = gen.small_workload(4, 1, cache_len=256, dtype="f32", paged=False)
    x = gen.generate(w, 2)
    assert abs(x.w_uk.var() * 512 - 1) < 0.02 and abs(x.w_uv.var() * 512 - 1) < 0.02
    assert abs(x.pool.var() - 1) < 0.02 and abs(x.q_nope.var() - 1) < 0.05


def test_named_workload_shapes():
    """Sizes of the five workloads, from their definitions (pages computed without drawing pools)."""
    W = gen.WORKLOADS
    assert W["tiny_fp32"].dtype == "f32" and W["tiny_fp32"].cache_len == 512
    c2 = W["b32_t4096"]
    assert (c2.batch, c2.q_len, c2.cache_len, c2.dtype) == (32, 1, 4096, "bf16")
    assert c2.batch * c2.cache_len // 64 == 2048
    c4 = W["mtp_b64_s2_t16384"]
    assert (c4.batch, c4.q_len, c4.cache_len) == (64, 2, 16386)
    assert c4.batch * (-(-c4.cache_len // 64)) == 16448
    c5 = W["long_b4_t131072"]
    assert c5.batch * c5.cache_len * 576 * 2 == 603979776
    assert c5.batch * c5.cache_len // 64 == 8192
    assert abs(c2.softmax_scale - 192 ** -0.5) < 1e-15


def test_tiny_named_workload_generates():
    x = gen.generate_named("tiny_fp32")
    assert x.pool.shape == (8, 64, 576) and x.pool.dtype == np.float32
    assert x.q_nope.shape == (1, 1, 128, 128) and x.w_uk.shape == (128, 512, 128)
    assert np.array_equal(x.seq_lens, [512])


@pytest.mark.parametrize("lens", [[0, 5], [64, 65], [1, 128]])
def test_explicit_lengths(lens):
    w = gen.small_workload(2, 1, cache_len=1, dtype="bf16", paged=True)
    x = gen.generate(w, 9, seq_lens=lens, poison_unused=True)
    assert list(x.seq_lens) == lens
    assert x.num_pages == sum(-(-L // 64) for L in lens) or x.num_pages == 1
