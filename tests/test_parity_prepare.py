"""GPU parity of the step before the path (mla_linear, mla_rope_append) against the fp64 oracle.

Bar: max |gpu - ref| / max |ref| <= 2e-2 per output (bf16 operands and outputs, fp32 arithmetic);
the c_KV copy and every untouched pool slot are checked bit for bit (unused slots are NaN).
"""
import math

import numpy as np
import pytest

from deepseek_mla_latent_amd import binding
from deepseek_mla_latent_amd import inputs as gen
from oracle import mla_decode as dec
from oracle import mla_prepare as ref
from tests.helpers import BF16_TOL, params_for, rel_err, to_device, to_host

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def _bf16_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _linear(x_bits, w_bits, m, k, n):
    import torch
    x, w = _bf16_dev(x_bits), _bf16_dev(w_bits)
    y = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws_bytes = binding.mla_linear_workspace_bytes(m, k, n)
    ws = torch.empty(max(ws_bytes, 16) // 4, dtype=torch.float32, device="cuda") if ws_bytes else None
    binding.mla_linear(x, w, y, m, k, n, ws)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("m,k,n", [(32, 7168, 2112), (1, 512, 128), (100, 1536, 256), (600, 1024, 192),
                                   (33, 576, 64)])
def test_linear(m, k, n):
    say("linear", m, k, n)
    rng = np.random.default_rng(m * 7 + k + n)
    x = gen.round_to_bf16_bits(rng.standard_normal((m, k), dtype=np.float32))
    w = gen.round_to_bf16_bits(rng.standard_normal((k, n), dtype=np.float32) / np.float32(math.sqrt(k)))
    y = to_host(_linear(x, w, m, k, n))
    want = ref.linear_reference(gen.bf16_bits_to_f32(x), gen.bf16_bits_to_f32(w))
    err = rel_err(y, want)
    say("  rel err", err, "splits ws", binding.mla_linear_workspace_bytes(m, k, n))
    assert not np.isnan(y).any() and err <= BF16_TOL


def test_linear_prefill_size_sampled_rows_and_determinism():
    m, k, n = 4096, 7168, 2112
    say("linear prefill size", m, k, n)
    rng = np.random.default_rng(5)
    x = gen.round_to_bf16_bits(rng.standard_normal((m, k), dtype=np.float32))
    w = gen.round_to_bf16_bits(rng.standard_normal((k, n), dtype=np.float32) / np.float32(math.sqrt(k)))
    y1 = _linear(x, w, m, k, n)
    y2 = _linear(x, w, m, k, n)
    import torch
    assert torch.equal(y1, y2)
    rows = [0, 31, 32, 1000, 2047, 4064, 4095]
    want = ref.linear_reference(gen.bf16_bits_to_f32(x[rows]), gen.bf16_bits_to_f32(w))
    assert rel_err(to_host(y1)[rows], want) <= BF16_TOL


def _rope_case(lens, S, seed, stride=2112, col=1536):
    """Pool with NaN in unused slots; kv_a rows of `stride` with [c_KV | k_pe] at column `col`."""
    import torch
    B = len(lens)
    w = gen.small_workload(B, S, cache_len=1, dtype="bf16", paged=True)
    x = gen.generate(w, seed, poison_unused=True, seq_lens=lens)
    rng = np.random.default_rng(seed + 1)
    kv_rows = gen.round_to_bf16_bits(rng.standard_normal((B * S, stride), dtype=np.float32))
    p = params_for(x)
    d = to_device(x)
    kv_dev = _bf16_dev(kv_rows)
    pool_before = d["pool"].clone()
    q_before = d["q_pe"].clone()
    kv_a = kv_dev.data_ptr() + col * 2  # rows of `stride` elements, [c_KV | k_pe] at column `col`
    binding.mla_rope_append(d["q_pe"], kv_a, stride, d["pool"], d["block_table"], d["seq_lens"], p)
    torch.cuda.synchronize()
    pos = ref.new_token_positions(x.seq_lens, S)
    q_want = ref.rope_reference(x.f32("q_pe"), pos)
    kva = gen.bf16_bits_to_f32(kv_rows[:, col:col + 576]).reshape(B, S, 576)
    k_rot = ref.rope_reference(kva[..., 512:], pos)
    pool_want = ref.append_kv_reference(x.f32("pool"), x.block_table, x.seq_lens, kva[..., :512], k_rot)
    return x, d, pool_before, q_before, kv_rows, pos, q_want, pool_want


@pytest.mark.parametrize("lens,S", [([9, 300, 64, 65], 1), ([5, 130, 1, 66], 2), ([2, 200], 5),
                                    ([131072, 70000], 2)])
def test_rope_append(lens, S):
    say("rope_append", lens, "S", S)
    x, d, pool_before, q_before, kv_rows, pos, q_want, pool_want = _rope_case(lens, S, 40 + S)
    q = to_host(d["q_pe"])
    err = rel_err(q, q_want)
    say("  q_pe rel err", err)
    assert err <= BF16_TOL
    import torch
    pool = d["pool"].cpu().view(torch.int16).numpy().view(np.uint16)
    before = pool_before.cpu().view(torch.int16).numpy().view(np.uint16)
    touched = np.zeros(pool.shape[:2], dtype=bool)
    for b, L in enumerate(x.seq_lens):
        for i in range(S):
            pp = int(pos[b, i])
            if pp < 0:
                continue
            pg, sl = x.block_table[b, pp // 64], pp % 64
            touched[pg, sl] = True
            np.testing.assert_array_equal(pool[pg, sl, :512], kv_rows[b * S + i, 1536:1536 + 512])  # a copy
            k_err = rel_err(gen.bf16_bits_to_f32(pool[pg, sl, 512:]), pool_want[pg, sl, 512:])
            assert k_err <= BF16_TOL, (b, i, k_err)
    np.testing.assert_array_equal(pool[~touched], before[~touched])  # NaN poison included, bit for bit


def test_prepared_inputs_feed_the_decode_path():
    """hidden -> fused projection -> RoPE + AppendKV -> absorbed decode, against the oracle chain
    (projection, rotation and append in fp64, then the non-absorbed decode reference)."""
    import torch
    say("prepare -> decode chain")
    B, S, D = 2, 2, 512
    lens = [130, 67]
    w = gen.small_workload(B, S, cache_len=1, dtype="bf16", paged=True)
    x = gen.generate(w, 77, poison_unused=True, seq_lens=lens)
    rng = np.random.default_rng(78)
    hidden = gen.round_to_bf16_bits(rng.standard_normal((B * S, D), dtype=np.float32))
    w_a = gen.round_to_bf16_bits(rng.standard_normal((D, 576), dtype=np.float32) / np.float32(math.sqrt(D)))
    p = params_for(x)
    d = to_device(x)
    y = _linear(hidden, w_a, B * S, D, 576)  # [c_KV | k_pe] only (no c^Q in this chain)
    binding.mla_rope_append(d["q_pe"], y, 576, d["pool"], d["block_table"], d["seq_lens"], p)
    bufs = binding.DecodeBuffers(p, 0)
    bufs.run(d["q_nope"], d["q_pe"], d["w_uk"], d["w_uv"], d["pool"], d["block_table"], d["seq_lens"])
    torch.cuda.synchronize()

    pos = ref.new_token_positions(x.seq_lens, S)
    kva = ref.linear_reference(gen.bf16_bits_to_f32(hidden), gen.bf16_bits_to_f32(w_a)).reshape(B, S, 576)
    pool = ref.append_kv_reference(x.f32("pool"), x.block_table, x.seq_lens, kva[..., :512],
                                   ref.rope_reference(kva[..., 512:], pos))
    q_pe = ref.rope_reference(x.f32("q_pe"), pos)
    r = dec.mla_decode_nonabsorbed(x.f32("q_nope"), q_pe, x.f32("w_uk"), x.f32("w_uv"), pool, x.block_table,
                                   x.seq_lens, softmax_scale=w.softmax_scale)
    err = rel_err(to_host(bufs.out), r["out"])
    say("  out rel err", err)
    assert err <= BF16_TOL


def test_output_projection_after_the_decode_path():
    """decode path out (B,S,H,128) -> W_O as a plain projection (16384 -> 7168) with mla_linear,
    against the oracle's non-absorbed output followed by its output projection."""
    import torch
    say("decode -> W_O")
    B, S, E = 4, 1, 7168
    w = gen.small_workload(B, S, ragged=(60, 330), dtype="bf16", paged=True)
    x = gen.generate(w, 91, poison_unused=True)
    rng = np.random.default_rng(92)
    w_o = gen.round_to_bf16_bits(rng.standard_normal((128 * 128, E), dtype=np.float32) / np.float32(128.0))
    p = params_for(x)
    d = to_device(x)
    bufs = binding.DecodeBuffers(p, 0)
    bufs.run(d["q_nope"], d["q_pe"], d["w_uk"], d["w_uv"], d["pool"], d["block_table"], d["seq_lens"])
    y = torch.full((B * S, E), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws_bytes = binding.mla_linear_workspace_bytes(B * S, 128 * 128, E)
    ws = torch.empty(max(ws_bytes, 16) // 4, dtype=torch.float32, device="cuda") if ws_bytes else None
    binding.mla_linear(bufs.out.reshape(B * S, 128 * 128), _bf16_dev(w_o), y, B * S, 128 * 128, E, ws)
    torch.cuda.synchronize()
    r = dec.mla_decode_nonabsorbed(x.f32("q_nope"), x.f32("q_pe"), x.f32("w_uk"), x.f32("w_uv"), x.f32("pool"),
                                   x.block_table, x.seq_lens, softmax_scale=w.softmax_scale)
    want = dec.o_proj_reference(r["out"], gen.bf16_bits_to_f32(w_o).reshape(128, 128, E)).reshape(B * S, E)
    err = rel_err(to_host(y), want)
    say("  rel err", err)
    assert err <= BF16_TOL
