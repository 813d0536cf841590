"""The bounds-checked build (libmla_latent_debug.so, compiled with MLA_DEBUG_BOUNDS) on the GPU.

Its kernels test every seq_lens entry and block_table entry they use against the documented
ranges, report violations in the device error word (read back with mla_debug_bounds_read), and go
on with a safe value.  Checked here, against the fp64 oracle:
  * clean inputs: the same results as the oracle (to the parity bar) and an error word of zero;
  * a seq_lens entry above max_seq_len: bit 1, and that row equals the oracle at max_seq_len;
    a negative entry: bit 1 and an empty row (o = 0, lse = -inf);
  * a page id at or past num_pages, or a negative one: bit 2, and every other sequence still
    equals the oracle; the cache append skips its write (the page stays as it was).
Every out-of-range value still points into memory this test allocated (spare pages after the
pool, a spare page before it, table rows wide enough for the oversized length), so a check that
failed to catch one could not fault the GPU.
"""
import ctypes
import os

import numpy as np
import pytest

from deepseek_mla_latent_amd import binding
from deepseek_mla_latent_amd import inputs as gen
from oracle import mla_decode as ref
from oracle import mla_prepare as ref_prep
from tests.helpers import BF16_TOL, check_lse, device_array, rel_err, to_host

pytestmark = pytest.mark.gpu

BAD_LEN, BAD_PAGE = binding.BOUNDS_BAD_SEQ_LEN, binding.BOUNDS_BAD_PAGE


def say(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module")
def dbg():
    if not os.path.exists(binding.DEBUG_LIB_PATH):
        pytest.fail("libmla_latent_debug.so is not built")
    lib = binding.load_library(binding.DEBUG_LIB_PATH)
    assert lib.mla_debug_bounds_enabled() == 1
    binding.mla_debug_bounds_read(lib)  # start from a cleared word
    return lib


def _t():
    import torch
    return torch


class Batch:
    """A paged bf16 decode batch on the GPU with spare memory around the pool: `lead` pages before
    the page the kernels see as page 0 and `tail` pages after the last real one."""

    def __init__(self, lens, seed, lead=1, tail=2, q_len=1):
        torch = _t()
        w = gen.small_workload(len(lens), q_len, cache_len=1, dtype="bf16", paged=True)
        self.x = gen.generate(w, seed, seq_lens=lens)
        self.w = w
        pool = self.x.pool
        spare = gen.round_to_bf16_bits(np.random.default_rng(seed + 1).standard_normal(
            (lead + tail,) + pool.shape[1:], dtype=np.float32))
        full = np.concatenate([spare[:lead], pool, spare[lead:]])
        self.pool_all = torch.from_numpy(full.view(np.int16)).view(torch.bfloat16).cuda()
        self.pool = self.pool_all[lead:]  # page 0 of the kernels; page -1 is the lead page
        self.num_pages = pool.shape[0]
        self.bt = self.x.block_table.copy()
        self.lens = np.asarray(lens, dtype=np.int32)
        self.q_lat_bits, _ = gen.generate_latent(w, seed + 2)
        self.q_lat = device_array(self.q_lat_bits, True)
        self.q_pe = device_array(self.x.q_pe, True)

    def params(self, max_seq_len, **kw):
        return binding.make_params(batch=self.w.batch, q_len=self.w.q_len, max_seq_len=max_seq_len,
                                   max_pages_per_seq=self.bt.shape[1], softmax_scale=self.w.softmax_scale,
                                   num_pages=self.num_pages, **kw)

    def attend(self, lib, p, splits):
        torch = _t()
        B, S = self.w.batch, self.w.q_len
        o = torch.full((B, S, 128, 512), float("nan"), device="cuda")
        lse = torch.full((B, S, 128), float("nan"), device="cuda")
        nb = lib.mla_decode_workspace_bytes(ctypes.byref(p), splits)
        ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
        bt = torch.from_numpy(self.bt).cuda()
        lens = torch.from_numpy(self.lens).cuda()
        code = lib.mla_decode_attn(self.q_lat.data_ptr(), self.q_pe.data_ptr(), self.pool.data_ptr(), bt.data_ptr(),
                                   lens.data_ptr(), o.data_ptr(), lse.data_ptr(), ws.data_ptr(), nb, splits,
                                   ctypes.byref(p), binding._stream(None))
        assert code == 0, code
        torch.cuda.synchronize()
        return to_host(o), to_host(lse)

    def oracle(self, lens, bt=None):
        return ref.latent_attention_reference(gen.bf16_bits_to_f32(self.q_lat_bits), self.x.f32("q_pe"),
                                              self.x.f32("pool"), self.x.block_table if bt is None else bt,
                                              np.asarray(lens, dtype=np.int32), softmax_scale=self.w.softmax_scale)


def _check_rows(o, lse, want, seqs):
    for b in seqs:
        err = rel_err(o[b], want["o_lat"][b])
        lerr = check_lse(lse[b], want["lse"][b], BF16_TOL)
        say(f"  seq {b}: o rel err {err:.2e} lse abs err {lerr:.2e}")
        assert err <= BF16_TOL


@pytest.mark.parametrize("splits", [1, 2])
def test_clean_inputs_match_the_oracle_and_report_nothing(dbg, splits):
    say("bounds build, clean inputs, splits", splits)
    bx = Batch([300, 64, 129], 501)
    o, lse = bx.attend(dbg, bx.params(300), splits)
    _check_rows(o, lse, bx.oracle(bx.lens), range(3))
    assert binding.mla_debug_bounds_read(dbg) == (0, 0)


@pytest.mark.parametrize("splits", [1, 2])
def test_seq_len_out_of_range_is_clamped_and_reported(dbg, splits):
    say("bounds build, seq_lens out of range, splits", splits)
    # the table and pool hold 237 tokens of sequence 0; the caller claims at most 200
    bx = Batch([237, 150, 90], 511)
    bx.lens = np.array([237, 150, -5], dtype=np.int32)
    o, lse = bx.attend(dbg, bx.params(200), splits)
    words = binding.mla_debug_bounds_read(dbg)
    say("  error word", words)
    assert words[0] == BAD_LEN and words[1] > 0
    _check_rows(o, lse, bx.oracle([200, 150, 0]), [0, 1])
    assert np.all(o[2] == 0) and np.all(np.isneginf(lse[2]))


@pytest.mark.parametrize("bad", ["past the pool", "negative"])
def test_page_id_out_of_range_is_reported_and_others_are_intact(dbg, bad):
    say("bounds build, page id", bad)
    bx = Batch([200, 180, 150], 521)
    bx.bt[1, 1] = bx.num_pages + 1 if bad == "past the pool" else -1  # a spare page either way
    o, lse = bx.attend(dbg, bx.params(200), 2)
    words = binding.mla_debug_bounds_read(dbg)
    say("  error word", words)
    assert words[0] == BAD_PAGE and words[1] > 0
    _check_rows(o, lse, bx.oracle(bx.lens), [0, 2])
    assert not np.isnan(o[1]).any()  # sequence 1 read page 0 in place of the bad one


def test_fused_call_reports_a_bad_page(dbg):
    torch = _t()
    say("bounds build, fused call with a bad page id")
    bx = Batch([300] * 16, 531)
    bx.bt[5, 2] = bx.num_pages + 1
    p = bx.params(300)
    w_uv = device_array(bx.x.w_uv, True)
    out = torch.empty((16, 1, 128, 128), dtype=torch.bfloat16, device="cuda")
    nb = dbg.mla_decode_attn_out_proj_workspace_bytes(ctypes.byref(p), 2)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    bt, lens = torch.from_numpy(bx.bt).cuda(), torch.from_numpy(bx.lens).cuda()
    code = dbg.mla_decode_attn_out_proj(bx.q_lat.data_ptr(), bx.q_pe.data_ptr(), bx.pool.data_ptr(), bt.data_ptr(),
                                        lens.data_ptr(), None, w_uv.data_ptr(), out.data_ptr(), None, None,
                                        ws.data_ptr(), nb, 2, ctypes.byref(p), binding._stream(None))
    assert code == 0
    words = binding.mla_debug_bounds_read(dbg)
    say("  error word", words)
    assert words[0] == BAD_PAGE and words[1] > 0
    want = ref.out_proj_reference(bx.oracle(bx.lens)["o_lat"], bx.x.f32("w_uv"))
    got = to_host(out)
    keep = [b for b in range(16) if b != 5]
    assert rel_err(got[keep], want[keep]) <= BF16_TOL


def test_cache_append_skips_a_bad_page(dbg):
    torch = _t()
    say("bounds build, rope_append into a bad page")
    bx = Batch([130, 67], 541)
    bad = bx.num_pages + 1
    bx.bt[1, (67 - 1) // 64] = bad
    kv_a = gen.round_to_bf16_bits(np.random.default_rng(542).standard_normal((2, 576), dtype=np.float32))
    kv_dev = device_array(kv_a, True)
    before = bx.pool_all.clone()
    p = bx.params(130)
    bt, lens = torch.from_numpy(bx.bt).cuda(), torch.from_numpy(bx.lens).cuda()
    code = dbg.mla_rope_append(bx.q_pe.data_ptr(), kv_dev.data_ptr(), 576, bx.pool.data_ptr(), bt.data_ptr(),
                               lens.data_ptr(), 10000.0, ctypes.byref(p), binding._stream(None))
    assert code == 0
    words = binding.mla_debug_bounds_read(dbg)
    say("  error word", words)
    assert words[0] == BAD_PAGE and words[1] > 0
    after = bx.pool_all
    lead = 1
    assert torch.equal(after[lead + bad], before[lead + bad])  # the bad page: untouched
    # sequence 0 appended its row (c_KV copied) at position 129
    pg = int(bx.bt[0, 129 // 64])
    got = after[lead + pg, 129 % 64, :512].cpu().view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, kv_a[0, :512])
    # both queries were rotated regardless
    pos = ref_prep.new_token_positions(bx.lens, 1)
    q_want = ref_prep.rope_reference(bx.x.f32("q_pe"), pos)
    assert rel_err(to_host(bx.q_pe), q_want) <= BF16_TOL


def test_prefill_reports_bad_entries(dbg):
    torch = _t()
    say("bounds build, prefill with a bad page id and a long seq_len")
    bx = Batch([160, 170], 551, q_len=1)
    bx.bt[0, 1] = bx.num_pages + 1
    p = binding.make_params(batch=2, q_len=96, max_seq_len=160, max_pages_per_seq=bx.bt.shape[1],
                            num_pages=bx.num_pages)
    nb = dbg.mla_prefill_kv_bytes(ctypes.byref(p))
    assert nb > 0
    kv = torch.empty(nb, dtype=torch.uint8, device="cuda")
    w_uk, w_uv = device_array(bx.x.w_uk, True), device_array(bx.x.w_uv, True)
    bt, lens = torch.from_numpy(bx.bt).cuda(), torch.from_numpy(bx.lens).cuda()
    code = dbg.mla_prefill_kv_up(bx.pool.data_ptr(), bt.data_ptr(), lens.data_ptr(), w_uk.data_ptr(), w_uv.data_ptr(),
                                 kv.data_ptr(), nb, ctypes.byref(p), binding._stream(None))
    assert code == 0
    words = binding.mla_debug_bounds_read(dbg)
    say("  kv_up error word", words)
    assert words[0] == BAD_PAGE | BAD_LEN and words[1] > 0  # page id of sequence 0, length of sequence 1
    q_nope = torch.zeros((2, 96, 128, 128), dtype=torch.bfloat16, device="cuda")
    q_pe = torch.zeros((2, 96, 128, 64), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((2, 96, 128, 128), dtype=torch.bfloat16, device="cuda")
    code = dbg.mla_prefill_attn(q_nope.data_ptr(), q_pe.data_ptr(), kv.data_ptr(), nb, lens.data_ptr(), out.data_ptr(),
                                None, ctypes.byref(p), binding._stream(None))
    assert code == 0
    words = binding.mla_debug_bounds_read(dbg)
    say("  prefill_attn error word", words)
    assert words[0] == BAD_LEN and words[1] > 0
    assert not torch.isnan(out.float()).any()
