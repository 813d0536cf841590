"""GPU parity of the prefill calls (multi-head form) against the fp64 oracle, through the C ABI.

Bar: max |gpu - ref| / max |ref| <= 2e-2 per output (bf16 operands, fp32 accumulation); lse within
2e-2 in absolute terms, and on sampled rows the oracle's logits normalised by the GPU's lse sum to
one within 2e-2; the k_pe copy and the zero rows past each sequence are checked bit for bit.  Unused cache slots are
NaN, so a read outside the sequences shows up as NaN.
"""
import numpy as np
import pytest

from deepseek_mla_latent_amd import binding
from deepseek_mla_latent_amd import inputs as gen
from oracle import mla_decode as ref
from oracle import mla_prefill as pf
from tests.helpers import BF16_TOL, check_lse, check_softmax_mass, params_for, rel_err, sample_rows, to_device, to_host

pytestmark = pytest.mark.gpu

H, DH, DR = 128, 128, 64


def say(*a):
    print("[case]", *a, flush=True)


def _kv_views(kv, B, Lp):
    """Split the flat bf16 buffer into [K_nope | V] (B,H,Lp,256) and k_pe (B,Lp,64)."""
    n = B * H * Lp * 2 * DH
    return kv[:n].view(B, H, Lp, 2 * DH), kv[n:n + B * Lp * DR].view(B, Lp, DR)


def _run_kv_up(x, p):
    import torch
    d = to_device(x)
    nbytes = binding.mla_prefill_kv_bytes(p)
    kv = torch.full((nbytes // 2,), float("nan"), dtype=torch.bfloat16, device="cuda")
    binding.mla_prefill_kv_up(d["pool"], d["block_table"], d["seq_lens"], d["w_uk"], d["w_uv"], kv, p)
    return d, kv


def _run_attn(d, kv, x, p):
    import torch
    w = x.workload
    out = torch.full((w.batch, w.q_len, H, DH), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((w.batch, w.q_len, H), float("nan"), device="cuda")
    binding.mla_prefill_attn(d["q_nope"], d["q_pe"], kv, d["seq_lens"], out, lse, p)
    torch.cuda.synchronize()
    return to_host(out), to_host(lse)


@pytest.mark.parametrize("lens", [[1, 63, 64, 65, 300], [129, 0, 200]])
def test_kv_up(lens):
    say("kv_up", lens)
    w = gen.small_workload(len(lens), 1, cache_len=1, dtype="bf16", paged=True)
    x = gen.generate(w, 31, poison_unused=True, seq_lens=lens)
    p = params_for(x)
    _, kv = _run_kv_up(x, p)
    import torch
    torch.cuda.synchronize()
    Lp = p.max_pages_per_seq * 64
    kvh, peh = _kv_views(kv, w.batch, Lp)
    kvh, peh_bits = to_host(kvh), peh.cpu().view(torch.int16).numpy().view(np.uint16)
    K, V, kpe = pf.kv_up_reference(x.f32("pool"), x.block_table, x.seq_lens, x.f32("w_uk"), x.f32("w_uv"))
    for b, L in enumerate(lens):
        end = -(-L // 64) * 64
        if L:
            err_k = rel_err(kvh[b, :, :L, :DH], K[b, :, :L])
            err_v = rel_err(kvh[b, :, :L, DH:], V[b, :, :L])
            say("  seq", b, "rel err K", err_k, "V", err_v)
            assert err_k <= BF16_TOL and err_v <= BF16_TOL
            rows = x.pool[x.block_table[b, np.arange(L) // 64], np.arange(L) % 64]
            np.testing.assert_array_equal(peh_bits[b, :L], rows[:, 512:])  # a copy: bit-exact
        assert np.all(kvh[b, :, L:end] == 0) and np.all(peh_bits[b, L:end] == 0)


def _oracle_kv_buffer(x, p):
    """The kv buffer in the library's layout, filled from the oracle's K/V rounded to bf16."""
    import torch
    B = x.workload.batch
    Lp = p.max_pages_per_seq * 64
    K, V, kpe = pf.kv_up_reference(x.f32("pool"), x.block_table, x.seq_lens, x.f32("w_uk"), x.f32("w_uv"))
    kvb = np.zeros((B, H, Lp, 2 * DH), np.uint16)
    peb = np.zeros((B, Lp, DR), np.uint16)
    Kr, Vr = np.zeros_like(K), np.zeros_like(V)
    for b, L in enumerate(x.seq_lens):
        kvb[b, :, :L, :DH] = gen.round_to_bf16_bits(K[b, :, :L])
        kvb[b, :, :L, DH:] = gen.round_to_bf16_bits(V[b, :, :L])
        Kr[b, :, :L] = gen.bf16_bits_to_f32(kvb[b, :, :L, :DH])
        Vr[b, :, :L] = gen.bf16_bits_to_f32(kvb[b, :, :L, DH:])
        peb[b, :L] = gen.round_to_bf16_bits(kpe[b, :L])
    flat = np.concatenate([kvb.ravel(), peb.ravel()])
    assert flat.size * 2 == binding.mla_prefill_kv_bytes(p)
    dev = torch.from_numpy(flat.view(np.int16)).view(torch.bfloat16).cuda()
    return dev, Kr, Vr, gen.bf16_bits_to_f32(peb)


@pytest.mark.parametrize("name,S,lens,causal", [
    ("whole prompt", 300, [300, 300], True),
    ("chunk", 100, [230, 300], True),
    ("non-causal", 100, [230, 300], False),
    ("short sequences", 64, [0, 1, 40, 64], True),
    ("long chunk over ragged tiles", 200, [333, 270], True),
])
def test_attention_on_oracle_kv(name, S, lens, causal):
    say("prefill attn", name, "S", S, "lens", lens, "causal", causal)
    w = gen.small_workload(len(lens), S, cache_len=1, dtype="bf16", paged=True)
    x = gen.generate(w, 41 + S, poison_unused=True, seq_lens=lens)
    p = params_for(x, causal=causal)
    d = to_device(x)
    kv, Kr, Vr, kpe = _oracle_kv_buffer(x, p)
    out, lse = _run_attn(d, kv, x, p)
    want = pf.mha_attention_reference(x.f32("q_nope"), x.f32("q_pe"), Kr, Vr, kpe, x.seq_lens,
                                      softmax_scale=w.softmax_scale, causal=causal)
    assert not np.isnan(out).any() and not np.isnan(lse).any()
    err = rel_err(out, want["out"])
    say("  out rel err", err)
    assert err <= BF16_TOL
    check_lse(lse, want["lse"], BF16_TOL)


def _end_to_end(x, heads, causal=True):
    p = params_for(x, causal=causal)
    d, kv = _run_kv_up(x, p)
    out, lse = _run_attn(d, kv, x, p)
    r = ref.mla_decode_nonabsorbed(x.f32("q_nope"), x.f32("q_pe"), x.f32("w_uk"), x.f32("w_uv"), x.f32("pool"),
                                   x.block_table, x.seq_lens, softmax_scale=x.workload.softmax_scale, heads=heads,
                                   causal=causal)
    sel = np.ix_(range(x.workload.batch), range(x.workload.q_len), heads)
    err = rel_err(out[sel], r["out"][sel])
    say("  out rel err", err)
    assert err <= BF16_TOL
    check_lse(lse[sel], r["lse"][sel], BF16_TOL)
    rows = [(b, i, h) for b, i, h in sample_rows(r["lse"]) if h in heads]
    merr = check_softmax_mass(ref.absorb_q_reference(x.f32("q_nope"), x.f32("w_uk")), x.f32("q_pe"), x.f32("pool"),
                              x.block_table, x.seq_lens, lse, rows, softmax_scale=x.workload.softmax_scale,
                              tol=BF16_TOL, causal=causal)
    say("  softmax mass err", merr)
    return out, lse


def test_end_to_end_small_all_heads():
    say("prefill end-to-end, whole prompts of 190 and 130 tokens, all heads")
    w = gen.small_workload(2, 130, cache_len=1, dtype="bf16", paged=True)
    x = gen.generate(w, 51, poison_unused=True, seq_lens=[190, 130])
    _end_to_end(x, list(range(128)))


def test_end_to_end_full_size():
    say("prefill end-to-end prefill_b1_s4096, heads 0 77 127")
    x = gen.generate_named("prefill_b1_s4096", poison_unused=True)
    _end_to_end(x, [0, 77, 127])


def test_matches_absorbed_decode_path():
    """The same outputs from the absorbed GPU route (absorb -> latent attention -> out-projection)."""
    import torch
    say("prefill vs absorbed GPU route, S = L = 200")
    w = gen.small_workload(1, 200, cache_len=200, dtype="bf16", paged=True)
    x = gen.generate(w, 61, poison_unused=True)
    p = params_for(x)
    d, kv = _run_kv_up(x, p)
    out, lse = _run_attn(d, kv, x, p)
    bufs = binding.DecodeBuffers(p, 0)
    bufs.run(d["q_nope"], d["q_pe"], d["w_uk"], d["w_uv"], d["pool"], d["block_table"], d["seq_lens"])
    torch.cuda.synchronize()
    assert rel_err(out, to_host(bufs.out)) <= BF16_TOL
    assert np.max(np.abs(lse - to_host(bufs.lse))) <= 2e-2


def test_deterministic():
    say("prefill run-to-run determinism")
    w = gen.small_workload(2, 150, cache_len=1, dtype="bf16", paged=True)
    x = gen.generate(w, 71, poison_unused=True, seq_lens=[150, 222])
    p = params_for(x)
    d, kv = _run_kv_up(x, p)
    a = _run_attn(d, kv, x, p)
    d2, kv2 = _run_kv_up(x, p)
    b = _run_attn(d2, kv2, x, p)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
