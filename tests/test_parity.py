"""GPU parity: every call of the C-ABI library against the fp64 CPU oracle on the same seeded inputs.

Bar (the stated tolerance of the method on bf16 inputs with fp32 accumulation, and on fp32 inputs):
max |gpu - ref| / max |ref| <= 2e-2 (bf16) and <= 1e-4 (fp32), per output tensor; lse within the
same numbers in absolute terms (-inf exactly where the oracle has it), and on sampled rows the
oracle's own logits normalised by the GPU's lse sum to one within them.  Every batch has its unused
cache slots poisoned with NaN, so a read outside the sequences shows up as NaN.
"""
import math

import numpy as np
import pytest

from deepseek_mla_latent_amd import binding
from deepseek_mla_latent_amd import inputs as gen
from oracle import mla_decode as ref
from tests.helpers import (check_lse, check_softmax_mass, device_array, params_for, rel_err, sample_rows, to_device,
                           to_host, tol_for)

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def _torch():
    import torch
    return torch


# ------------------------------------------------------------------------------------ projections
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("tokens", [1, 2, 4, 5, 33, 128])
def test_absorb_q(dtype, tokens):
    say("absorb_q", dtype, tokens)
    torch = _torch()
    w = gen.small_workload(tokens, 1, cache_len=1, dtype=dtype, paged=False)
    x = gen.generate(w, 100 + tokens)
    d = to_device(x)
    p = params_for(x)
    q_lat = torch.empty((tokens, 1, 128, 512), dtype=d["q_nope"].dtype, device="cuda")
    binding.mla_absorb_q(d["q_nope"], d["w_uk"], q_lat, p)
    torch.cuda.synchronize()
    want = ref.absorb_q_reference(x.f32("q_nope"), x.f32("w_uk"))
    err = rel_err(to_host(q_lat), want)
    say("  rel err", err)
    assert err <= tol_for(x)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("tokens", [1, 2, 4, 5, 33, 128])
def test_out_proj(dtype, tokens):
    say("out_proj", dtype, tokens)
    torch = _torch()
    w = gen.small_workload(tokens, 1, cache_len=1, dtype=dtype, paged=False)
    x = gen.generate(w, 200 + tokens)
    _, o_lat = gen.generate_latent(w, 300 + tokens)
    d = to_device(x)
    p = params_for(x)
    o_dev = torch.from_numpy(o_lat).cuda()
    out = torch.empty((tokens, 1, 128, 128), dtype=d["w_uv"].dtype, device="cuda")
    binding.mla_out_proj(o_dev, d["w_uv"], out, p)
    torch.cuda.synchronize()
    want = ref.out_proj_reference(o_lat, x.f32("w_uv"))
    err = rel_err(to_host(out), want)
    say("  rel err", err)
    assert err <= tol_for(x)


# ------------------------------------------------------------------------------------ attention
def _run_attn(x, q_lat_bits, splits, causal=True):
    torch = _torch()
    d = to_device(x)
    p = params_for(x, causal=causal)
    w = x.workload
    q_lat = device_array(q_lat_bits, x.is_bf16)
    o = torch.full((w.batch, w.q_len, 128, 512), float("nan"), device="cuda")
    lse = torch.full((w.batch, w.q_len, 128), float("nan"), device="cuda")
    ws_bytes = binding.mla_decode_workspace_bytes(p, splits)
    ws = torch.empty(max(ws_bytes, 16) // 4, dtype=torch.float32, device="cuda") if ws_bytes else None
    binding.mla_decode_attn(q_lat, d["q_pe"], d["pool"], d["block_table"], d["seq_lens"], o, lse, ws, splits, p)
    torch.cuda.synchronize()
    return to_host(o), to_host(lse)


def _attn_case(x, seed, splits, causal=True):
    q_lat, _ = gen.generate_latent(x.workload, seed)
    q_lat_f32 = gen.bf16_bits_to_f32(q_lat) if x.is_bf16 else q_lat
    o, lse = _run_attn(x, q_lat, splits, causal)
    want = ref.latent_attention_reference(q_lat_f32, x.f32("q_pe"), x.f32("pool"), x.block_table, x.seq_lens,
                                          softmax_scale=x.workload.softmax_scale, causal=causal)
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    err = rel_err(o, want["o_lat"])
    lerr = check_lse(lse, want["lse"], tol_for(x))
    merr = check_softmax_mass(q_lat_f32, x.f32("q_pe"), x.f32("pool"), x.block_table, x.seq_lens, lse,
                              sample_rows(want["lse"], seed=seed), softmax_scale=x.workload.softmax_scale,
                              tol=tol_for(x), causal=causal)
    say("  o_lat rel err", err, "lse abs err", lerr, "mass err", merr)
    assert err <= tol_for(x)
    return o, lse


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("splits", [1, 2, 3, 0])
def test_attention_ragged_paged(dtype, splits):
    say("attn ragged paged", dtype, "splits", splits)
    w = gen.small_workload(3, 1, ragged=(1, 300), dtype=dtype, paged=True)
    x = gen.generate(w, 7, poison_unused=True)
    _attn_case(x, 8, splits)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [True, False])
def test_attention_two_query_tokens(dtype, causal):
    say("attn S=2", dtype, "causal", causal)
    w = gen.small_workload(3, 2, ragged=(2, 260), dtype=dtype, paged=True)
    x = gen.generate(w, 9, poison_unused=True)
    _attn_case(x, 10, 2, causal)
    _attn_case(x, 10, 1, causal)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_attention_edge_lengths(dtype):
    """Empty, single-token, page-boundary and off-by-one lengths; L < S for the causal S=2 case."""
    lens = [0, 1, 63, 64, 65, 128, 129, 2]
    say("attn edge lengths", dtype, lens)
    w = gen.small_workload(len(lens), 1, cache_len=1, dtype=dtype, paged=True)
    x = gen.generate(w, 11, poison_unused=True, seq_lens=lens)
    for splits in (1, 2, 0):
        o, lse = _attn_case(x, 12, splits)
        assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))
    w2 = gen.small_workload(3, 2, cache_len=1, dtype=dtype, paged=True)
    x2 = gen.generate(w2, 13, poison_unused=True, seq_lens=[1, 0, 65])
    o, lse = _attn_case(x2, 14, 2)
    assert np.all(np.isneginf(lse[0, 0])) and np.all(np.isfinite(lse[0, 1]))


def test_attention_split_invariance_and_determinism():
    say("attn split invariance")
    w = gen.small_workload(2, 1, ragged=(500, 900), dtype="bf16", paged=True)
    x = gen.generate(w, 15, poison_unused=True)
    q_lat, _ = gen.generate_latent(w, 16)
    outs = {s: _run_attn(x, q_lat, s) for s in (1, 2, 7, 0)}
    for s in (2, 7, 0):
        assert rel_err(outs[s][0], outs[1][0]) <= 5e-3
        assert np.max(np.abs(outs[s][1] - outs[1][1])) <= 5e-3
    again = _run_attn(x, q_lat, 7)
    assert np.array_equal(again[0], outs[7][0]) and np.array_equal(again[1], outs[7][1])


def test_attention_page_permutation_is_bitwise_invisible():
    say("attn page permutation")
    w = gen.small_workload(2, 1, ragged=(100, 400), dtype="bf16", paged=False)
    x = gen.generate(w, 17, poison_unused=True)
    q_lat, _ = gen.generate_latent(w, 18)
    a = _run_attn(x, q_lat, 3)
    perm = np.random.default_rng(19).permutation(x.num_pages)
    pool2 = np.empty_like(x.pool)
    pool2[perm] = x.pool
    bt2 = np.where(x.block_table >= 0, perm[np.maximum(x.block_table, 0)], -1).astype(np.int32)
    x2 = gen.DecodeInputs(w, x.seq_lens, bt2, pool2, x.q_nope, x.q_pe, x.w_uk, x.w_uv)
    b = _run_attn(x2, q_lat, 3)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_attention_rescale_path():
    """Later tiles score far above earlier ones, so the running max is raised (and O rescaled) many
    times: rows of tile t are scaled by 1 + t before rounding to bf16."""
    say("attn rescale path")
    w = gen.small_workload(2, 1, ragged=(290, 330), dtype="bf16", paged=True)
    x = gen.generate(w, 27, poison_unused=True)
    pool = gen.bf16_bits_to_f32(x.pool).copy()
    for b in range(w.batch):
        for j in range(int(x.seq_lens[b])):
            page, slot = x.block_table[b, j // 64], j % 64
            pool[page, slot] *= np.float32(1 + j // 32)
    x = gen.DecodeInputs(w, x.seq_lens, x.block_table, gen.round_to_bf16_bits(pool), x.q_nope, x.q_pe, x.w_uk,
                         x.w_uv)
    for splits in (1, 2):
        _attn_case(x, 28, splits)


# ------------------------------------------------------------------------------------ end to end
def _end_to_end(x, seqs, heads, splits=0):
    """GPU q_nope -> q_lat -> (o_lat, lse) -> out against the non-absorbed oracle on sampled (b, h)."""
    torch = _torch()
    w = x.workload
    d = to_device(x)
    p = params_for(x)
    bufs = binding.DecodeBuffers(p, splits)
    bufs.run(d["q_nope"], d["q_pe"], d["w_uk"], d["w_uv"], d["pool"], d["block_table"], d["seq_lens"])
    torch.cuda.synchronize()
    tol = tol_for(x)
    q_lat = to_host(bufs.q_lat)
    want_q = ref.absorb_q_reference(x.f32("q_nope")[seqs], x.f32("w_uk"))
    assert rel_err(q_lat[seqs], want_q) <= tol
    r = ref.mla_decode_nonabsorbed(x.f32("q_nope"), x.f32("q_pe"), x.f32("w_uk"), x.f32("w_uv"), x.f32("pool"),
                                   x.block_table, x.seq_lens, softmax_scale=w.softmax_scale, seqs=seqs, heads=heads)
    sel = np.ix_(seqs, range(w.q_len), heads)
    errs = {k: rel_err(to_host(getattr(bufs, k))[sel], r[k][sel]) for k in ("o_lat", "out")}
    say("  rel errs", errs)
    for k, e in errs.items():
        assert e <= tol, k
    lse = to_host(bufs.lse)
    check_lse(lse[sel], r["lse"][sel], tol)
    rows = [(b, i, h) for b in seqs for i in range(w.q_len) for h in heads if np.isfinite(r["lse"][b, i, h])]
    merr = check_softmax_mass(ref.absorb_q_reference(x.f32("q_nope"), x.f32("w_uk")), x.f32("q_pe"), x.f32("pool"),
                              x.block_table, x.seq_lens, lse, rows, softmax_scale=w.softmax_scale, tol=tol)
    say("  softmax mass err", merr)
    assert not torch.isnan(bufs.out).any().item()


def test_end_to_end_tiny_fp32_full():
    say("end-to-end tiny_fp32 (all heads)")
    x = gen.generate_named("tiny_fp32", poison_unused=True)
    _end_to_end(x, [0], list(range(128)))


@pytest.mark.parametrize("name,seqs,heads", [
    ("b32_t4096", [0, 13, 31], [0, 37, 64, 127]),
    ("ragged_b128", [0, 77, 127], [5, 96]),
    ("mtp_b64_s2_t16384", [0, 63], [1, 127]),
    ("long_b4_t131072", [1, 3], [0, 100]),
])
def test_end_to_end_full_size(name, seqs, heads):
    say("end-to-end", name, "seqs", seqs, "heads", heads)
    x = gen.generate_named(name, poison_unused=True)
    _end_to_end(x, seqs, heads)


def test_end_to_end_small_mtp_all_heads():
    say("end-to-end small S=2 paged, all heads")
    w = gen.small_workload(2, 2, ragged=(66, 400), dtype="bf16", paged=True)
    x = gen.generate(w, 21, poison_unused=True)
    _end_to_end(x, [0, 1], list(range(128)))


# ------------------------------------------------------------------------------------ boundary
@pytest.mark.parametrize("variant", ["causal", "tree", "fp8", "fused", "fused fp8", "fused fp32"])
def test_graph_capture_replays_match_eager(variant):
    """The step's calls captured in one HIP graph; replays interleaved with eager work all match the
    eager run bit for bit (decode as is, with a draft-tree mask, with the FP8 projections, and the
    fused attention + merge/W_UV call in bf16 and FP8 at 16 rows, where the merge runs inside the
    W_UV kernel, and in fp32 at 2 rows, where it runs inside the out-projection's dot products)."""
    say("graph capture", variant)
    torch = _torch()
    S = 4 if variant == "tree" else 1
    B = 2 if variant == "fused fp32" else (16 if variant.startswith("fused") else 4)
    w = gen.small_workload(B, S, ragged=(200, 700), dtype="f32" if variant.endswith("fp32") else "bf16", paged=True)
    x = gen.generate(w, 23, poison_unused=True)
    d = to_device(x)
    p = params_for(x, causal=variant != "tree")
    kw = {}
    w_uk, w_uv = d["w_uk"], d["w_uv"]
    if variant == "tree":
        kw["tree_parents"] = torch.from_numpy(gen.draft_trees(4, S, 24)).cuda()
    if variant.startswith("fused"):
        kw["fused"] = True
    if variant.endswith("fp8"):
        w_uk = torch.empty(binding.mla_fp8_weight_bytes(), dtype=torch.uint8, device="cuda")
        w_uv = torch.empty_like(w_uk)
        binding.mla_quantize_w_uk_fp8(d["w_uk"], w_uk, p)
        binding.mla_quantize_w_uv_fp8(d["w_uv"], w_uv, p)
        kw["fp8"] = True
    args = (d["q_nope"], d["q_pe"], w_uk, w_uv, d["pool"], d["block_table"], d["seq_lens"])
    eager = binding.DecodeBuffers(p)
    eager.run(*args, **kw)
    torch.cuda.synchronize()
    ref_out, ref_lse = eager.out.clone(), eager.lse.clone()
    gb = binding.DecodeBuffers(p)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        gb.run(*args, **kw)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gb.run(*args, **kw)
    for it in range(4):
        gb.out.fill_(float("nan"))
        gb.lse.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda").sum()  # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(gb.out, ref_out) and torch.equal(gb.lse, ref_lse), it
        del junk


def test_error_leaves_outputs_untouched():
    say("error path canary")
    torch = _torch()
    w = gen.small_workload(2, 1, cache_len=300, dtype="bf16", paged=True)
    x = gen.generate(w, 25)
    d = to_device(x)
    p = params_for(x)
    q_lat = torch.zeros((2, 1, 128, 512), dtype=torch.bfloat16, device="cuda")
    o = torch.full((2, 1, 128, 512), 7.0, device="cuda")
    lse = torch.full((2, 1, 128), 7.0, device="cuda")
    need = binding.mla_decode_workspace_bytes(p, 3)
    small = torch.empty(need // 4 - 1, dtype=torch.float32, device="cuda")
    with pytest.raises(binding.MlaError) as e:
        binding.mla_decode_attn(q_lat, d["q_pe"], d["pool"], d["block_table"], d["seq_lens"], o, lse, small, 3, p)
    assert e.value.code == -5
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()) and bool((lse == 7.0).all())
