"""GPU parity of the fused attention + out-projection (mla_decode_attn_out_proj) against the fp64
oracle: out = W_UV^T o_lat with (o_lat, lse) the latent attention over the visible keys.

Bar as for the separate calls: max |gpu - ref| / max |ref| <= 2e-2 per output tensor (bf16); lse
within 2e-2 in absolute terms and -inf exactly where the oracle has it, and the oracle's logits of
sampled rows normalised by the GPU's lse sum to one within 2e-2.  Unused
cache slots hold NaN, so a read outside the sequences shows up as NaN.  The optional latent outputs
must not change `out`, which is checked bit for bit.
"""
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


def _run_fused(x, q_lat_bits, splits, causal=True, parents=None, latent=True):
    import torch
    d = to_device(x)
    p = params_for(x, causal=causal)
    w = x.workload
    q_lat = device_array(q_lat_bits, x.is_bf16)
    par = None if parents is None else torch.from_numpy(np.ascontiguousarray(parents, dtype=np.int32)).cuda()
    out = torch.full((w.batch, w.q_len, 128, 128), float("nan"), device="cuda").to(
        torch.bfloat16 if x.is_bf16 else torch.float32)
    o = torch.full((w.batch, w.q_len, 128, 512), float("nan"), device="cuda") if latent else None
    lse = torch.full((w.batch, w.q_len, 128), float("nan"), device="cuda") if latent else None
    ws_bytes = binding.mla_decode_attn_out_proj_workspace_bytes(p, splits)
    ws = torch.full((ws_bytes // 4,), float("nan"), device="cuda")
    binding.mla_decode_attn_out_proj(q_lat, d["q_pe"], d["pool"], d["block_table"], d["seq_lens"], par, d["w_uv"],
                                     out, o, lse, ws, splits, p)
    torch.cuda.synchronize()
    return to_host(out), (to_host(o) if latent else None), (to_host(lse) if latent else None)


def _check(x, q_lat_bits, splits, causal=True, parents=None):
    out, o, lse = _run_fused(x, q_lat_bits, splits, causal, parents)
    q = gen.bf16_bits_to_f32(q_lat_bits) if x.is_bf16 else q_lat_bits
    want = ref.latent_attention_reference(q, x.f32("q_pe"), x.f32("pool"),
                                          x.block_table, x.seq_lens, softmax_scale=x.workload.softmax_scale,
                                          causal=causal, tree=parents)
    want_out = ref.out_proj_reference(want["o_lat"], x.f32("w_uv"))
    for name, got in (("out", out), ("o_lat", o), ("lse", lse)):
        assert not np.isnan(got).any(), name
    errs = {"out": rel_err(out, want_out), "o_lat": rel_err(o, want["o_lat"])}
    say("  rel errs", errs)
    for k, e in errs.items():
        assert e <= tol_for(x), k
    check_lse(lse, want["lse"], tol_for(x))
    check_softmax_mass(q, x.f32("q_pe"), x.f32("pool"), x.block_table, x.seq_lens, lse,
                       sample_rows(want["lse"]), softmax_scale=x.workload.softmax_scale, tol=tol_for(x),
                       causal=causal, tree=parents)
    bare, _, _ = _run_fused(x, q_lat_bits, splits, causal, parents, latent=False)
    assert np.array_equal(bare, out)


@pytest.mark.parametrize("splits", [1, 2, 3, 0])
def test_fused_ragged_paged(splits):
    say("fused ragged paged, splits", splits)
    w = gen.small_workload(3, 1, ragged=(1, 300), dtype="bf16", paged=True)
    x = gen.generate(w, 7, poison_unused=True)
    q_lat, _ = gen.generate_latent(w, 8)
    _check(x, q_lat, splits)


def test_fused_routes():
    """Which kernels run: the merge inside the W_UV kernel needs 16 query rows and two splits."""
    mk = lambda B: binding.make_params(batch=B, q_len=1, max_seq_len=300, softmax_scale=0.1,  # noqa: E731
                                       dtype=binding.MLA_BF16)
    ws = binding.mla_decode_attn_out_proj_workspace_bytes
    olat = 128 * 512 * 4
    assert ws(mk(16), 2) == 16 * 2 * 128 * (512 * 2 + 4) + 16 + 16 * 8  # + the range plan (header, rows)
    assert ws(mk(16), 1) == 16 * olat
    assert ws(mk(15), 2) == binding.mla_decode_workspace_bytes(mk(15), 2) + 15 * olat


def test_fused_edge_lengths():
    """Empty (out 0, lse -inf), single-token, page-boundary and off-by-one lengths."""
    lens = [0, 1, 63, 64, 65, 128, 129, 2]
    w = gen.small_workload(len(lens), 1, cache_len=1, dtype="bf16", paged=True)
    x = gen.generate(w, 11, poison_unused=True, seq_lens=lens)
    q_lat, _ = gen.generate_latent(w, 12)
    for splits in (1, 2, 0):
        say("fused edge lengths", lens, "splits", splits)
        _check(x, q_lat, splits)


@pytest.mark.parametrize("B,S,causal", [(5, 1, True), (3, 7, True), (3, 2, False), (17, 1, True)])
def test_fused_row_blocks(B, S, causal):
    """Row counts that do not fill the 16-row blocks of the merge (5, 21, 6, 17 rows)."""
    say("fused rows", B * S, "causal", causal)
    w = gen.small_workload(B, S, ragged=(S, 200), dtype="bf16", paged=True)
    x = gen.generate(w, 30 + B, poison_unused=True)
    q_lat, _ = gen.generate_latent(w, 31 + B)
    _check(x, q_lat, 0, causal)
    _check(x, q_lat, 2, causal)


def test_fused_many_splits():
    """More splits than the two batches of four the merge keeps in flight (24 two-page and 47
    one-page ranges), over one full 16-row block, so the merge runs inside the W_UV kernel."""
    lens = [3000, 2500] + [1200 + 97 * i for i in range(14)]
    w = gen.small_workload(len(lens), 1, cache_len=1, dtype="bf16", paged=True)
    x = gen.generate(w, 51, poison_unused=True, seq_lens=lens)
    q_lat, _ = gen.generate_latent(w, 52)
    for splits in (24, 47):
        say("fused splits", splits)
        _check(x, q_lat, splits)


@pytest.mark.parametrize("B,S,splits", [(1, 1, 0), (3, 1, 0), (2, 2, 3), (1, 1, 1), (6, 1, 0)])
def test_fused_fp32(B, S, splits):
    """fp32 (bar 1e-4): with at most 4 query rows and several splits the merge of the fp32 partials
    runs inside the out-projection's dot products; one split, or more rows, take the separate
    kernels."""
    say("fused fp32 B", B, "S", S, "splits", splits)
    w = gen.small_workload(B, S, ragged=(40, 700), dtype="f32", paged=True)
    x = gen.generate(w, 50 + 10 * B + S, poison_unused=True)
    q_lat, _ = gen.generate_latent(w, 70 + B)
    _check(x, q_lat, splits)


def test_fused_fp32_tiny_full_size():
    """The tiny fp32 workload (1 row, 512 cached tokens, contiguous) through the fused call, every
    head."""
    say("fused fp32 tiny_fp32")
    x = gen.generate_named("tiny_fp32", poison_unused=True)
    q_lat, _ = gen.generate_latent(x.workload, 71)
    _check(x, q_lat, 0)


@pytest.mark.parametrize("S,splits", [(8, 0), (8, 3), (64, 1)])
def test_fused_tree(S, splits):
    say("fused tree S", S, "splits", splits)
    lens = [S + 100, 70, max(S - 1, 1)]
    w = gen.small_workload(len(lens), S, cache_len=1, dtype="bf16", paged=True)
    x = gen.generate(w, 60 + S, poison_unused=True, seq_lens=lens)
    q_lat, _ = gen.generate_latent(w, 61 + S)
    parents = gen.draft_trees(len(lens), S, 62 + S)
    _check(x, q_lat, splits, causal=False, parents=parents)


@pytest.mark.parametrize("name,seqs,heads", [
    ("b32_t4096", [0, 13, 31], [0, 37, 64, 127]),
    ("ragged_b128", [0, 77, 127], [5, 96]),
    ("mtp_b64_s2_t16384", [0, 63], [1, 127]),
    ("tree_b32_s8_t4096", [0, 17, 31], [3, 64, 126]),
])
def test_fused_step_full_size_sampled(name, seqs, heads):
    """The whole fused step (absorb -> attention + merge + W_UV) at the benchmark sizes against the
    non-absorbed oracle on sampled sequences and heads (the draft-tree workload through its
    parents; at one split it takes the separate kernels)."""
    import torch
    tree = name in gen.TREE_WORKLOADS
    x = gen.generate_named(name, poison_unused=True)
    parents = gen.draft_trees(x.workload.batch, x.workload.q_len, gen.TREE_SEEDS[name]) if tree else None
    say("fused full size", name, seqs, heads)
    d = to_device(x)
    p = params_for(x, causal=not tree)
    bufs = binding.DecodeBuffers(p, 0)
    bufs.run(d["q_nope"], d["q_pe"], d["w_uk"], d["w_uv"], d["pool"], d["block_table"], d["seq_lens"], fused=True,
             tree_parents=None if parents is None else torch.from_numpy(parents).cuda())
    torch.cuda.synchronize()
    w = x.workload
    r = ref.mla_decode_nonabsorbed(x.f32("q_nope"), x.f32("q_pe"), x.f32("w_uk"), x.f32("w_uv"), x.f32("pool"),
                                   x.block_table, x.seq_lens, softmax_scale=w.softmax_scale, seqs=seqs, heads=heads,
                                   tree=parents)
    sel = np.ix_(seqs, range(w.q_len), heads)
    errs = {k: rel_err(to_host(getattr(bufs, k))[sel], r[k][sel]) for k in ("o_lat", "out")}
    say("  rel errs", errs)
    for k, e in errs.items():
        assert e <= tol_for(x), k
    assert not torch.isnan(bufs.out).any().item()


def test_fused_graph_replays_match_eager():
    """The fused step captured in a HIP graph: every replay equals the eager result bit for bit,
    with eager work and synchronisations between the replays."""
    import torch
    w = gen.small_workload(4, 1, ragged=(64, 700), dtype="bf16", paged=True)
    x = gen.generate(w, 71, poison_unused=True)
    d = to_device(x)
    p = params_for(x)
    bufs = binding.DecodeBuffers(p, 0)

    def run():
        bufs.run(d["q_nope"], d["q_pe"], d["w_uk"], d["w_uv"], d["pool"], d["block_table"], d["seq_lens"],
                 fused=True, latent_outputs=False)

    run()
    torch.cuda.synchronize()
    eager = bufs.out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for k in range(3):
        bufs.out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        say("  replay", k)
        assert torch.equal(bufs.out, eager)
        run()
        torch.cuda.synchronize()
