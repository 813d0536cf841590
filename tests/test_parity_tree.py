"""GPU parity of tree-masked verify (mla_decode_attn_tree) against the fp64 oracle.

Bar as for the attention call: max |gpu - ref| / max |ref| <= 2e-2 (bf16) and <= 1e-4 (fp32) for
o_lat; lse within the same numbers in absolute terms, -inf exactly where the oracle has it; on
sampled rows the oracle's logits normalised by the GPU's lse sum to one within them.
Unused cache slots hold NaN, so a read outside the sequences shows up as NaN.
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


def _run_tree(x, q_lat_bits, parents, splits, seqs=None):
    import torch
    d = to_device(x)
    p = params_for(x, causal=False)
    w = x.workload
    q_lat = device_array(q_lat_bits, x.is_bf16)
    par = torch.from_numpy(np.ascontiguousarray(parents, dtype=np.int32)).cuda()
    o = torch.full((w.batch, w.q_len, 128, 512), float("nan"), device="cuda")
    lse = torch.full((w.batch, w.q_len, 128), float("nan"), device="cuda")
    ws_bytes = binding.mla_decode_workspace_bytes(p, splits)
    ws = torch.empty(max(ws_bytes, 16) // 4, dtype=torch.float32, device="cuda") if ws_bytes else None
    binding.mla_decode_attn_tree(q_lat, d["q_pe"], d["pool"], d["block_table"], d["seq_lens"], par, o, lse, ws,
                                 splits, p)
    torch.cuda.synchronize()
    return to_host(o), to_host(lse)


def _check(x, q_lat_bits, parents, o, lse, seqs=None, oracle_parents=None):
    q = gen.bf16_bits_to_f32(q_lat_bits) if x.is_bf16 else q_lat_bits
    want = ref.latent_attention_reference(q, x.f32("q_pe"), x.f32("pool"), x.block_table, x.seq_lens,
                                          softmax_scale=x.workload.softmax_scale, seqs=seqs,
                                          tree=parents if oracle_parents is None else oracle_parents)
    sel = slice(None) if seqs is None else list(seqs)
    o, lse, wo, wl = o[sel], lse[sel], want["o_lat"][sel], want["lse"][sel]
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    err = rel_err(o, wo)
    say("  o_lat rel err", err)
    assert err <= tol_for(x)
    check_lse(lse, wl, tol_for(x))
    tree = parents if oracle_parents is None else oracle_parents
    full = np.full(want["lse"].shape, np.nan)
    full[sel] = lse
    check_softmax_mass(q, x.f32("q_pe"), x.f32("pool"), x.block_table, x.seq_lens, full,
                       sample_rows(want["lse"], seqs=None if seqs is None else list(seqs)),
                       softmax_scale=x.workload.softmax_scale, tol=tol_for(x), tree=tree)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("S,splits", [(2, 1), (7, 2), (7, 0), (16, 3), (64, 1), (64, 0)])
def test_tree_attention(dtype, S, splits):
    say("tree attn", dtype, "S", S, "splits", splits)
    lens = [S + 100, 70, max(S - 1, 1)]  # the last one holds fewer tokens than the tree has nodes
    w = gen.small_workload(len(lens), S, cache_len=1, dtype=dtype, paged=True)
    x = gen.generate(w, 100 + S, poison_unused=True, seq_lens=lens)
    q_lat, _ = gen.generate_latent(w, 200 + S)
    parents = gen.draft_trees(len(lens), S, 300 + S)
    o, lse = _run_tree(x, q_lat, parents, splits)
    _check(x, q_lat, parents, o, lse)


def test_tree_masked_tiles_and_splits():
    """Two chains (nodes 0-39 and 40-63) cached at 128..191 and at 96..159: with one page per
    split, a whole split (and a range's first tile) can be hidden from a node, e.g. node 63 sees
    none of nodes 0-31 and node 5 none of nodes 32-63."""
    S = 64
    parents = np.arange(-1, S - 1, dtype=np.int32)
    parents[40] = -1
    for lens in ([192, 160], [160, 192]):
        say("tree masked splits", lens)
        w = gen.small_workload(2, S, cache_len=1, dtype="bf16", paged=True)
        x = gen.generate(w, 41, poison_unused=True, seq_lens=lens)
        q_lat, _ = gen.generate_latent(w, 42)
        tree = np.stack([parents, parents])
        for splits in (3, 2, 1):
            o, lse = _run_tree(x, q_lat, tree, splits)
            _check(x, q_lat, tree, o, lse)


def test_chain_tree_matches_the_causal_call():
    import torch
    S = 5
    say("chain tree vs causal")
    w = gen.small_workload(3, S, ragged=(S, 400), dtype="bf16", paged=True)
    x = gen.generate(w, 51, poison_unused=True)
    q_lat, _ = gen.generate_latent(w, 52)
    chain = np.tile(np.arange(-1, S - 1, dtype=np.int32), (3, 1))
    o_t, lse_t = _run_tree(x, q_lat, chain, 2)
    d = to_device(x)
    p = params_for(x, causal=True)
    o = torch.full((3, S, 128, 512), float("nan"), device="cuda")
    lse = torch.full((3, S, 128), float("nan"), device="cuda")
    ws = torch.empty(binding.mla_decode_workspace_bytes(p, 2) // 4, dtype=torch.float32, device="cuda")
    binding.mla_decode_attn(device_array(q_lat, True), d["q_pe"], d["pool"], d["block_table"], d["seq_lens"], o, lse,
                            ws, 2, p)
    torch.cuda.synchronize()
    assert rel_err(o_t, to_host(o)) <= 1e-5
    assert np.max(np.abs(lse_t - to_host(lse))) <= 1e-5


def test_parents_outside_the_range_end_the_walk():
    """A parent >= j (or < -1) ends node j's ancestor walk: the result equals the tree with -1 there."""
    S = 6
    say("tree invalid parents")
    bad = np.array([[-1, 0, 5, 1, -7, 4]], dtype=np.int32)  # node 2 names a later node, node 4 -7
    fixed = np.array([[-1, 0, -1, 1, -1, 4]], dtype=np.int32)
    w = gen.small_workload(1, S, cache_len=1, dtype="f32", paged=True)
    x = gen.generate(w, 61, poison_unused=True, seq_lens=[90])
    q_lat, _ = gen.generate_latent(w, 62)
    o, lse = _run_tree(x, q_lat, bad, 0)
    _check(x, q_lat, bad, o, lse, oracle_parents=fixed)


def test_tree_verify_at_decode_size_sampled():
    """32 sequences of 4096 cached tokens, 8-node draft trees (bf16), library split choice; the
    oracle checks four sampled sequences whole."""
    S = 8
    say("tree verify b32 t4096 S8")
    w = gen.small_workload(32, S, cache_len=4096, dtype="bf16", paged=True)
    x = gen.generate(w, 71, poison_unused=True)
    q_lat, _ = gen.generate_latent(w, 72)
    parents = gen.draft_trees(32, S, 73)
    o, lse = _run_tree(x, q_lat, parents, 0)
    _check(x, q_lat, parents, o, lse, seqs=[0, 9, 22, 31])
