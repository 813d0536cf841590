"""Property-based GPU parity: hypothesis draws small decode batches and every one must match the oracle.

Drawn for the causal / full rule: batch 1..4, query tokens S in {1, 2}, per-sequence cache lengths L >= S (up to five pages, so
ragged last pages and multi-tile walks both occur), contiguous or randomly permuted pages, causal or
not, the split count (1, 2, 3, 5 or the library's own choice) and the dtype.  Unused pool slots are
NaN, so any read outside the sequences fails the NaN check.  Same bar as the fixed parity cases:
max |gpu - ref| / max |ref| <= 2e-2 (bf16) or 1e-4 (fp32) on o_lat, the same numbers in absolute
terms on lse, and on sampled rows the oracle's logits normalised by the GPU's lse sum to one within them.
Drawn for tree-masked verify: batch 1..3, trees of 1, 3, 8, 17 or 64 nodes with random parents
(several roots, and parents out of range, which end the ancestor walk), lengths 1..320 (so some
sequences hold fewer tokens than their tree), split counts and dtypes as above.
Drawn for the fused attention + out-projection (bf16, and its FP8 form): batch 1..24 and S in
{1, 2, 3}, so both of its routes run; split counts up to 9; the causal / full rule or a drawn
draft tree; the optional latent outputs on or off.
"""
import numpy as np
import pytest

from deepseek_mla_latent_amd import binding
from deepseek_mla_latent_amd import inputs as gen
from oracle import mla_decode as ref
from tests.helpers import (check_lse, check_softmax_mass, device_array, params_for, rel_err, sample_rows, to_device,
                           to_host, tol_for)

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import HealthCheck, given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402

pytestmark = pytest.mark.gpu


@st.composite
def decode_cases(draw):
    batch = draw(st.integers(1, 4))
    q_len = draw(st.sampled_from([1, 2]))
    lens = draw(st.lists(st.integers(q_len, 5 * 64), min_size=batch, max_size=batch))
    return dict(batch=batch, q_len=q_len, lens=lens, paged=draw(st.booleans()), causal=draw(st.booleans()),
                splits=draw(st.sampled_from([0, 1, 2, 3, 5])), dtype=draw(st.sampled_from(["bf16", "f32"])),
                seed=draw(st.integers(0, 2**31 - 1)))


@settings(max_examples=40, deadline=None, derandomize=True, suppress_health_check=list(HealthCheck))
@given(case=decode_cases())
def test_attention_matches_oracle(case):
    import torch
    print("[case]", case, flush=True)
    w = gen.small_workload(case["batch"], case["q_len"], cache_len=1, dtype=case["dtype"], paged=case["paged"])
    x = gen.generate(w, case["seed"], poison_unused=True, seq_lens=case["lens"])
    q_lat, _ = gen.generate_latent(w, case["seed"] + 1)
    d = to_device(x)
    p = params_for(x, causal=case["causal"])
    o = torch.full((w.batch, w.q_len, 128, 512), float("nan"), device="cuda")
    lse = torch.full((w.batch, w.q_len, 128), float("nan"), device="cuda")
    ws_bytes = binding.mla_decode_workspace_bytes(p, case["splits"])
    ws = torch.empty(max(ws_bytes, 16) // 4, dtype=torch.float32, device="cuda") if ws_bytes else None
    binding.mla_decode_attn(device_array(q_lat, x.is_bf16), d["q_pe"], d["pool"], d["block_table"],
                            d["seq_lens"], o, lse, ws, case["splits"], p)
    torch.cuda.synchronize()
    o, lse = to_host(o), to_host(lse)

    q_lat_f32 = gen.bf16_bits_to_f32(q_lat) if x.is_bf16 else q_lat
    want = ref.latent_attention_reference(q_lat_f32, x.f32("q_pe"), x.f32("pool"), x.block_table, x.seq_lens,
                                          softmax_scale=w.softmax_scale, causal=case["causal"])
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    assert rel_err(o, want["o_lat"]) <= tol_for(x)
    check_lse(lse, want["lse"], tol_for(x))
    check_softmax_mass(q_lat_f32, x.f32("q_pe"), x.f32("pool"), x.block_table, x.seq_lens, lse,
                       sample_rows(want["lse"], n=16, seed=case["seed"]), softmax_scale=w.softmax_scale,
                       tol=tol_for(x), causal=case["causal"])


@st.composite
def tree_cases(draw):
    """Draft trees as parent tables: each node's parent is -1 or an earlier node, with an occasional
    out-of-range parent (>= j or < -1), which ends that node's ancestor walk."""
    batch = draw(st.integers(1, 3))
    q_len = draw(st.sampled_from([1, 3, 8, 17, 64]))
    parents = []
    for _ in range(batch):
        row = []
        for j in range(q_len):
            kind = draw(st.integers(0, 9))
            if kind == 0:
                row.append(-1)
            elif kind == 1:
                row.append(draw(st.sampled_from([j, j + 3, -2, 1000])))  # out of range: a root in effect
            else:
                row.append(draw(st.integers(0, j - 1)) if j > 0 else -1)
        parents.append(row)
    lens = draw(st.lists(st.integers(1, 5 * 64), min_size=batch, max_size=batch))
    return dict(batch=batch, q_len=q_len, parents=parents, lens=lens, paged=draw(st.booleans()),
                splits=draw(st.sampled_from([0, 1, 2, 3, 5])), dtype=draw(st.sampled_from(["bf16", "f32"])),
                seed=draw(st.integers(0, 2**31 - 1)))


@settings(max_examples=30, deadline=None, derandomize=True, suppress_health_check=list(HealthCheck))
@given(case=tree_cases())
def test_tree_attention_matches_oracle(case):
    """mla_decode_attn_tree on drawn trees (lengths may be shorter than the tree) against the oracle
    run on the same tree with out-of-range parents replaced by -1."""
    import torch
    print("[case]", case, flush=True)
    w = gen.small_workload(case["batch"], case["q_len"], cache_len=1, dtype=case["dtype"], paged=case["paged"])
    x = gen.generate(w, case["seed"], poison_unused=True, seq_lens=case["lens"])
    q_lat, _ = gen.generate_latent(w, case["seed"] + 1)
    parents = np.array(case["parents"], dtype=np.int32).reshape(case["batch"], case["q_len"])
    d = to_device(x)
    p = params_for(x, causal=False)
    o = torch.full((w.batch, w.q_len, 128, 512), float("nan"), device="cuda")
    lse = torch.full((w.batch, w.q_len, 128), float("nan"), device="cuda")
    ws_bytes = binding.mla_decode_workspace_bytes(p, case["splits"])
    ws = torch.empty(max(ws_bytes, 16) // 4, dtype=torch.float32, device="cuda") if ws_bytes else None
    binding.mla_decode_attn_tree(device_array(q_lat, x.is_bf16), d["q_pe"], d["pool"], d["block_table"],
                                 d["seq_lens"], torch.from_numpy(parents).cuda(), o, lse, ws, case["splits"], p)
    torch.cuda.synchronize()
    o, lse = to_host(o), to_host(lse)

    valid = np.where((parents >= -1) & (parents < np.arange(case["q_len"])[None, :]), parents, -1)
    q_lat_f32 = gen.bf16_bits_to_f32(q_lat) if x.is_bf16 else q_lat
    want = ref.latent_attention_reference(q_lat_f32, x.f32("q_pe"), x.f32("pool"), x.block_table, x.seq_lens,
                                          softmax_scale=w.softmax_scale, tree=valid)
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    assert rel_err(o, want["o_lat"]) <= tol_for(x)
    check_lse(lse, want["lse"], tol_for(x))
    check_softmax_mass(q_lat_f32, x.f32("q_pe"), x.f32("pool"), x.block_table, x.seq_lens, lse,
                       sample_rows(want["lse"], n=16, seed=case["seed"]), softmax_scale=w.softmax_scale,
                       tol=tol_for(x), tree=valid)


@st.composite
def fused_cases(draw):
    batch = draw(st.integers(1, 24))
    q_len = draw(st.sampled_from([1, 2, 3]))
    lens = draw(st.lists(st.integers(q_len, 5 * 64), min_size=batch, max_size=batch))
    tree = draw(st.booleans())
    parents = [[draw(st.integers(-1, j - 1)) for j in range(q_len)] for _ in range(batch)] if tree else None
    return dict(batch=batch, q_len=q_len, lens=lens, paged=draw(st.booleans()), causal=draw(st.booleans()),
                parents=parents, splits=draw(st.sampled_from([0, 1, 2, 3, 5, 9])), latent=draw(st.booleans()),
                seed=draw(st.integers(0, 2**31 - 1)))


@settings(max_examples=30, deadline=None, derandomize=True, suppress_health_check=list(HealthCheck))
@given(case=fused_cases())
def test_fused_attention_out_proj_matches_oracle(case):
    """mla_decode_attn_out_proj (bf16) on drawn batches, on both of its routes (fewer or more than
    16 query rows; one or several splits), with or without a draft tree and the latent outputs:
    out against W_UV^T of the oracle's latent attention, o_lat and lse when asked for."""
    import torch
    print("[case]", case, flush=True)
    w = gen.small_workload(case["batch"], case["q_len"], cache_len=1, dtype="bf16", paged=case["paged"])
    x = gen.generate(w, case["seed"], poison_unused=True, seq_lens=case["lens"])
    q_lat, _ = gen.generate_latent(w, case["seed"] + 1)
    d = to_device(x)
    p = params_for(x, causal=case["causal"])
    parents = None if case["parents"] is None else np.array(case["parents"], dtype=np.int32)
    out = torch.full((w.batch, w.q_len, 128, 128), float("nan"), device="cuda").to(torch.bfloat16)
    o = torch.full((w.batch, w.q_len, 128, 512), float("nan"), device="cuda") if case["latent"] else None
    lse = torch.full((w.batch, w.q_len, 128), float("nan"), device="cuda") if case["latent"] else None
    ws_bytes = binding.mla_decode_attn_out_proj_workspace_bytes(p, case["splits"])
    ws = torch.full((max(ws_bytes, 16) // 4,), float("nan"), device="cuda")
    binding.mla_decode_attn_out_proj(device_array(q_lat, True), d["q_pe"], d["pool"], d["block_table"],
                                     d["seq_lens"], None if parents is None else torch.from_numpy(parents).cuda(),
                                     d["w_uv"], out, o, lse, ws, case["splits"], p)
    torch.cuda.synchronize()

    want = ref.latent_attention_reference(gen.bf16_bits_to_f32(q_lat), x.f32("q_pe"), x.f32("pool"), x.block_table,
                                          x.seq_lens, softmax_scale=w.softmax_scale, causal=case["causal"],
                                          tree=parents)
    got = to_host(out)
    assert not np.isnan(got).any()
    assert rel_err(got, ref.out_proj_reference(want["o_lat"], x.f32("w_uv"))) <= tol_for(x)
    if case["latent"]:
        o, lse = to_host(o), to_host(lse)
        assert not np.isnan(o).any() and not np.isnan(lse).any()
        assert rel_err(o, want["o_lat"]) <= tol_for(x)
        check_lse(lse, want["lse"], tol_for(x))
        check_softmax_mass(gen.bf16_bits_to_f32(q_lat), x.f32("q_pe"), x.f32("pool"), x.block_table, x.seq_lens, lse,
                           sample_rows(want["lse"], n=16, seed=case["seed"]), softmax_scale=w.softmax_scale,
                           tol=tol_for(x), causal=case["causal"], tree=parents)


@settings(max_examples=20, deadline=None, derandomize=True, suppress_health_check=list(HealthCheck))
@given(case=fused_cases())
def test_fused_attention_out_proj_fp8_matches_oracle(case):
    """mla_decode_attn_out_proj_fp8 on the same drawn batches: out against the oracle's FP8
    out-projection of its latent attention, within 2e-2 plus the oracle's own distance between its
    FP8 products of the bf16-rounded and of the exact o_lat (the call codes merged rows that carry
    one bf16 rounding), and within the oracle's own FP8 error plus 2e-2 of the unquantised product;
    o_lat and lse at the bf16 bar when asked for."""
    import torch
    from oracle import fp8 as ref8
    print("[case]", case, flush=True)
    w = gen.small_workload(case["batch"], case["q_len"], cache_len=1, dtype="bf16", paged=case["paged"])
    x = gen.generate(w, case["seed"], poison_unused=True, seq_lens=case["lens"])
    q_lat, _ = gen.generate_latent(w, case["seed"] + 1)
    d = to_device(x)
    p = params_for(x, causal=case["causal"])
    parents = None if case["parents"] is None else np.array(case["parents"], dtype=np.int32)
    uv = torch.zeros(binding.mla_fp8_weight_bytes(), dtype=torch.uint8, device="cuda")
    binding.mla_quantize_w_uv_fp8(d["w_uv"], uv, p)
    out = torch.full((w.batch, w.q_len, 128, 128), float("nan"), device="cuda").to(torch.bfloat16)
    o = torch.full((w.batch, w.q_len, 128, 512), float("nan"), device="cuda") if case["latent"] else None
    lse = torch.full((w.batch, w.q_len, 128), float("nan"), device="cuda") if case["latent"] else None
    ws_bytes = binding.mla_decode_attn_out_proj_workspace_bytes(p, case["splits"])
    ws = torch.full((max(ws_bytes, 16) // 4,), float("nan"), device="cuda")
    binding.mla_decode_attn_out_proj_fp8(device_array(q_lat, True), d["q_pe"], d["pool"], d["block_table"],
                                         d["seq_lens"], None if parents is None else torch.from_numpy(parents).cuda(),
                                         uv, out, o, lse, ws, case["splits"], p)
    torch.cuda.synchronize()

    want = ref.latent_attention_reference(gen.bf16_bits_to_f32(q_lat), x.f32("q_pe"), x.f32("pool"), x.block_table,
                                          x.seq_lens, softmax_scale=w.softmax_scale, causal=case["causal"],
                                          tree=parents)
    o_ref = want["o_lat"].astype(np.float32)
    fp8_ref, _, _ = ref8.out_proj_fp8_reference(o_ref, x.f32("w_uv"))
    moved, _, _ = ref8.out_proj_fp8_reference(gen.bf16_bits_to_f32(gen.round_to_bf16_bits(o_ref)), x.f32("w_uv"))
    exact = ref.out_proj_reference(want["o_lat"], x.f32("w_uv"))
    got = to_host(out)
    assert not np.isnan(got).any()
    sens, q_err = rel_err(moved, fp8_ref), rel_err(fp8_ref, exact)
    err, err_exact = rel_err(got, fp8_ref), rel_err(got, exact)
    print(f"[case]   out vs fp8 oracle {err:.2e} (bar 2e-2 + {sens:.2e}), vs unquantised {err_exact:.2e} "
          f"(bar {q_err:.2e} + 2e-2)", flush=True)
    assert err <= 2e-2 + sens and err_exact <= q_err + 2e-2
    if case["latent"]:
        o, lse = to_host(o), to_host(lse)
        assert not np.isnan(o).any() and not np.isnan(lse).any()
        assert rel_err(o, want["o_lat"]) <= tol_for(x)
        check_lse(lse, want["lse"], tol_for(x))
