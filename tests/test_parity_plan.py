"""GPU: the key ranges of the split attention follow the rows' lengths.

With k > 1 ranges per row and at most 256 query rows, the attention cuts row r (P_r pages of
visible keys) into max(1, ceil(P_r / C)) ranges of C pages, C the smallest page count for which the
rows need at most rows * k ranges, numbered row after row; the per-row (first slot, count) table it
leaves after the partials in the workspace is what the merges read.  Above 256 rows every row gets
k ranges.  Each case compares that table with the plan restated here from its definition (C by a
plain scan, not the kernel's bisection) and the outputs with the fp64 oracle, on batches where the
plan differs from k equal ranges per row: one long row among short ones, S = 2 with the causal rule,
both merges (the separate one and the one inside the W_UV kernel), and the 256-row boundary.
Bar: as in test_parity.py.
"""
import numpy as np
import pytest

from deepseek_mla_latent_amd import binding
from deepseek_mla_latent_amd import inputs as gen
from oracle import mla_decode as ref
from tests.helpers import (check_lse, check_softmax_mass, device_array, params_for, rel_err, sample_rows, to_device,
                           to_host, tol_for)

pytestmark = pytest.mark.gpu

PAGE = 64


def say(*a):
    print("[case]", *a, flush=True)


def _cdiv(a, b):
    return -(-a // b)


def plan_reference(x, k, causal=True, budget=None):
    """(first, count) per row and the chunk C, from the plan's definition (budget: the ranges the
    rows may take, rows * k unless the library allows more)."""
    w = x.workload
    S = w.q_len
    rows = w.batch * S
    max_pages = _cdiv(x.max_seq_len, PAGE)
    pps = _cdiv(max_pages, k)  # pages per fixed range (k as the library reports it)
    pages = []
    for r in range(rows):
        b, i = divmod(r, S)
        L = int(x.seq_lens[b])
        n = min(max(L - S + i + 1, 0), L) if causal else L
        pages.append(min(_cdiv(n, PAGE), k * pps))
    if rows > 256:
        return [(r * k, k) for r in range(rows)], pps
    G = rows * k if budget is None else budget
    C = next(c for c in range(1, pps + 1) if sum(max(1, _cdiv(p, c)) for p in pages) <= G)
    counts = [max(1, _cdiv(p, C)) for p in pages]
    firsts = np.concatenate([[0], np.cumsum(counts)[:-1]]).astype(int)
    return list(zip(firsts.tolist(), counts)), C


def _table(ws, x, k, elem, slots=None):
    """The plan after the partials (`slots` of them, rows * k by default): header word 0 (1: every
    row has k fixed slots), then the rows."""
    rows = x.workload.batch * x.workload.q_len
    off = (rows * k if slots is None else slots) * 128 * (512 * elem + 4)
    t = ws.view(-1).view(__import__("torch").int32)[off // 4: off // 4 + 4 + 2 * rows].cpu().numpy()
    entries = [(int(t[4 + 2 * r]), int(t[4 + 2 * r + 1])) for r in range(rows)]
    assert int(t[0]) == int(entries == [(r * k, k) for r in range(rows)])
    return entries


def _oracle(x, q_lat_bits, causal):
    q = gen.bf16_bits_to_f32(q_lat_bits) if x.is_bf16 else q_lat_bits
    return q, ref.latent_attention_reference(q, x.f32("q_pe"), x.f32("pool"), x.block_table, x.seq_lens,
                                             softmax_scale=x.workload.softmax_scale, causal=causal)


def _check_attn(x, seed, splits, causal=True):
    import torch
    w = x.workload
    q_lat_bits, _ = gen.generate_latent(w, seed)
    d = to_device(x)
    p = params_for(x, causal=causal)
    k = binding.mla_decode_num_splits(p, splits)
    o = torch.full((w.batch, w.q_len, 128, 512), float("nan"), device="cuda")
    lse = torch.full((w.batch, w.q_len, 128), float("nan"), device="cuda")
    nb = binding.mla_decode_workspace_bytes(p, splits)
    ws = torch.full((nb // 4,), float("nan"), device="cuda")
    binding.mla_decode_attn(device_array(q_lat_bits, x.is_bf16), d["q_pe"], d["pool"], d["block_table"],
                            d["seq_lens"], o, lse, ws, splits, p)
    torch.cuda.synchronize()
    want_plan, C = plan_reference(x, k, causal)
    got_plan = _table(ws, x, k, 2 if x.is_bf16 else 4)
    say("  k", k, "chunk", C, "most ranges in a row", max(c for _, c in want_plan))
    assert got_plan == want_plan
    q, want = _oracle(x, q_lat_bits, causal)
    o, lse = to_host(o), to_host(lse)
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    err = rel_err(o, want["o_lat"])
    check_lse(lse, want["lse"], tol_for(x))
    check_softmax_mass(q, x.f32("q_pe"), x.f32("pool"), x.block_table, x.seq_lens, lse,
                       sample_rows(want["lse"], seed=seed), softmax_scale=w.softmax_scale, tol=tol_for(x),
                       causal=causal)
    say("  o_lat rel err", err)
    assert err <= tol_for(x)
    return want_plan


def _skewed_lens(n, long_len, lo, hi, seed):
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi, size=n).astype(np.int32)
    lens[n // 3] = long_len
    return lens


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_plan_one_long_row(dtype):
    lens = _skewed_lens(24, 4000, 30, 400, 1)
    say("plan: one long row among 23 short", dtype)
    w = gen.small_workload(len(lens), 1, cache_len=1, dtype=dtype, paged=True)
    x = gen.generate(w, 31, poison_unused=True, seq_lens=lens)
    plan = _check_attn(x, 32, 4)
    assert max(c for _, c in plan) > 4  # the long row got more ranges than the fixed split
    assert plan != [(4 * r, 4) for r in range(len(lens))]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_plan_two_query_tokens_causal(dtype):
    lens = _skewed_lens(20, 1500, 2, 300, 2)
    lens[3] = 1  # shorter than S: its first row sees nothing
    say("plan: S = 2, causal, ragged", dtype)
    w = gen.small_workload(len(lens), 2, cache_len=1, dtype=dtype, paged=True)
    x = gen.generate(w, 33, poison_unused=True, seq_lens=lens)
    _check_attn(x, 34, 3)


def test_plan_empty_rows_and_all_equal():
    lens = np.array([0, 0, 512, 0, 512, 512, 0, 512], np.int32)
    say("plan: empty rows among equal ones")
    w = gen.small_workload(len(lens), 1, cache_len=1, dtype="bf16", paged=True)
    x = gen.generate(w, 35, poison_unused=True, seq_lens=lens)
    plan = _check_attn(x, 36, 4)
    assert all(c == 1 for (_, c), L in zip(plan, lens) if L == 0)
    lens = np.full(6, 700, np.int32)  # equal lengths: the fixed ranges
    x = gen.generate(gen.small_workload(6, 1, cache_len=1, dtype="bf16", paged=True), 37, poison_unused=True,
                     seq_lens=lens)
    plan = _check_attn(x, 38, 3)
    assert plan == [(3 * r, 3) for r in range(6)]


def test_plan_above_256_rows_is_fixed():
    lens = _skewed_lens(260, 300, 1, 130, 3)
    say("plan: 260 rows, fixed ranges")
    w = gen.small_workload(len(lens), 1, cache_len=1, dtype="bf16", paged=True)
    x = gen.generate(w, 39, poison_unused=True, seq_lens=lens)
    plan = _check_attn(x, 40, 2)
    assert plan == [(2 * r, 2) for r in range(len(lens))]


def test_plan_in_the_fused_merge():
    """The merge inside the W_UV kernel reads the same plan (32 rows: two 16-row blocks)."""
    import torch
    lens = _skewed_lens(32, 3000, 20, 500, 4)
    say("plan: fused route, one long row among 31")
    w = gen.small_workload(len(lens), 1, cache_len=1, dtype="bf16", paged=True)
    x = gen.generate(w, 41, poison_unused=True, seq_lens=lens)
    q_lat_bits, _ = gen.generate_latent(w, 42)
    d = to_device(x)
    p = params_for(x)
    splits = 4
    k = binding.mla_decode_num_splits(p, splits)
    out = torch.full((w.batch, 1, 128, 128), float("nan"), device="cuda").to(torch.bfloat16)
    o = torch.full((w.batch, 1, 128, 512), float("nan"), device="cuda")
    lse = torch.full((w.batch, 1, 128), float("nan"), device="cuda")
    nb = binding.mla_decode_attn_out_proj_workspace_bytes(p, splits)
    ws = torch.full((nb // 4,), float("nan"), device="cuda")
    binding.mla_decode_attn_out_proj(device_array(q_lat_bits, True), d["q_pe"], d["pool"], d["block_table"],
                                     d["seq_lens"], None, d["w_uv"], out, o, lse, ws, splits, p)
    torch.cuda.synchronize()
    want_plan, _ = plan_reference(x, k)
    assert _table(ws, x, k, 2) == want_plan
    assert max(c for _, c in want_plan) > k
    q, want = _oracle(x, q_lat_bits, True)
    want_out = ref.out_proj_reference(want["o_lat"], x.f32("w_uv"))
    out, o, lse = to_host(out), to_host(o), to_host(lse)
    errs = {"out": rel_err(out, want_out), "o_lat": rel_err(o, want["o_lat"])}
    say("  rel errs", errs)
    for name, e in errs.items():
        assert e <= tol_for(x), name
    check_lse(lse, want["lse"], tol_for(x))


def _longest_first_budget(rows, k):
    """Ranges the library lets rows of unequal length take with its own split choice (bf16): 9/8 of
    one per compute unit for 33..256 query rows, when rows * k is fewer."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    want = -(-9 * cus // 8)
    return want if 32 < rows <= 256 and k > 1 and rows * k < want else rows * k


@pytest.mark.parametrize("route", ["separate merge", "merge in out-projection"])
def test_plan_longest_first(route):
    """128 ragged rows with the library's split choice: more ranges than compute units, dispatched
    longest first.  Every row's slots and count match the plan restated here with the larger budget;
    every range is computed exactly once (workspace and outputs start as NaN, so a range left out
    shows); outputs match the oracle and a second call is bitwise equal."""
    import torch
    rng = np.random.default_rng(5)
    lens = rng.integers(1, 2200, size=128).astype(np.int32)
    lens[[7, 40, 99]] = 0          # empty rows: one empty range each, dispatched last
    lens[[3, 4, 5]] = 640          # equal remainders (ties broken by row)
    lens[60] = 4096                # a long row with several full ranges
    say("plan: longest first, 128 ragged rows,", route)
    w = gen.small_workload(len(lens), 1, cache_len=1, dtype="bf16", paged=True)
    x = gen.generate(w, 43, poison_unused=True, seq_lens=lens)
    q_lat_bits, _ = gen.generate_latent(w, 44)
    d = to_device(x)
    p = params_for(x)
    k = binding.mla_decode_num_splits(p, 0)
    budget = _longest_first_budget(len(lens), k)
    fused = route != "separate merge"

    def run():
        o = torch.full((w.batch, 1, 128, 512), float("nan"), device="cuda")
        lse = torch.full((w.batch, 1, 128), float("nan"), device="cuda")
        if fused:
            nb = binding.mla_decode_attn_out_proj_workspace_bytes(p, 0)
            ws = torch.full((nb // 4,), float("nan"), device="cuda")
            out = torch.full((w.batch, 1, 128, 128), float("nan"), device="cuda").to(torch.bfloat16)
            binding.mla_decode_attn_out_proj(device_array(q_lat_bits, True), d["q_pe"], d["pool"], d["block_table"],
                                             d["seq_lens"], None, d["w_uv"], out, o, lse, ws, 0, p)
        else:
            nb = binding.mla_decode_workspace_bytes(p, 0)
            ws = torch.full((nb // 4,), float("nan"), device="cuda")
            out = None
            binding.mla_decode_attn(device_array(q_lat_bits, True), d["q_pe"], d["pool"], d["block_table"],
                                    d["seq_lens"], o, lse, ws, 0, p)
        torch.cuda.synchronize()
        return ws, o, lse, out

    ws, o, lse, out = run()
    want_plan, C = plan_reference(x, k, budget=budget)
    nranges = sum(c for _, c in want_plan)
    say("  k", k, "budget", budget, "chunk", C, "ranges", nranges)
    assert budget > len(lens) * k  # the larger budget is in force on this device
    assert nranges > len(lens) * k  # and the plan uses it: a second wave of ranges
    assert _table(ws, x, k, 2, slots=budget) == want_plan
    q, want = _oracle(x, q_lat_bits, True)
    o_h, lse_h = to_host(o), to_host(lse)
    assert not np.isnan(o_h).any() and not np.isnan(lse_h).any()
    err = rel_err(o_h, want["o_lat"])
    check_lse(lse_h, want["lse"], tol_for(x))
    check_softmax_mass(q, x.f32("q_pe"), x.f32("pool"), x.block_table, x.seq_lens, lse_h,
                       sample_rows(want["lse"], seed=45), softmax_scale=w.softmax_scale, tol=tol_for(x))
    errs = {"o_lat": err}
    if fused:
        out_h = to_host(out)
        assert not np.isnan(out_h).any()
        errs["out"] = rel_err(out_h, ref.out_proj_reference(want["o_lat"], x.f32("w_uv")))
    say("  rel errs", errs)
    for name, e in errs.items():
        assert e <= tol_for(x), name
    _, o2, lse2, out2 = run()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    if fused:
        assert torch.equal(out, out2)


hypothesis = pytest.importorskip("hypothesis")
from hypothesis import HealthCheck, given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402


@st.composite
def _ragged_batches(draw):
    # query-row counts where rows * k stays below 9/8 of 256 compute units (k = ceil(256 / rows)), so
    # the larger budget applies: 64 or 70 sequences of 2 query tokens, 86..90 or 128..140 of one
    batch, q_len = draw(st.sampled_from([(64, 2), (70, 2), (86, 1), (90, 1), (128, 1), (140, 1)]))
    kinds = draw(st.lists(st.sampled_from(["empty", "short", "mid", "long", "long"]), min_size=batch,
                          max_size=batch))
    span = {"empty": (0, 0), "short": (1, 200), "mid": (200, 1200), "long": (1200, 2600)}
    lens = [draw(st.integers(*span[k])) for k in kinds]
    return dict(batch=batch, q_len=q_len, lens=lens, seed=draw(st.integers(0, 2**31 - 1)))


@settings(max_examples=8, deadline=None, derandomize=True, suppress_health_check=list(HealthCheck))
@given(case=_ragged_batches())
def test_plan_longest_first_drawn(case):
    """Drawn ragged batches of 64..140 sequences (S = 1 or 2, causal; empty, short and long rows)
    with the library's split count: the slot table matches the plan restated with the library's
    range budget, every range is computed (NaN-filled workspace and outputs), and o_lat and lse match
    the oracle on every row."""
    import torch
    say("plan: drawn ragged batch", {k: v for k, v in case.items() if k != "lens"}, "rows",
        case["batch"] * case["q_len"])
    w = gen.small_workload(case["batch"], case["q_len"], cache_len=1, dtype="bf16", paged=True)
    lens = np.maximum(np.array(case["lens"], np.int32), 0)
    x = gen.generate(w, case["seed"] % 100000, poison_unused=True, seq_lens=lens)
    q_lat_bits, _ = gen.generate_latent(w, case["seed"] % 100000 + 1)
    d = to_device(x)
    p = params_for(x)
    k = binding.mla_decode_num_splits(p, 0)
    rows = case["batch"] * case["q_len"]
    budget = _longest_first_budget(rows, k)
    nb = binding.mla_decode_workspace_bytes(p, 0)
    ws = torch.full((max(nb, 16) // 4,), float("nan"), device="cuda")
    o = torch.full((w.batch, w.q_len, 128, 512), float("nan"), device="cuda")
    lse = torch.full((w.batch, w.q_len, 128), float("nan"), device="cuda")
    binding.mla_decode_attn(device_array(q_lat_bits, True), d["q_pe"], d["pool"], d["block_table"], d["seq_lens"],
                            o, lse, ws if nb else None, 0, p)
    torch.cuda.synchronize()
    if k > 1:
        want_plan, C = plan_reference(x, k, budget=budget)
        say("  k", k, "budget", budget, "chunk", C, "ranges", sum(c for _, c in want_plan))
        assert _table(ws, x, k, 2, slots=budget) == want_plan
    q, want = _oracle(x, q_lat_bits, True)
    o_h, lse_h = to_host(o), to_host(lse)
    assert not np.isnan(o_h).any() and not np.isnan(lse_h).any()
    assert rel_err(o_h, want["o_lat"]) <= tol_for(x)
    check_lse(lse_h, want["lse"], tol_for(x))
