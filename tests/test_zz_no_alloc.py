"""mla_decode_attn_out_proj_static (static scratch, no allocation) against mla_decode_attn_out_proj
with a caller workspace, through the C ABI: same kernels and split plan, so every output must be
bitwise equal. Two calls in a row on the same GPU, the second on a smaller batch (the scratch then
holds the first call's partials), both on the merge-in-out-projection route and on the separate
kernels' route, and the first call again after them."""
import numpy as np
import pytest

from deepseek_mla_latent_amd import binding
from deepseek_mla_latent_amd import inputs as gen
from tests.helpers import params_for, to_device

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def _run(x, q_lat_bits, splits, static):
    import torch
    d = to_device(x)
    p = params_for(x)
    w = x.workload
    q_lat = torch.from_numpy(np.ascontiguousarray(q_lat_bits).view(np.int16)).view(torch.bfloat16).cuda()
    out = torch.full((w.batch, w.q_len, 128, 128), float("nan"), device="cuda").to(torch.bfloat16)
    o = torch.full((w.batch, w.q_len, 128, 512), float("nan"), device="cuda")
    lse = torch.full((w.batch, w.q_len, 128), float("nan"), device="cuda")
    args = (q_lat, d["q_pe"], d["pool"], d["block_table"], d["seq_lens"], None, d["w_uv"], out, o, lse)
    if static:
        binding.mla_decode_attn_out_proj_static(*args, splits, p)
    else:
        nbytes = binding.mla_decode_attn_out_proj_workspace_bytes(p, splits)
        ws = torch.empty(max(nbytes, 16) // 4 + 4, dtype=torch.float32, device="cuda")
        binding.mla_decode_attn_out_proj(*args, ws, splits, p)
    torch.cuda.synchronize()
    return out.cpu(), o.cpu(), lse.cpu()


def _same(a, b):
    import torch
    return all(torch.equal(u, v) for u, v in zip(a, b))


@pytest.mark.parametrize("route", ["merge in out-projection", "separate kernels", "longest first"])
def test_static_scratch_matches_workspace_call(route):
    import torch
    # 24 query rows and auto splits take the merge inside the W_UV kernel; 6 rows take the
    # separate kernels (o_lat in the scratch when not asked for; asked for here); 128 and 90 ragged
    # rows take more key ranges than compute units (the longest-first plan: more partial slots)
    big_b, small_b = {"merge in out-projection": (24, 17), "separate kernels": (6, 3),
                      "longest first": (128, 90)}[route]
    hi = 2000 if route == "longest first" else 900
    cases = []
    for B, seed in ((big_b, 31), (small_b, 32)):
        w = gen.small_workload(B, 1, ragged=(40, hi), dtype="bf16", paged=True)
        x = gen.generate(w, seed, poison_unused=True)
        q_lat, _ = gen.generate_latent(w, seed + 100)
        cases.append((x, q_lat))
    results = []
    for x, q_lat in cases:  # first the larger batch, then the smaller one
        say("static vs workspace", route, "batch", x.workload.batch)
        got = _run(x, q_lat, 0, static=True)
        want = _run(x, q_lat, 0, static=False)
        assert not torch.isnan(got[0].float()).any()
        assert _same(got, want), x.workload.batch
        results.append(got)
    x, q_lat = cases[0]
    say("static again on the first batch")
    assert _same(_run(x, q_lat, 0, static=True), results[0])


def test_static_scratch_rejects_oversized_requests_before_launch():
    import torch
    w = gen.small_workload(2, 1, cache_len=300, dtype="bf16", paged=True)
    x = gen.generate(w, 33)
    d = to_device(x)
    p = binding.make_params(batch=4096, q_len=2, max_seq_len=131072, softmax_scale=w.softmax_scale)
    out = torch.full((2, 1, 128, 128), 7.0, device="cuda").to(torch.bfloat16)
    with pytest.raises(binding.MlaError) as e:
        binding.mla_decode_attn_out_proj_static(d["q_pe"], d["q_pe"], d["pool"], d["block_table"], d["seq_lens"],
                                                None, d["w_uv"], out, None, None, 8, p)
    assert e.value.code == -9
    torch.cuda.synchronize()
    assert bool((out.float() == 7.0).all())
