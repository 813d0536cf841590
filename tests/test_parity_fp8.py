"""GPU parity of the FP8 block-quantised per-head products against the fp64 FP8 oracle.

The weight codes and scales the GPU writes are compared bit for bit with the oracle's (the
quantisation decision is taken in fp32 on both sides). The products use the same codes, so they
differ from the oracle only by fp32 summation order and the final bf16 rounding. Bar:
max |gpu - ref| / max |ref| <= 4e-3. The FP8 products' distance from the unquantised bf16 ones
is reported and bounded at 5%.
"""
import numpy as np
import pytest

from deepseek_mla_latent_amd import binding
from deepseek_mla_latent_amd import inputs as gen
from oracle import fp8 as ref
from oracle import mla_decode as dec
from tests.helpers import params_for, rel_err, to_device, to_host

pytestmark = pytest.mark.gpu
FP8_TOL = 4e-3


def say(*a):
    print("[case]", *a, flush=True)


def _packed(w_bits, transpose):
    import torch
    p = binding.make_params(batch=1, q_len=1, max_seq_len=1)
    w = torch.from_numpy(np.ascontiguousarray(w_bits).view(np.int16)).view(torch.bfloat16).cuda()
    packed = torch.zeros(binding.mla_fp8_weight_bytes(), dtype=torch.uint8, device="cuda")
    (binding.mla_quantize_w_uv_fp8 if transpose else binding.mla_quantize_w_uk_fp8)(w, packed, p)
    torch.cuda.synchronize()
    return packed


def _unpack(packed):
    a = packed.cpu().numpy()
    n = 128 * 512 * 128
    return a[:n].reshape(128, -1), a[n:n + 128 * 4 * 4].view(np.float32).reshape(128, 4)


@pytest.mark.parametrize("which", ["w_uk", "w_uv"])
def test_weight_quantisation_is_bit_exact(which):
    say("fp8 weight quantisation", which)
    w = gen.small_workload(1, 1, cache_len=1, dtype="bf16", paged=False)
    x = gen.generate(w, 501)
    bits = getattr(x, which)
    packed = _packed(bits, which == "w_uv")
    codes, scales = _unpack(packed)
    vals, sc = ref.quantize(gen.bf16_bits_to_f32(bits), (1, 128, 128))  # sc: (H, 4, 1)
    want_codes = ref.e4m3_encode(vals)  # (H, 512, 128)
    if which == "w_uv":
        want_codes = np.ascontiguousarray(np.swapaxes(want_codes, 1, 2))  # (H, 128, 512)
    np.testing.assert_array_equal(scales, sc[:, :, 0])
    np.testing.assert_array_equal(codes.reshape(want_codes.shape), want_codes)


@pytest.mark.parametrize("which", ["w_uk", "w_uv"])
def test_weight_codes_at_ties_subnormals_and_zero_blocks(which):
    """Blocks whose maximum is 448 (factor exactly 1) holding exact E4M3 ties (normal and
    subnormal, both signs), a block of -0.0 and a block of +0.0 (codes 0), next to random blocks:
    the codes must match the oracle's round-to-nearest-even bit for bit."""
    say("fp8 weight edge codes", which)
    rng = np.random.default_rng(502)
    w = rng.standard_normal((128, 512, 128)).astype(np.float32) / np.float32(np.sqrt(512))
    ties = np.array([1.0625, 1.1875, 3.25, 3.75, 0.5 * 2.0 ** -9, 1.5 * 2.0 ** -9, 2.5 * 2.0 ** -9,
                     7.5 * 2.0 ** -9, 2.0 ** -6 + 2.0 ** -10, 240.0, 432.0, 2.0 ** -11], dtype=np.float32)
    for h, cb in ((0, 0), (5, 3), (127, 1)):
        blk = np.zeros((128, 128), np.float32)
        vals = np.concatenate([ties, -ties])
        blk.flat[:vals.size] = vals
        blk[-1, -1] = 448.0
        w[h, 128 * cb:128 * cb + 128] = blk
    w[1, 0:128] = -0.0
    w[2, 128:256] = 0.0
    bits = gen.round_to_bf16_bits(w)
    assert np.array_equal(gen.bf16_bits_to_f32(bits)[0, :128], w[0, :128])  # every tie is a bf16 value
    packed = _packed(bits, which == "w_uv")
    codes, scales = _unpack(packed)
    vals, sc = ref.quantize(gen.bf16_bits_to_f32(bits), (1, 128, 128))
    want_codes = ref.e4m3_encode(vals)
    if which == "w_uv":
        want_codes = np.ascontiguousarray(np.swapaxes(want_codes, 1, 2))
    np.testing.assert_array_equal(scales, sc[:, :, 0])
    np.testing.assert_array_equal(codes.reshape(want_codes.shape), want_codes)
    assert scales[0, 0] == np.float32(1.0) and scales[1, 0] == 0 and scales[2, 1] == 0


@pytest.mark.parametrize("tokens", [1, 33, 128])
def test_absorb_q_fp8(tokens):
    say("absorb_q fp8", tokens)
    import torch
    w = gen.small_workload(tokens, 1, cache_len=1, dtype="bf16", paged=False)
    x = gen.generate(w, 600 + tokens)
    d = to_device(x)
    p = params_for(x)
    packed = _packed(x.w_uk, False)
    q_lat = torch.full((tokens, 1, 128, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    binding.mla_absorb_q_fp8(d["q_nope"], packed, q_lat, p)
    torch.cuda.synchronize()
    got = to_host(q_lat)
    want, _, _ = ref.absorb_q_fp8_reference(x.f32("q_nope"), x.f32("w_uk"))
    err = rel_err(got, want)
    exact = dec.absorb_q_reference(x.f32("q_nope"), x.f32("w_uk"))
    say("  rel err vs fp8 oracle", err, " vs unquantised", rel_err(got, exact))
    assert err <= FP8_TOL
    assert rel_err(got, exact) <= 0.05


@pytest.mark.parametrize("tokens", [1, 33, 128])
def test_out_proj_fp8(tokens):
    say("out_proj fp8", tokens)
    import torch
    w = gen.small_workload(tokens, 1, cache_len=1, dtype="bf16", paged=False)
    x = gen.generate(w, 700 + tokens)
    _, o_lat = gen.generate_latent(w, 800 + tokens)
    o_lat[0, 0, 5, :] = 0.0  # an all-zero activation vector: codes 0, output 0
    p = params_for(x)
    packed = _packed(x.w_uv, True)
    out = torch.full((tokens, 1, 128, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    binding.mla_out_proj_fp8(torch.from_numpy(o_lat).cuda(), packed, out, p)
    torch.cuda.synchronize()
    got = to_host(out)
    want, _, _ = ref.out_proj_fp8_reference(o_lat, x.f32("w_uv"))
    err = rel_err(got, want)
    exact = dec.out_proj_reference(o_lat, x.f32("w_uv"))
    say("  rel err vs fp8 oracle", err, " vs unquantised", rel_err(got, exact))
    assert np.all(got[0, 0, 5] == 0)
    assert err <= FP8_TOL
    assert rel_err(got, exact) <= 0.05


def test_fp8_decode_path_end_to_end():
    """absorb (FP8) -> latent attention -> out-proj (FP8), against the oracle's FP8 absorb, the
    latent attention reference and its FP8 out-projection."""
    import torch
    say("fp8 decode path")
    w = gen.small_workload(3, 1, ragged=(100, 700), dtype="bf16", paged=True)
    x = gen.generate(w, 901, poison_unused=True)
    d = to_device(x)
    p = params_for(x)
    uk, uv = _packed(x.w_uk, False), _packed(x.w_uv, True)
    bufs = binding.DecodeBuffers(p, 0)
    binding.mla_absorb_q_fp8(d["q_nope"], uk, bufs.q_lat, p)
    binding.mla_decode_attn(bufs.q_lat, d["q_pe"], d["pool"], d["block_table"], d["seq_lens"], bufs.o_lat, bufs.lse,
                            bufs.workspace, 0, p)
    binding.mla_out_proj_fp8(bufs.o_lat, uv, bufs.out, p)
    torch.cuda.synchronize()
    q_lat, _, _ = ref.absorb_q_fp8_reference(x.f32("q_nope"), x.f32("w_uk"))
    q_lat = gen.bf16_bits_to_f32(gen.round_to_bf16_bits(q_lat.astype(np.float32)))  # the call's bf16 output
    att = dec.latent_attention_reference(q_lat, x.f32("q_pe"), x.f32("pool"), x.block_table, x.seq_lens,
                                         softmax_scale=w.softmax_scale)
    want, _, _ = ref.out_proj_fp8_reference(att["o_lat"].astype(np.float32), x.f32("w_uv"))
    err = rel_err(to_host(bufs.out), want)
    say("  out rel err", err)
    assert err <= 2e-2


@pytest.mark.parametrize("batch,q_len,splits,lens", [
    (16, 1, 2, None),             # merge, coding and FP8 product in one kernel
    (32, 1, 0, None),             # the library's split count
    (8, 2, 3, None),              # two query tokens (16 rows), causal
    (17, 1, 2, [0] + [300] * 16),  # a row with no keys: o_lat = 0, codes 0, out = 0; a ragged last block
    (3, 1, 2, None),              # fewer than 16 rows: attention + merge, then the FP8 out-projection
    (16, 1, 1, None),             # one split: attention writes o_lat, then the FP8 out-projection
])
def test_fused_attention_out_proj_fp8(batch, q_len, splits, lens):
    """mla_decode_attn_out_proj_fp8 against the oracle's latent attention followed by its FP8
    out-projection.  The call codes its own merged rows (bf16 partials merged in fp32), which
    differ from the exact o_lat by about one bf16 rounding, and E4M3 coding amplifies that: a value
    within that distance of a rounding point takes the neighbouring code.  The oracle measures this
    itself: s = the distance between its FP8 product of the bf16-rounded o_lat and its FP8 product
    of the exact one (1.1e-2 to 2.1e-2 on these cases).  Bars: out within 2e-2 + s of the FP8
    oracle, and within q + 2e-2 of the unquantised product, q being the oracle's own FP8 error
    (2.7e-2 to 4.5e-2 here); o_lat and lse (optional outputs) at the bf16 bar as in the bf16 call."""
    import torch
    from tests.helpers import check_lse
    say("fused attention + out-proj fp8", batch, q_len, splits, "lens" if lens else "ragged")
    w = gen.small_workload(batch, q_len, ragged=None if lens else (100, 700), cache_len=1 if lens else None,
                           dtype="bf16", paged=True)
    x = gen.generate(w, 950 + batch + splits, poison_unused=True, seq_lens=lens)
    d = to_device(x)
    p = params_for(x)
    q_bits, _ = gen.generate_latent(w, 951 + batch)
    q_lat = torch.from_numpy(np.ascontiguousarray(q_bits).view(np.int16)).view(torch.bfloat16).cuda()
    uv = _packed(x.w_uv, True)
    out = torch.full((batch, q_len, 128, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    o = torch.full((batch, q_len, 128, 512), float("nan"), device="cuda")
    lse = torch.full((batch, q_len, 128), float("nan"), device="cuda")
    nb = binding.mla_decode_attn_out_proj_workspace_bytes(p, splits)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
    binding.mla_decode_attn_out_proj_fp8(q_lat, d["q_pe"], d["pool"], d["block_table"], d["seq_lens"], None, uv, out,
                                         o, lse, ws, splits, p, workspace_bytes=nb)
    torch.cuda.synchronize()
    att = dec.latent_attention_reference(gen.bf16_bits_to_f32(q_bits), x.f32("q_pe"), x.f32("pool"), x.block_table,
                                         x.seq_lens, softmax_scale=w.softmax_scale)
    o_ref = att["o_lat"].astype(np.float32)
    want, _, _ = ref.out_proj_fp8_reference(o_ref, x.f32("w_uv"))
    exact = dec.out_proj_reference(att["o_lat"], x.f32("w_uv"))
    moved, _, _ = ref.out_proj_fp8_reference(gen.bf16_bits_to_f32(gen.round_to_bf16_bits(o_ref)), x.f32("w_uv"))
    sens, q_err = rel_err(moved, want), rel_err(want, exact)
    got = to_host(out)
    err, err_exact = rel_err(got, want), rel_err(got, exact)
    o_err, l_err = rel_err(to_host(o), att["o_lat"]), check_lse(to_host(lse), att["lse"], 2e-2)
    say(f"  out rel err vs fp8 oracle {err:.2e} (bar 2e-2 + {sens:.2e}), vs unquantised {err_exact:.2e} "
        f"(bar {q_err:.2e} + 2e-2); o_lat {o_err:.2e}; lse {l_err:.2e}")
    assert not np.isnan(got).any()
    assert err <= 2e-2 + sens and err_exact <= q_err + 2e-2 and o_err <= 2e-2
    if lens:
        assert np.all(got[0] == 0)
