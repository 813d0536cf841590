"""The C-ABI library on the host: it loads, exports every declared function, and rejects every
host-checkable bad argument with the documented status before touching the GPU."""
import ctypes

import pytest

from deepseek_mla_latent_amd import binding
from tests.helpers import declared_functions

lib = pytest.importorskip("deepseek_mla_latent_amd.binding").load_library()

FAKE = 0x10000  # 16-byte aligned non-null address that is never dereferenced (calls fail first)
MISALIGNED = 0x10008


def P(**kw):
    base = dict(batch=2, q_len=1, max_seq_len=300, softmax_scale=0.1, dtype=binding.MLA_BF16)
    base.update(kw)
    return binding.make_params(**base)


def test_every_declared_function_is_exported():
    names = declared_functions()
    assert set(names) == set(binding.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for code, name in binding.STATUS.items():
        assert lib.mla_status_str(code).decode().startswith(name)
    assert lib.mla_status_str(-99).decode() == "unknown mla_status"


def _absorb(params, a=FAKE, b=FAKE, c=FAKE):
    return lib.mla_absorb_q(a, b, c, ctypes.byref(params), None)


def _outp(params, a=FAKE, b=FAKE, c=FAKE):
    return lib.mla_out_proj(a, b, c, ctypes.byref(params), None)


def _attn(params, ptrs=None, ws=None, ws_bytes=0, splits=2):
    p = dict(q_lat=FAKE, q_pe=FAKE, pool=FAKE, bt=FAKE, lens=FAKE, o=FAKE, lse=FAKE)
    p.update(ptrs or {})
    return lib.mla_decode_attn(p["q_lat"], p["q_pe"], p["pool"], p["bt"], p["lens"], p["o"], p["lse"], ws, ws_bytes,
                               splits, ctypes.byref(params), None)


@pytest.mark.parametrize("fn", [_absorb, _outp])
def test_projection_errors(fn):
    assert fn(P(), a=None) == -1
    assert fn(P(), c=None) == -1
    assert fn(P(dtype=7)) == -3
    assert fn(P(num_heads=64)) == -6
    assert fn(P(kv_lora_rank=256)) == -6
    assert fn(P(head_dim=64)) == -6
    assert fn(P(page_size=32)) == -6
    assert fn(P(q_len=0)) == -2
    assert fn(P(batch=-1)) == -2
    assert fn(P(), b=MISALIGNED) == -4
    assert lib.mla_absorb_q(FAKE, FAKE, FAKE, None, None) == -1
    assert fn(P(batch=0)) == 0  # empty batch: nothing to do, nothing enqueued


def test_attention_errors():
    assert _attn(P(), {"q_lat": None}) == -1
    assert _attn(P(), {"lens": None}) == -1
    assert _attn(P(), {"pool": None}) == -1
    assert _attn(P(), {"o": None}) == -1
    assert _attn(P(), {"q_pe": MISALIGNED}) == -4
    assert _attn(P(dtype=2)) == -3
    assert _attn(P(rope_dim=32)) == -6
    assert _attn(P(max_pages_per_seq=2)) == -2  # 300 tokens need 5 pages per sequence
    assert _attn(P(), splits=-1) == -2
    assert _attn(P(softmax_scale=float("inf"))) == -2
    assert _attn(P(softmax_scale=0.0)) == -2  # the kernels scale a tile's maximum: the scale must be > 0
    assert _attn(P(softmax_scale=-0.1)) == -2
    # explicit split count: workspace size is host-computable, no device query
    need = lib.mla_decode_workspace_bytes(ctypes.byref(P()), 2)
    plan = 16 + 16  # the range plan: a 16-byte header, then (first slot, range count) of each of the 2 rows
    assert need == 2 * 1 * 2 * 128 * (512 * 2 + 4) + plan  # bf16 partials + fp32 lse + range plan
    assert lib.mla_decode_workspace_bytes(ctypes.byref(P(dtype=binding.MLA_F32)), 2) == \
        2 * 1 * 2 * 128 * (512 + 1) * 4 + plan
    assert _attn(P(), ws=None, ws_bytes=0, splits=2) == -1
    assert _attn(P(), ws=FAKE, ws_bytes=need - 4, splits=2) == -5
    assert _attn(P(), ws=MISALIGNED, ws_bytes=need, splits=2) == -4
    assert _attn(P(batch=0), splits=2) == 0


def _tree(params, ptrs=None, parents=FAKE, ws=FAKE, ws_bytes=1 << 30, splits=2):
    p = dict(q_lat=FAKE, q_pe=FAKE, pool=FAKE, bt=FAKE, lens=FAKE, o=FAKE, lse=FAKE)
    p.update(ptrs or {})
    return lib.mla_decode_attn_tree(p["q_lat"], p["q_pe"], p["pool"], p["bt"], p["lens"], parents, p["o"], p["lse"],
                                    ws, ws_bytes, splits, ctypes.byref(params), None)


def test_tree_attention_errors():
    assert _tree(P(q_len=4), parents=None) == -1
    assert _tree(P(q_len=65)) == -2  # one 64-bit visibility mask per query row
    assert _tree(P(q_len=4), {"q_lat": None}) == -1
    assert _tree(P(q_len=4), {"o": MISALIGNED}) == -4
    assert _tree(P(q_len=4, softmax_scale=-1.0)) == -2
    assert _tree(P(q_len=4, dtype=5)) == -3
    assert _tree(P(q_len=4), ws=FAKE, ws_bytes=16) == -5
    assert _tree(P(q_len=4, batch=0), parents=None) == 0  # empty batch: nothing to do


def _fused(params, ptrs=None, parents=None, ws=FAKE, ws_bytes=1 << 30, splits=2):
    p = dict(q_lat=FAKE, q_pe=FAKE, pool=FAKE, bt=FAKE, lens=FAKE, w_uv=FAKE, out=FAKE, o=None, lse=None)
    p.update(ptrs or {})
    return lib.mla_decode_attn_out_proj(p["q_lat"], p["q_pe"], p["pool"], p["bt"], p["lens"], parents, p["w_uv"],
                                        p["out"], p["o"], p["lse"], ws, ws_bytes, splits, ctypes.byref(params), None)


def test_fused_attention_out_proj_errors():
    row = 128 * (512 * 2 + 4)  # one split's bf16 partial rows and lse values of one query row
    olat = 128 * 512 * 4  # one query row of o_lat
    ws = lambda params, k: lib.mla_decode_attn_out_proj_workspace_bytes(ctypes.byref(params), k)  # noqa: E731
    plan = lambda rows: 16 + (rows * 8 + 15) // 16 * 16  # noqa: E731  the range plan: header + rows, padded
    assert ws(P(batch=16), 2) == 16 * 2 * row + plan(16)  # merge inside the W_UV kernel
    assert ws(P(batch=16), 1) == 16 * olat  # one split: the separate kernels, o_lat in the workspace
    assert ws(P(), 2) == 2 * 2 * row + plan(2) + 2 * olat  # two rows: separate merge, o_lat in the workspace
    assert ws(P(), 1) == 2 * olat
    assert _fused(P(batch=16), ws_bytes=16 * 2 * row + plan(16) - 4) == -5
    row32 = 128 * (512 * 4 + 4)  # fp32 partial rows and lse values
    assert ws(P(dtype=binding.MLA_F32), 2) == 2 * 2 * row32 + plan(2)  # fp32, <= 4 rows: merge in the GEMV
    assert ws(P(dtype=binding.MLA_F32, batch=6), 2) == 6 * 2 * row32 + plan(6) + 6 * olat  # separate kernels
    assert _fused(P(), {"w_uv": None}) == -1
    assert _fused(P(), {"out": None}) == -1
    assert _fused(P(), {"q_lat": None}) == -1
    assert _fused(P(), {"out": MISALIGNED}) == -4
    assert _fused(P(), {"o": MISALIGNED}) == -4  # the latent outputs are optional, aligned when given
    assert _fused(P(q_len=65), parents=FAKE) == -2
    assert _fused(P(softmax_scale=-1.0)) == -2
    assert _fused(P(), ws_bytes=2 * 2 * row + 2 * olat - 4) == -5
    assert _fused(P(), ws=None, ws_bytes=0, splits=1) == -1
    assert _fused(P(batch=0), {"w_uv": None}) == 0  # empty batch: nothing to do


def test_split_planning_is_page_aligned():
    # explicit requests are clamped to the page count and trimmed of empty trailing splits
    for L, req, want in [(300, 2, 2), (300, 5, 5), (300, 9, 5), (64, 4, 1), (4096, 8, 8), (4096, 7, 7),
                         (16386, 2, 2), (129, 3, 3)]:
        got = lib.mla_decode_num_splits(ctypes.byref(P(max_seq_len=L)), req)
        assert got == want, (L, req, got)
    assert lib.mla_decode_workspace_bytes(ctypes.byref(P(max_seq_len=64)), 4) == 0  # one split: no workspace
    assert lib.mla_decode_num_splits(ctypes.byref(P(head_dim=1)), 2) == -6


def _kv_up(params, ptrs=None, kv_bytes=None):
    p = dict(pool=FAKE, bt=FAKE, lens=FAKE, wk=FAKE, wv=FAKE, kv=FAKE)
    p.update(ptrs or {})
    if kv_bytes is None:
        kv_bytes = lib.mla_prefill_kv_bytes(ctypes.byref(params))
    return lib.mla_prefill_kv_up(p["pool"], p["bt"], p["lens"], p["wk"], p["wv"], p["kv"], kv_bytes,
                                 ctypes.byref(params), None)


def _pf_attn(params, ptrs=None, kv_bytes=None):
    p = dict(qn=FAKE, qp=FAKE, kv=FAKE, lens=FAKE, out=FAKE, lse=FAKE)
    p.update(ptrs or {})
    if kv_bytes is None:
        kv_bytes = lib.mla_prefill_kv_bytes(ctypes.byref(params))
    return lib.mla_prefill_attn(p["qn"], p["qp"], p["kv"], kv_bytes, p["lens"], p["out"], p["lse"],
                                ctypes.byref(params), None)


def test_prefill_kv_bytes():
    # [K_nope | V] (B, H, Lp, 256) + k_pe (B, Lp, 64), bf16; Lp = 5 pages * 64 for 300 tokens
    assert lib.mla_prefill_kv_bytes(ctypes.byref(P(q_len=300))) == 2 * 320 * (128 * 256 + 64) * 2
    assert lib.mla_prefill_kv_bytes(ctypes.byref(P(q_len=300, max_pages_per_seq=8))) == 2 * 512 * (128 * 256 + 64) * 2
    assert lib.mla_prefill_kv_bytes(ctypes.byref(P(dtype=binding.MLA_F32))) == 0
    assert lib.mla_prefill_kv_bytes(ctypes.byref(P(head_dim=64))) == 0


@pytest.mark.parametrize("fn", [_kv_up, _pf_attn])
def test_prefill_errors(fn):
    first = "pool" if fn is _kv_up else "qn"
    assert fn(P(q_len=300), {first: None}) == -1
    assert fn(P(q_len=300), {"lens": None}) == -1
    assert fn(P(q_len=300), {first: MISALIGNED}) == -4
    assert fn(P(q_len=300, dtype=binding.MLA_F32), kv_bytes=1 << 30) == -3  # bf16 only
    assert fn(P(q_len=300, num_heads=64), kv_bytes=1 << 30) == -6
    assert fn(P(q_len=300, max_pages_per_seq=2), kv_bytes=1 << 30) == -2
    need = lib.mla_prefill_kv_bytes(ctypes.byref(P(q_len=300)))
    assert fn(P(q_len=300), kv_bytes=need - 2) == -5
    assert fn(P(q_len=300, batch=0), kv_bytes=0) == 0
    assert lib.mla_prefill_kv_up(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None, None) == -1


def test_linear_errors():
    def lin(m=32, k=128, n=64, x=FAKE, w=FAKE, y=FAKE):
        return lib.mla_linear(x, w, y, m, k, n, None, 0, None)
    assert lin(k=100) == -2  # k not a multiple of 64
    assert lin(n=96) == -2   # n not a multiple of 64
    assert lin(m=-1) == -2
    assert lin(m=1 << 20, k=4096) == -2  # x larger than 4 GiB
    assert lin(x=None) == -1
    assert lin(y=MISALIGNED) == -4
    assert lin(m=0) == 0
    assert lib.mla_linear_workspace_bytes(32, 100, 64) == 0


def test_rope_append_errors():
    def ra(params, stride=576, base=10000.0, **ptrs):
        p = dict(q=FAKE, kv=FAKE, pool=FAKE, bt=FAKE, lens=FAKE)
        p.update(ptrs)
        return lib.mla_rope_append(p["q"], p["kv"], stride, p["pool"], p["bt"], p["lens"], base, ctypes.byref(params),
                                   None)
    assert ra(P(dtype=binding.MLA_F32)) == -3
    assert ra(P(), stride=512) == -2
    assert ra(P(), stride=580) == -2   # rows must stay 16-byte aligned
    assert ra(P(), base=0.0) == -2
    assert ra(P(), base=float("nan")) == -2
    assert ra(P(max_pages_per_seq=2)) == -2
    assert ra(P(), q=None) == -1
    assert ra(P(), pool=None) == -1
    assert ra(P(), kv=MISALIGNED) == -4
    assert ra(P(batch=0)) == 0
    assert ra(P(num_heads=64)) == -6


def test_fp8_errors():
    assert lib.mla_fp8_weight_bytes() == 128 * 512 * 128 + 128 * 4 * 4
    nb = lib.mla_fp8_weight_bytes()
    assert lib.mla_quantize_w_uk_fp8(FAKE, FAKE, nb, ctypes.byref(P(dtype=binding.MLA_F32)), None) == -3
    assert lib.mla_quantize_w_uk_fp8(FAKE, FAKE, nb - 1, ctypes.byref(P()), None) == -5
    assert lib.mla_quantize_w_uv_fp8(None, FAKE, nb, ctypes.byref(P()), None) == -1
    assert lib.mla_quantize_w_uv_fp8(FAKE, MISALIGNED, nb, ctypes.byref(P()), None) == -4
    for fn in (lib.mla_absorb_q_fp8, lib.mla_out_proj_fp8):
        assert fn(FAKE, FAKE, FAKE, ctypes.byref(P(dtype=binding.MLA_F32)), None) == -3
        assert fn(None, FAKE, FAKE, ctypes.byref(P()), None) == -1
        assert fn(FAKE, FAKE, MISALIGNED, ctypes.byref(P()), None) == -4
        assert fn(FAKE, FAKE, FAKE, ctypes.byref(P(head_dim=64)), None) == -6
        assert fn(FAKE, FAKE, FAKE, ctypes.byref(P(batch=0)), None) == 0
    # the fused FP8 call takes bf16 activations only (the plain fused call also takes fp32)
    assert lib.mla_decode_attn_out_proj_fp8(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, None, FAKE, 1 << 30,
                                            2, ctypes.byref(P(dtype=binding.MLA_F32)), None) == -3


def _run_py(code):
    import subprocess
    import sys
    from tests.helpers import ROOT
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)


def test_library_binds_to_the_runtime_torch_uses():
    """Loaded through the binding, the library shares torch's HIP runtime (one runtime mapped)."""
    r = _run_py("from deepseek_mla_latent_amd import binding\n"
                "binding.load_library()\n"
                "print(len(binding._hip_runtimes_mapped()))")
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "1"


def test_a_second_runtime_is_refused():
    """The library opened raw before torch drags in a second HIP runtime; the binding refuses it."""
    r = _run_py("import ctypes\n"
                "from deepseek_mla_latent_amd import binding\n"
                "ctypes.CDLL(binding.LIB_PATH)\n"
                "import torch\n"
                "assert len(binding._hip_runtimes_mapped()) == 2\n"
                "try:\n"
                "    binding.load_library()\n"
                "except binding.MlaRuntimeConflict:\n"
                "    print('refused')\n")
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "refused"


def test_static_scratch_limit_is_checked_on_the_host():
    """mla_decode_attn_out_proj_static refuses a request larger than its static scratch before it
    touches any device (explicit split count: no device query either)."""
    p = P(batch=4096, q_len=2, max_seq_len=131072)
    need = binding.mla_decode_attn_out_proj_workspace_bytes(p, 8)
    assert need > (64 << 20)
    r = lib.mla_decode_attn_out_proj_static(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, None, 8,
                                            ctypes.byref(p), None)
    assert r == -9
    assert lib.mla_status_str(-9).decode().startswith("MLA_ERR_SCRATCH")
    assert lib.mla_decode_attn_out_proj_static(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, None, 8,
                                               None, None) == -1


def test_release_library_has_no_bounds_checks():
    assert lib.mla_debug_bounds_enabled() == 0
    words = (ctypes.c_uint32 * 2)()
    assert lib.mla_debug_bounds_read(words, 1) == -6


def test_num_pages_must_not_be_negative():
    assert _attn(P(num_pages=-1)) == -2
    assert _tree(P(q_len=4, num_pages=-1)) == -2
    assert _fused(P(num_pages=-1)) == -2
    assert lib.mla_prefill_kv_bytes(ctypes.byref(P(num_pages=-1))) == 0
    assert lib.mla_rope_append(FAKE, FAKE, 576, FAKE, FAKE, FAKE, 10000.0, ctypes.byref(P(num_pages=-1)), None) == -2
    assert _attn(P(num_pages=7), ws=FAKE, ws_bytes=1 << 30) != -2  # any count >= 0 passes the host checks


def test_size_queries_do_not_wrap():
    """Shapes whose buffers would not fit a 64-bit size (or whose grid would not fit a launch) give
    size 0 and are rejected by the call, instead of a wrapped-around small size."""
    huge = P(batch=1 << 24, max_seq_len=2 ** 31 - 1, max_pages_per_seq=2 ** 31 - 1)
    assert lib.mla_decode_workspace_bytes(ctypes.byref(huge), 2 ** 31 - 1) == 0
    assert lib.mla_decode_attn_out_proj_workspace_bytes(ctypes.byref(huge), 2 ** 31 - 1) == 0
    assert _attn(huge, ws=FAKE, ws_bytes=2 ** 63, splits=2 ** 31 - 1) == -2
    wide = P(batch=1 << 20, max_seq_len=64, max_pages_per_seq=1 << 20)
    assert lib.mla_prefill_kv_bytes(ctypes.byref(wide)) == 0
    assert lib.mla_prefill_kv_up(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2 ** 63, ctypes.byref(wide), None) == -2


@pytest.fixture(scope="module")
def debug_lib():
    import os
    if not os.path.exists(binding.DEBUG_LIB_PATH):
        pytest.skip("bounds-checked library not built")
    return binding.load_library(binding.DEBUG_LIB_PATH)


def test_bounds_checked_library_exports_the_same_functions(debug_lib):
    for n in declared_functions():
        assert hasattr(debug_lib, n), n
    assert debug_lib.mla_debug_bounds_enabled() == 1
    assert debug_lib.mla_debug_bounds_read(None, 1) == -1


def test_bounds_checked_library_rejects_the_same_arguments(debug_lib):
    def attn(params, ptrs=None, ws=None, ws_bytes=0, splits=2):
        p = dict(q_lat=FAKE, q_pe=FAKE, pool=FAKE, bt=FAKE, lens=FAKE, o=FAKE, lse=FAKE)
        p.update(ptrs or {})
        return debug_lib.mla_decode_attn(p["q_lat"], p["q_pe"], p["pool"], p["bt"], p["lens"], p["o"], p["lse"], ws,
                                         ws_bytes, splits, ctypes.byref(params), None)
    for kw, ptrs, want in ((dict(), {"q_lat": None}, -1), (dict(), {"q_pe": MISALIGNED}, -4), (dict(dtype=2), None, -3),
                           (dict(rope_dim=32), None, -6), (dict(max_pages_per_seq=2), None, -2),
                           (dict(num_pages=-3), None, -2), (dict(softmax_scale=0.0), None, -2)):
        assert attn(P(**kw), ptrs) == want, (kw, ptrs)
    assert debug_lib.mla_decode_workspace_bytes(ctypes.byref(P()), 2) == lib.mla_decode_workspace_bytes(
        ctypes.byref(P()), 2)
