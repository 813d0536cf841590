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
    # explicit split count: workspace size is host-computable, no device query
    need = lib.mla_decode_workspace_bytes(ctypes.byref(P()), 2)
    assert need == 2 * 1 * 2 * 128 * (512 * 2 + 4)  # bf16 partials + fp32 lse
    assert lib.mla_decode_workspace_bytes(ctypes.byref(P(dtype=binding.MLA_F32)), 2) == 2 * 1 * 2 * 128 * (512 + 1) * 4
    assert _attn(P(), ws=None, ws_bytes=0, splits=2) == -1
    assert _attn(P(), ws=FAKE, ws_bytes=need - 4, splits=2) == -5
    assert _attn(P(), ws=MISALIGNED, ws_bytes=need, splits=2) == -4
    assert _attn(P(batch=0), splits=2) == 0


def test_split_planning_is_page_aligned():
    # explicit requests are clamped to the page count and trimmed of empty trailing splits
    for L, req, want in [(300, 2, 2), (300, 5, 5), (300, 9, 5), (64, 4, 1), (4096, 8, 8), (4096, 7, 7),
                         (16386, 2, 2), (129, 3, 3)]:
        got = lib.mla_decode_num_splits(ctypes.byref(P(max_seq_len=L)), req)
        assert got == want, (L, req, got)
    assert lib.mla_decode_workspace_bytes(ctypes.byref(P(max_seq_len=64)), 4) == 0  # one split: no workspace
    assert lib.mla_decode_num_splits(ctypes.byref(P(head_dim=1)), 2) == -6
