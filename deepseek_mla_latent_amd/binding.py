"""ctypes binding of ``libmla_latent.so`` (declared in ``include/mla_latent.h``).

Argument marshalling only: every step of the decode path runs in the library's HIP
kernels.  Functions keep the C names; tensor arguments are torch tensors on the GPU
(torch provides device memory and the current stream), or raw integer device pointers.
There is no fallback: if the library is missing the import of this module still works,
but every call raises ``MlaLibraryMissing``.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmla_latent.so")
DEBUG_LIB_PATH = os.path.join(PKG, "libmla_latent_debug.so")  # bounds-checked build of the same sources

MLA_F32 = 0
MLA_BF16 = 1

STATUS = {
    0: "MLA_OK", -1: "MLA_ERR_NULL", -2: "MLA_ERR_SHAPE", -3: "MLA_ERR_DTYPE", -4: "MLA_ERR_ALIGN",
    -5: "MLA_ERR_WORKSPACE", -6: "MLA_ERR_UNSUPPORTED", -7: "MLA_ERR_LAUNCH", -8: "MLA_ERR_DEVICE",
    -9: "MLA_ERR_SCRATCH",
}
EXPORTS = ("mla_absorb_q", "mla_decode_workspace_bytes", "mla_decode_num_splits", "mla_decode_attn",
           "mla_decode_attn_tree", "mla_decode_attn_out_proj_workspace_bytes", "mla_decode_attn_out_proj",
           "mla_out_proj", "mla_prefill_kv_bytes", "mla_prefill_kv_up", "mla_prefill_attn",
           "mla_linear_workspace_bytes", "mla_linear", "mla_rope_append", "mla_fp8_weight_bytes",
           "mla_quantize_w_uk_fp8", "mla_quantize_w_uv_fp8", "mla_absorb_q_fp8", "mla_out_proj_fp8", "mla_status_str",
           "mla_debug_attn_schedule", "mla_decode_attn_out_proj_static", "mla_debug_bounds_enabled",
           "mla_debug_bounds_read", "mla_decode_attn_out_proj_fp8")
BOUNDS_BAD_SEQ_LEN = 1  # error-word bits of the bounds-checked build
BOUNDS_BAD_PAGE = 2


class MlaLibraryMissing(RuntimeError):
    pass


class MlaError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {mla_status_str(code)} ({code})")


class mla_params(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("q_len", ctypes.c_int32), ("num_heads", ctypes.c_int32),
        ("kv_lora_rank", ctypes.c_int32), ("rope_dim", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float), ("causal", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
    ]


_lib = None


class MlaRuntimeConflict(RuntimeError):
    """More than one HIP runtime is mapped into the process."""


def _hip_runtimes_mapped():
    """Paths of the HIP runtime libraries mapped into this process (Linux)."""
    try:
        with open("/proc/self/maps") as f:
            return sorted({line.split()[-1] for line in f if "libamdhip64" in line})
    except OSError:
        return []


def declare(lib, *, partial: bool = False):
    """Set the ctypes signatures of every exported function on ``lib`` (a ctypes.CDLL).  With
    ``partial``, functions the library does not export are skipped (a host-only build of the
    C-ABI layer links a subset of the sources)."""

    class _Lib:
        def __getattr__(self, name):
            if partial and not hasattr(lib, name):
                return _Sink()
            return getattr(lib, name)

    class _Sink:
        pass

    L = _Lib()
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    pp = ctypes.POINTER(mla_params)
    L.mla_absorb_q.argtypes = [vp, vp, vp, pp, vp]
    L.mla_absorb_q.restype = i32
    L.mla_decode_workspace_bytes.argtypes = [pp, i32]
    L.mla_decode_workspace_bytes.restype = sz
    L.mla_decode_num_splits.argtypes = [pp, i32]
    L.mla_decode_num_splits.restype = i32
    L.mla_decode_attn.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, sz, i32, pp, vp]
    L.mla_decode_attn.restype = i32
    L.mla_decode_attn_tree.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i32, pp, vp]
    L.mla_decode_attn_tree.restype = i32
    L.mla_decode_attn_out_proj_workspace_bytes.argtypes = [pp, i32]
    L.mla_decode_attn_out_proj_workspace_bytes.restype = sz
    L.mla_decode_attn_out_proj.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i32, pp, vp]
    L.mla_decode_attn_out_proj.restype = i32
    L.mla_decode_attn_out_proj_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i32, pp, vp]
    L.mla_decode_attn_out_proj_fp8.restype = i32
    L.mla_decode_attn_out_proj_static.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, pp, vp]
    L.mla_decode_attn_out_proj_static.restype = i32
    L.mla_out_proj.argtypes = [vp, vp, vp, pp, vp]
    L.mla_out_proj.restype = i32
    L.mla_prefill_kv_bytes.argtypes = [pp]
    L.mla_prefill_kv_bytes.restype = sz
    L.mla_prefill_kv_up.argtypes = [vp, vp, vp, vp, vp, vp, sz, pp, vp]
    L.mla_prefill_kv_up.restype = i32
    L.mla_prefill_attn.argtypes = [vp, vp, vp, sz, vp, vp, vp, pp, vp]
    L.mla_prefill_attn.restype = i32
    L.mla_linear_workspace_bytes.argtypes = [i32, i32, i32]
    L.mla_linear_workspace_bytes.restype = sz
    L.mla_linear.argtypes = [vp, vp, vp, i32, i32, i32, vp, sz, vp]
    L.mla_linear.restype = i32
    L.mla_rope_append.argtypes = [vp, vp, i32, vp, vp, vp, ctypes.c_float, pp, vp]
    L.mla_rope_append.restype = i32
    L.mla_fp8_weight_bytes.argtypes = []
    L.mla_fp8_weight_bytes.restype = sz
    for name in ("mla_quantize_w_uk_fp8", "mla_quantize_w_uv_fp8"):
        getattr(L, name).argtypes = [vp, vp, sz, pp, vp]
        getattr(L, name).restype = i32
    for name in ("mla_absorb_q_fp8", "mla_out_proj_fp8"):
        getattr(L, name).argtypes = [vp, vp, vp, pp, vp]
        getattr(L, name).restype = i32
    L.mla_status_str.argtypes = [i32]
    L.mla_status_str.restype = ctypes.c_char_p
    L.mla_debug_attn_schedule.argtypes = [i32, ctypes.POINTER(i32), ctypes.POINTER(i32), ctypes.POINTER(i32)]
    L.mla_debug_attn_schedule.restype = i32
    L.mla_debug_bounds_enabled.argtypes = []
    L.mla_debug_bounds_enabled.restype = i32
    L.mla_debug_bounds_read.argtypes = [ctypes.POINTER(ctypes.c_uint32), i32]
    L.mla_debug_bounds_read.restype = i32
    return lib


def load_library(path: Optional[str] = None):
    """Load the shared library once; raise MlaLibraryMissing if it is not built.

    The library must run on the same HIP runtime as the framework that owns the device memory it
    is handed.  torch ships its own copy of the runtime under the same soname, so torch is
    imported first: the library's dependency then resolves to the copy already loaded.  Loaded the
    other way round, the process would hold two runtimes (the library's launches going through one
    while torch's memory and streams belong to the other); that state is refused.
    """
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise MlaLibraryMissing(f"{p} is not built; run `python -m deepseek_mla_latent_amd.build`")
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(p)
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise MlaRuntimeConflict(f"{p} was loaded next to another HIP runtime: {runtimes}; load it in a process "
                                 "whose HIP runtime is already the one torch uses (import torch first)")
    declare(lib)
    if path is None:
        _lib = lib
    return lib


def make_params(*, batch: int, q_len: int, max_seq_len: int, max_pages_per_seq: Optional[int] = None,
                softmax_scale: Optional[float] = None, causal: bool = True, dtype: int = MLA_BF16,
                num_heads: int = 128, kv_lora_rank: int = 512, rope_dim: int = 64, head_dim: int = 128,
                page_size: int = 64, num_pages: int = 0) -> mla_params:
    if max_pages_per_seq is None:
        max_pages_per_seq = max(1, -(-max_seq_len // page_size))
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(head_dim + rope_dim)
    return mla_params(batch, q_len, num_heads, kv_lora_rank, rope_dim, head_dim, page_size, max_pages_per_seq,
                      max_seq_len, softmax_scale, 1 if causal else 0, dtype, num_pages)


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_cuda:
        raise ValueError("tensor arguments must be on the GPU")
    if not x.is_contiguous():
        raise ValueError("tensor arguments must be contiguous")
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(code: int, where: str):
    if code != 0:
        raise MlaError(code, where)


def mla_debug_attn_schedule(ntiles: int):
    """(a_buffer, b_buffer, p_buffer) lists of the attention kernel's LDS rings over ntiles tiles."""
    arrs = [(ctypes.c_int32 * ntiles)() for _ in range(3)]
    _check(load_library().mla_debug_attn_schedule(ntiles, *arrs), "mla_debug_attn_schedule")
    return tuple(list(a) for a in arrs)


def mla_debug_bounds_read(lib=None, clear: bool = True):
    """(violation bits, report count) of the bounds-checked library's error word (waits for the
    device); clears it unless ``clear`` is False."""
    words = (ctypes.c_uint32 * 2)()
    _check((lib or load_library()).mla_debug_bounds_read(words, 1 if clear else 0), "mla_debug_bounds_read")
    return int(words[0]), int(words[1])


def mla_status_str(code: int) -> str:
    try:
        return load_library().mla_status_str(code).decode()
    except MlaLibraryMissing:
        return STATUS.get(code, "unknown")


def mla_absorb_q(q_nope, w_uk, q_lat, params: mla_params, stream=None) -> None:
    lib = load_library()
    _check(lib.mla_absorb_q(_ptr(q_nope), _ptr(w_uk), _ptr(q_lat), ctypes.byref(params), _stream(stream)),
           "mla_absorb_q")


def mla_decode_workspace_bytes(params: mla_params, num_splits: int = 0) -> int:
    return int(load_library().mla_decode_workspace_bytes(ctypes.byref(params), num_splits))


def mla_decode_num_splits(params: mla_params, num_splits: int = 0) -> int:
    r = int(load_library().mla_decode_num_splits(ctypes.byref(params), num_splits))
    _check(min(r, 0), "mla_decode_num_splits")
    return r


def mla_decode_attn(q_lat, q_pe, kv_pool, block_table, seq_lens, o_lat, lse, workspace, num_splits: int,
                    params: mla_params, stream=None, workspace_bytes: Optional[int] = None) -> None:
    lib = load_library()
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None or isinstance(workspace, int) else \
            workspace.numel() * workspace.element_size()
    _check(lib.mla_decode_attn(_ptr(q_lat), _ptr(q_pe), _ptr(kv_pool), _ptr(block_table), _ptr(seq_lens),
                               _ptr(o_lat), _ptr(lse), _ptr(workspace), workspace_bytes, num_splits,
                               ctypes.byref(params), _stream(stream)), "mla_decode_attn")


def mla_decode_attn_tree(q_lat, q_pe, kv_pool, block_table, seq_lens, tree_parents, o_lat, lse, workspace,
                         num_splits: int, params: mla_params, stream=None,
                         workspace_bytes: Optional[int] = None) -> None:
    lib = load_library()
    _check(lib.mla_decode_attn_tree(_ptr(q_lat), _ptr(q_pe), _ptr(kv_pool), _ptr(block_table), _ptr(seq_lens),
                                    _ptr(tree_parents), _ptr(o_lat), _ptr(lse), _ptr(workspace),
                                    _nbytes(workspace, workspace_bytes), num_splits, ctypes.byref(params),
                                    _stream(stream)), "mla_decode_attn_tree")


def mla_decode_attn_out_proj_workspace_bytes(params: mla_params, num_splits: int = 0) -> int:
    return int(load_library().mla_decode_attn_out_proj_workspace_bytes(ctypes.byref(params), num_splits))


def mla_decode_attn_out_proj(q_lat, q_pe, kv_pool, block_table, seq_lens, tree_parents, w_uv, out, o_lat, lse,
                             workspace, num_splits: int, params: mla_params, stream=None,
                             workspace_bytes: Optional[int] = None) -> None:
    lib = load_library()
    _check(lib.mla_decode_attn_out_proj(_ptr(q_lat), _ptr(q_pe), _ptr(kv_pool), _ptr(block_table), _ptr(seq_lens),
                                        _ptr(tree_parents), _ptr(w_uv), _ptr(out), _ptr(o_lat), _ptr(lse),
                                        _ptr(workspace), _nbytes(workspace, workspace_bytes), num_splits,
                                        ctypes.byref(params), _stream(stream)), "mla_decode_attn_out_proj")


def mla_decode_attn_out_proj_fp8(q_lat, q_pe, kv_pool, block_table, seq_lens, tree_parents, w_uv_fp8, out, o_lat,
                                 lse, workspace, num_splits: int, params: mla_params, stream=None,
                                 workspace_bytes: Optional[int] = None) -> None:
    lib = load_library()
    _check(lib.mla_decode_attn_out_proj_fp8(_ptr(q_lat), _ptr(q_pe), _ptr(kv_pool), _ptr(block_table),
                                            _ptr(seq_lens), _ptr(tree_parents), _ptr(w_uv_fp8), _ptr(out), _ptr(o_lat),
                                            _ptr(lse), _ptr(workspace), _nbytes(workspace, workspace_bytes),
                                            num_splits, ctypes.byref(params), _stream(stream)),
           "mla_decode_attn_out_proj_fp8")


def mla_decode_attn_out_proj_static(q_lat, q_pe, kv_pool, block_table, seq_lens, tree_parents, w_uv, out, o_lat,
                                    lse, num_splits: int, params: mla_params, stream=None) -> None:
    lib = load_library()
    _check(lib.mla_decode_attn_out_proj_static(_ptr(q_lat), _ptr(q_pe), _ptr(kv_pool), _ptr(block_table),
                                               _ptr(seq_lens), _ptr(tree_parents), _ptr(w_uv), _ptr(out),
                                               _ptr(o_lat), _ptr(lse), num_splits, ctypes.byref(params),
                                               _stream(stream)), "mla_decode_attn_out_proj_static")


def mla_out_proj(o_lat, w_uv, out, params: mla_params, stream=None) -> None:
    lib = load_library()
    _check(lib.mla_out_proj(_ptr(o_lat), _ptr(w_uv), _ptr(out), ctypes.byref(params), _stream(stream)),
           "mla_out_proj")


def _nbytes(x, given: Optional[int]) -> int:
    if given is not None:
        return given
    return 0 if x is None or isinstance(x, int) else x.numel() * x.element_size()


def mla_prefill_kv_bytes(params: mla_params) -> int:
    return int(load_library().mla_prefill_kv_bytes(ctypes.byref(params)))


def mla_prefill_kv_up(kv_pool, block_table, seq_lens, w_uk, w_uv, kv, params: mla_params, stream=None,
                      kv_bytes: Optional[int] = None) -> None:
    lib = load_library()
    _check(lib.mla_prefill_kv_up(_ptr(kv_pool), _ptr(block_table), _ptr(seq_lens), _ptr(w_uk), _ptr(w_uv), _ptr(kv),
                                 _nbytes(kv, kv_bytes), ctypes.byref(params), _stream(stream)), "mla_prefill_kv_up")


def mla_prefill_attn(q_nope, q_pe, kv, seq_lens, out, lse, params: mla_params, stream=None,
                     kv_bytes: Optional[int] = None) -> None:
    lib = load_library()
    _check(lib.mla_prefill_attn(_ptr(q_nope), _ptr(q_pe), _ptr(kv), _nbytes(kv, kv_bytes), _ptr(seq_lens), _ptr(out),
                                _ptr(lse), ctypes.byref(params), _stream(stream)), "mla_prefill_attn")


def mla_linear_workspace_bytes(m: int, k: int, n: int) -> int:
    return int(load_library().mla_linear_workspace_bytes(m, k, n))


def mla_linear(x, w, y, m: int, k: int, n: int, workspace=None, stream=None,
               workspace_bytes: Optional[int] = None) -> None:
    lib = load_library()
    _check(lib.mla_linear(_ptr(x), _ptr(w), _ptr(y), m, k, n, _ptr(workspace), _nbytes(workspace, workspace_bytes),
                          _stream(stream)), "mla_linear")


def mla_rope_append(q_pe, kv_a, kv_a_stride: int, kv_pool, block_table, seq_lens, params: mla_params,
                    rope_base: float = 10000.0, stream=None) -> None:
    lib = load_library()
    _check(lib.mla_rope_append(_ptr(q_pe), _ptr(kv_a), kv_a_stride, _ptr(kv_pool), _ptr(block_table), _ptr(seq_lens),
                               rope_base, ctypes.byref(params), _stream(stream)), "mla_rope_append")


def mla_fp8_weight_bytes() -> int:
    return int(load_library().mla_fp8_weight_bytes())


def mla_quantize_w_uk_fp8(w_uk, packed, params: mla_params, stream=None, packed_bytes: Optional[int] = None) -> None:
    _check(load_library().mla_quantize_w_uk_fp8(_ptr(w_uk), _ptr(packed), _nbytes(packed, packed_bytes),
                                                ctypes.byref(params), _stream(stream)), "mla_quantize_w_uk_fp8")


def mla_quantize_w_uv_fp8(w_uv, packed, params: mla_params, stream=None, packed_bytes: Optional[int] = None) -> None:
    _check(load_library().mla_quantize_w_uv_fp8(_ptr(w_uv), _ptr(packed), _nbytes(packed, packed_bytes),
                                                ctypes.byref(params), _stream(stream)), "mla_quantize_w_uv_fp8")


def mla_absorb_q_fp8(q_nope, w_uk_fp8, q_lat, params: mla_params, stream=None) -> None:
    _check(load_library().mla_absorb_q_fp8(_ptr(q_nope), _ptr(w_uk_fp8), _ptr(q_lat), ctypes.byref(params),
                                           _stream(stream)), "mla_absorb_q_fp8")


def mla_out_proj_fp8(o_lat, w_uv_fp8, out, params: mla_params, stream=None) -> None:
    _check(load_library().mla_out_proj_fp8(_ptr(o_lat), _ptr(w_uv_fp8), _ptr(out), ctypes.byref(params),
                                           _stream(stream)), "mla_out_proj_fp8")


class DecodeBuffers:
    """Device tensors for one decode step: intermediates, outputs and workspace (torch-allocated).

    Allocation happens here, once, outside the calls; ``run`` only enqueues the three library
    calls, so it can be captured in a HIP graph and replayed.
    """

    def __init__(self, params: mla_params, num_splits: int = 0, device="cuda"):
        import torch
        self.params = params
        self.num_splits = num_splits
        B, S, H = params.batch, params.q_len, params.num_heads
        dt = torch.bfloat16 if params.dtype == MLA_BF16 else torch.float32
        self.q_lat = torch.empty((B, S, H, params.kv_lora_rank), dtype=dt, device=device)
        self.o_lat = torch.empty((B, S, H, params.kv_lora_rank), dtype=torch.float32, device=device)
        self.lse = torch.empty((B, S, H), dtype=torch.float32, device=device)
        self.out = torch.empty((B, S, H, params.head_dim), dtype=dt, device=device)
        ws = max(mla_decode_workspace_bytes(params, num_splits),  # room for the fused route too
                 mla_decode_attn_out_proj_workspace_bytes(params, num_splits))
        self.workspace = torch.empty(max(ws, 16) // 4 + 4, dtype=torch.float32, device=device) if ws else None

    def run(self, q_nope, q_pe, w_uk, w_uv, kv_pool, block_table, seq_lens, stream=None, fp8: bool = False,
            tree_parents=None, fused: bool = False, latent_outputs: bool = True):
        """The three calls; with ``fp8`` the weights are packed FP8 weights and the two projections
        run block-quantised (mla_absorb_q_fp8 / mla_out_proj_fp8); with ``tree_parents`` (B, S)
        int32 the attention is the tree-masked verify (mla_decode_attn_tree).  With ``fused`` the
        attention and the out-projection are one call, mla_decode_attn_out_proj, which writes o_lat
        and lse only with ``latent_outputs``."""
        p = self.params
        (mla_absorb_q_fp8 if fp8 else mla_absorb_q)(q_nope, w_uk, self.q_lat, p, stream)
        if fused:
            (mla_decode_attn_out_proj_fp8 if fp8 else mla_decode_attn_out_proj)(
                self.q_lat, q_pe, kv_pool, block_table, seq_lens, tree_parents, w_uv, self.out,
                self.o_lat if latent_outputs else None, self.lse if latent_outputs else None, self.workspace,
                self.num_splits, p, stream)
            return self.out
        if tree_parents is None:
            mla_decode_attn(self.q_lat, q_pe, kv_pool, block_table, seq_lens, self.o_lat, self.lse, self.workspace,
                            self.num_splits, p, stream)
        else:
            mla_decode_attn_tree(self.q_lat, q_pe, kv_pool, block_table, seq_lens, tree_parents, self.o_lat, self.lse,
                                 self.workspace, self.num_splits, p, stream)
        (mla_out_proj_fp8 if fp8 else mla_out_proj)(self.o_lat, w_uv, self.out, p, stream)
        return self.out
