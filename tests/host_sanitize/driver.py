"""Drive the AddressSanitizer / UndefinedBehaviorSanitizer build of the C-ABI layer (mla_api.cpp
with stubs.cpp in place of the kernels and the HIP runtime), in a process started with the
sanitizer runtime preloaded.  Every "device" buffer is host memory of exactly the size the header
documents (or a size query returns), so a range the layer computes wrongly is an out-of-bounds read
in a launcher stand-in.  Prints one line per case; exits non-zero on any failure (the sanitizers
abort the process themselves).

usage: driver.py <library>
"""
import ctypes
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from deepseek_mla_latent_amd import binding  # noqa: E402  (imports no GPU framework)

lib = binding.declare(ctypes.CDLL(sys.argv[1]), partial=True)
lib.san_launches.argtypes = [ctypes.c_int]
lib.san_launches.restype = ctypes.c_long
lib.san_set_cus.argtypes = [ctypes.c_int]
libc = ctypes.CDLL(None)
libc.posix_memalign.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t, ctypes.c_size_t]
KINDS = dict(attn=0, lse_merge=1, absorb=2, merge_out_proj=3, out_proj=4, kv_up=5, prefill=6, linear=7, quant=8,
             absorb_fp8=9, out_proj_fp8=10, rope=11, merge_out_proj_f32=12)
H, DC, DR, DH, PAGE, ROW = 128, 512, 64, 128, 64, 576
INT32_MAX = 2 ** 31 - 1


def buf(nbytes):
    """nbytes of 16-byte-aligned host memory (the sanitizer's allocator: its end is poisoned); None
    for 0 bytes, like a caller that passes no buffer."""
    if nbytes == 0:
        return None
    p = ctypes.c_void_p()
    assert libc.posix_memalign(ctypes.byref(p), 16, nbytes) == 0
    ctypes.memset(p, 0, nbytes)
    return p.value


def table(batch, pages, num_pages):
    """block table (batch x pages) of valid page ids and the matching seq_lens (host int32)."""
    bt = (ctypes.c_int32 * max(1, batch * pages))()
    for i in range(batch * pages):
        bt[i] = i % max(1, num_pages)
    return bt


def lens(batch, value):
    a = (ctypes.c_int32 * max(1, batch))()
    for i in range(batch):
        a[i] = value
    return a


def addr(x):
    return ctypes.addressof(x) if x is not None and not isinstance(x, int) else x


def expect(code, where, want=0):
    if code != want:
        raise SystemExit(f"FAIL {where}: status {code}, expected {want}")


def launched(kind, before):
    return lib.san_launches(KINDS[kind]) - before[KINDS[kind]]


def counts():
    return [lib.san_launches(k) for k in range(len(KINDS))]


def params(**kw):
    return binding.make_params(**kw)


def case_decode(batch, q_len, max_seq_len, splits, dtype, num_pages=0, tree=False, cus=256, slots=None):
    """slots: the partial slots the workspace must hold (checked against its size when given)."""
    lib.san_set_cus(cus)
    e = 2 if dtype == binding.MLA_BF16 else 4
    p = params(batch=batch, q_len=q_len, max_seq_len=max_seq_len, dtype=dtype, num_pages=num_pages)
    pages = p.max_pages_per_seq
    rows = batch * q_len
    q_lat, q_pe = buf(rows * H * DC * e), buf(rows * H * DR * e)
    pool = buf(max(1, num_pages) * PAGE * ROW * e)
    bt, ln = table(batch, pages, num_pages), lens(batch, max_seq_len)
    o, lse = buf(rows * H * DC * 4), buf(rows * H * 4)
    nbytes = lib.mla_decode_workspace_bytes(ctypes.byref(p), splits)
    if slots is not None:  # partials (bf16 or fp32 rows of 512, fp32 lse) and the (first, count) table
        assert nbytes == slots * H * (DC * e + 4) + 16 + (rows * 8 + 15) // 16 * 16, (nbytes, slots)
    ws = buf(nbytes)
    before = counts()
    if tree:
        par = (ctypes.c_int32 * (batch * q_len))(*([-1] * (batch * q_len)))
        code = lib.mla_decode_attn_tree(q_lat, q_pe, pool, addr(bt), addr(ln), addr(par), o, lse, ws, nbytes, splits,
                                        ctypes.byref(p), None)
    else:
        code = lib.mla_decode_attn(q_lat, q_pe, pool, addr(bt), addr(ln), o, lse, ws, nbytes, splits, ctypes.byref(p),
                                   None)
    expect(code, f"decode B={batch} S={q_len} L={max_seq_len} splits={splits} dtype={dtype}")
    assert launched("attn", before) == (1 if rows else 0)
    n_split = lib.mla_decode_num_splits(ctypes.byref(p), splits)
    assert launched("lse_merge", before) == (1 if rows and n_split > 1 else 0)
    # lse is optional
    code = lib.mla_decode_attn(q_lat, q_pe, pool, addr(bt), addr(ln), o, None, ws, nbytes, splits, ctypes.byref(p),
                               None)
    expect(code, "decode without lse")
    print(f"decode B={batch} S={q_len} L={max_seq_len} splits={splits}->{n_split} dtype={dtype} tree={tree} ok")


def case_fused(batch, q_len, max_seq_len, splits, latent_outputs, fp8=False, dtype=binding.MLA_BF16):
    lib.san_set_cus(256)
    p = params(batch=batch, q_len=q_len, max_seq_len=max_seq_len, dtype=dtype)
    e = 2 if dtype == binding.MLA_BF16 else 4
    rows = batch * q_len
    q_lat, q_pe, pool = buf(rows * H * DC * e), buf(rows * H * DR * e), buf(PAGE * ROW * e)
    bt, ln = table(batch, p.max_pages_per_seq, 1), lens(batch, max_seq_len)
    w_uv = buf(lib.mla_fp8_weight_bytes() if fp8 else H * DC * DH * e)
    out = buf(rows * H * DH * e)
    o = buf(rows * H * DC * 4) if latent_outputs else None
    lse = buf(rows * H * 4) if latent_outputs else None
    nbytes = lib.mla_decode_attn_out_proj_workspace_bytes(ctypes.byref(p), splits)
    ws = buf(nbytes)
    before = counts()
    call = lib.mla_decode_attn_out_proj_fp8 if fp8 else lib.mla_decode_attn_out_proj
    code = call(q_lat, q_pe, pool, addr(bt), addr(ln), None, w_uv, out, o, lse, ws, nbytes, splits, ctypes.byref(p),
                None)
    expect(code, f"fused B={batch} S={q_len} splits={splits} fp8={fp8}")
    assert launched("attn", before) == 1
    assert launched("merge_out_proj", before) + launched("merge_out_proj_f32", before) + \
        launched("out_proj_fp8" if fp8 else "out_proj", before) == 1
    if dtype == binding.MLA_F32 and rows <= 4 and lib.mla_decode_num_splits(ctypes.byref(p), splits) > 1:
        assert launched("merge_out_proj_f32", before) == 1 and launched("lse_merge", before) == 0
    print(f"fused B={batch} S={q_len} L={max_seq_len} splits={splits} latent={latent_outputs} fp8={fp8} "
          f"dtype={dtype} ok (merge in W_UV: {launched('merge_out_proj', before)}, "
          f"in the fp32 GEMV: {launched('merge_out_proj_f32', before)})")


def case_projections(tokens, dtype):
    e = 2 if dtype == binding.MLA_BF16 else 4
    p = params(batch=tokens, q_len=1, max_seq_len=64, dtype=dtype)
    q_nope, w, q_lat = buf(tokens * H * DH * e), buf(H * DC * DH * e), buf(tokens * H * DC * e)
    expect(lib.mla_absorb_q(q_nope, w, q_lat, ctypes.byref(p), None), "absorb")
    o_lat, out = buf(tokens * H * DC * 4), buf(tokens * H * DH * e)
    expect(lib.mla_out_proj(o_lat, w, out, ctypes.byref(p), None), "out_proj")
    if dtype == binding.MLA_BF16:
        nb = lib.mla_fp8_weight_bytes()
        packed = buf(nb)
        expect(lib.mla_quantize_w_uk_fp8(w, packed, nb, ctypes.byref(p), None), "quantize uk")
        expect(lib.mla_quantize_w_uv_fp8(w, packed, nb, ctypes.byref(p), None), "quantize uv")
        expect(lib.mla_absorb_q_fp8(q_nope, packed, q_lat, ctypes.byref(p), None), "absorb fp8")
        expect(lib.mla_out_proj_fp8(o_lat, packed, out, ctypes.byref(p), None), "out_proj fp8")
    print(f"projections tokens={tokens} dtype={dtype} ok")


def case_prefill(batch, q_len, max_seq_len, extra_pages):
    pages = -(-max_seq_len // PAGE) + extra_pages
    p = params(batch=batch, q_len=q_len, max_seq_len=max_seq_len, max_pages_per_seq=pages, num_pages=batch * pages)
    pool = buf(batch * pages * PAGE * ROW * 2)
    bt, ln = table(batch, pages, batch * pages), lens(batch, max_seq_len)
    w = buf(H * DC * DH * 2)
    nbytes = lib.mla_prefill_kv_bytes(ctypes.byref(p))
    kv = buf(nbytes)
    expect(lib.mla_prefill_kv_up(pool, addr(bt), addr(ln), w, w, kv, nbytes, ctypes.byref(p), None), "kv_up")
    rows = batch * q_len
    q_nope, q_pe, out, lse = buf(rows * H * DH * 2), buf(rows * H * DR * 2), buf(rows * H * DH * 2), buf(rows * H * 4)
    expect(lib.mla_prefill_attn(q_nope, q_pe, kv, nbytes, addr(ln), out, lse, ctypes.byref(p), None), "prefill_attn")
    print(f"prefill B={batch} S={q_len} L={max_seq_len} table pages={pages} ok")


def case_linear(m, k, n, cus):
    lib.san_set_cus(cus)
    x, w, y = buf(m * k * 2), buf(k * n * 2), buf(m * n * 2)
    nbytes = lib.mla_linear_workspace_bytes(m, k, n)
    ws = buf(nbytes)
    expect(lib.mla_linear(x, w, y, m, k, n, ws, nbytes, None), f"linear {m}x{k}x{n}")
    print(f"linear M={m} K={k} N={n} cus={cus} workspace={nbytes} ok")


def case_rope(batch, q_len, cache, stride):
    p = params(batch=batch, q_len=q_len, max_seq_len=cache, num_pages=batch * -(-cache // PAGE))
    rows = batch * q_len
    q_pe, kv_a = buf(rows * H * DR * 2), buf(((rows - 1) * stride + ROW) * 2)
    pool = buf(p.num_pages * PAGE * ROW * 2)
    bt, ln = table(batch, p.max_pages_per_seq, p.num_pages), lens(batch, cache)
    expect(lib.mla_rope_append(q_pe, kv_a, stride, pool, addr(bt), addr(ln), 10000.0, ctypes.byref(p), None), "rope")
    print(f"rope B={batch} S={q_len} L={cache} stride={stride} ok")


def case_extremes():
    """Size queries at the edges of every field: the arithmetic must neither overflow nor crash."""
    for kw in (dict(batch=1, q_len=1, max_seq_len=INT32_MAX), dict(batch=1 << 24, q_len=1, max_seq_len=INT32_MAX),
               dict(batch=1, q_len=1 << 24, max_seq_len=INT32_MAX), dict(batch=INT32_MAX, q_len=INT32_MAX, max_seq_len=0),
               dict(batch=4096, q_len=4096, max_seq_len=1 << 20), dict(batch=0, q_len=1, max_seq_len=INT32_MAX)):
        p = params(**kw, max_pages_per_seq=INT32_MAX)
        for s in (0, 1, 2, 7, INT32_MAX):
            lib.mla_decode_workspace_bytes(ctypes.byref(p), s)
            lib.mla_decode_num_splits(ctypes.byref(p), s)
            lib.mla_decode_attn_out_proj_workspace_bytes(ctypes.byref(p), s)
        lib.mla_prefill_kv_bytes(ctypes.byref(p))
    for m, k, n in ((INT32_MAX, 64, 64), (64, 1 << 30, 64), (1, 64, INT32_MAX - 63), (0, 64, 64)):
        lib.mla_linear_workspace_bytes(m, k, n)
    for code in list(binding.STATUS) + [-99, INT32_MAX, -INT32_MAX - 1]:
        lib.mla_status_str(code)
    print("extremes ok")


if __name__ == "__main__":
    case_extremes()
    for dt in (binding.MLA_BF16, binding.MLA_F32):
        case_decode(5, 1, 300, 0, dt)
        case_decode(5, 1, 300, 1, dt)
        case_decode(2, 2, 1000, 3, dt, num_pages=40)
        case_decode(3, 1, 0, 0, dt)  # no cached token at all
        case_decode(0, 1, 100, 0, dt)  # empty batch
        case_projections(3, dt)
    case_decode(1, 1, PAGE * 512 * 2 + 1, 0, binding.MLA_BF16)  # more pages than one workgroup stages
    case_decode(64, 2, 16386, 0, binding.MLA_BF16, cus=304)
    # 33..256 rows, bf16, the library's split count: up to ceil(9/8 * CUs) ranges (longest first)
    case_decode(128, 1, 8192, 0, binding.MLA_BF16, cus=256, slots=288)
    case_decode(128, 1, 8192, 2, binding.MLA_BF16, cus=256, slots=256)  # split count given: rows * k
    case_decode(128, 1, 8192, 0, binding.MLA_F32, cus=256, slots=256)   # fp32: rows * k
    case_decode(32, 1, 4096, 0, binding.MLA_BF16, cus=256, slots=256)   # 32 rows: rows * k
    case_decode(100, 1, 8192, 0, binding.MLA_BF16, cus=256, slots=300)  # rows * k = 300 >= 288
    case_decode(2, 8, 4104, 2, binding.MLA_BF16, tree=True)
    case_decode(2, 8, 4104, 0, binding.MLA_BF16, tree=True, cus=1)
    case_fused(16, 1, 700, 2, False)
    case_fused(16, 1, 700, 2, True)
    case_fused(2, 1, 700, 2, False)
    case_fused(2, 1, 700, 1, False)
    case_fused(32, 1, 4096, 0, True)
    case_fused(128, 1, 8192, 0, True)  # the merge in the W_UV kernel over 288 partial slots
    for args in ((1, 1, 512, 0, False), (1, 1, 512, 0, True), (2, 2, 700, 3, True), (1, 1, 300, 1, True),
                 (6, 1, 700, 0, False)):  # fp32: the merge in the GEMV (<= 4 rows), else separate kernels
        case_fused(*args, dtype=binding.MLA_F32)
    for args in ((16, 1, 700, 2, False), (2, 1, 700, 2, True), (32, 1, 4096, 0, True), (4, 1, 300, 1, False)):
        case_fused(*args, fp8=True)
    case_prefill(2, 96, 160, 0)
    case_prefill(1, 300, 300, 2)
    for m, k, n, cus in ((32, 1024, 512, 256), (600, 7168, 2112, 256), (1, 64, 64, 1), (0, 64, 64, 256)):
        case_linear(m, k, n, cus)
    case_rope(3, 2, 130, ROW)
    case_rope(2, 1, 64, 1024)
    print("DRIVER OK")
