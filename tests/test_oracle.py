"""Pins of the fp64 decode oracle against things other than itself.

* (a) the absorbed order (W_UK folded into the query, W_UV applied after the
  latent sum) agrees with the non-absorbed order — the identity the izhida
  answer "专家" and §二/§三 of the absorption note rest on;
* (c) softmax rows sum to one and are non-negative;
* special cases with closed forms (one key; zero query -> mean of the keys);
* W_UK = W_UV = [I; 0] turns MLA into MQA with a 192-d key, which must equal
  torch's scaled_dot_product_attention (a library routine) in fp64;
* causal S = 2 equals two S = 1 calls; paging is invisible; splitting the
  keys in two and merging the halves by log-sum-exp gives the whole;
* tiny inputs against a brute-force pure-Python evaluation.
"""
import math

import numpy as np
import pytest
import torch

from deepseek_mla_latent_amd import inputs as gen
from oracle import mla_decode as ref


def _tiny(seed=0, B=2, S=2, H=4, Dc=16, Dr=4, Dh=8, lens=(7, 13), page=4, paged=True):
    """Hand-made tiny problem with distinct dims so any transposed operand breaks shapes or values."""
    rng = np.random.default_rng(seed)
    lens = np.array(lens, dtype=np.int32)
    npg = [-(-int(L) // page) for L in lens]
    P = sum(npg)
    order = rng.permutation(P) if paged else np.arange(P)
    bt = np.full((B, max(npg)), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        bt[b, :npg[b]] = order[off:off + npg[b]]
        off += npg[b]
    pool = rng.standard_normal((P, page, Dc + Dr))
    return dict(q_nope=rng.standard_normal((B, S, H, Dh)), q_pe=rng.standard_normal((B, S, H, Dr)),
                w_uk=rng.standard_normal((H, Dc, Dh)) / math.sqrt(Dc),
                w_uv=rng.standard_normal((H, Dc, Dh)) / math.sqrt(Dc),
                pool=pool, block_table=bt, seq_lens=lens, page=page, Dc=Dc)


def _absorbed(t, scale, causal=True):
    q_lat = ref.absorb_q_reference(t["q_nope"], t["w_uk"])
    att = ref.latent_attention_reference(q_lat, t["q_pe"], t["pool"], t["block_table"], t["seq_lens"],
                                         softmax_scale=scale, page_size=t["page"], causal=causal)
    return att["o_lat"], att["lse"], ref.out_proj_reference(att["o_lat"], t["w_uv"])


def _nonabsorbed(t, scale, causal=True, **kw):
    return ref.mla_decode_nonabsorbed(t["q_nope"], t["q_pe"], t["w_uk"], t["w_uv"], t["pool"], t["block_table"],
                                      t["seq_lens"], softmax_scale=scale, page_size=t["page"], causal=causal, **kw)


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


@pytest.mark.parametrize("causal", [True, False])
def test_absorbed_equals_nonabsorbed_tiny(causal):
    t = _tiny()
    scale = 1 / math.sqrt(12)
    o_lat, lse, out = _absorbed(t, scale, causal)
    r = _nonabsorbed(t, scale, causal)
    assert _rel(o_lat, r["o_lat"]) < 1e-12
    assert np.max(np.abs(lse - r["lse"])) < 1e-12
    assert _rel(out, r["out"]) < 1e-12


def test_absorbed_equals_nonabsorbed_real_dims():
    """Same identity at the real head dims (128 heads, d_c 512, d_R 64, d_h 128), paged, S = 2."""
    w = gen.small_workload(2, 2, ragged=(70, 200), dtype="f32", paged=True)
    x = gen.generate(w, 11)
    t = dict(q_nope=x.q_nope, q_pe=x.q_pe, w_uk=x.w_uk, w_uv=x.w_uv, pool=x.pool, block_table=x.block_table,
             seq_lens=x.seq_lens, page=64, Dc=512)
    o_lat, lse, out = _absorbed(t, w.softmax_scale)
    r = _nonabsorbed(t, w.softmax_scale)
    assert _rel(o_lat, r["o_lat"]) < 1e-12
    assert np.max(np.abs(lse - r["lse"])) < 1e-12
    assert _rel(out, r["out"]) < 1e-12


def test_softmax_rows_sum_to_one():
    t = _tiny(seed=3)
    r = _nonabsorbed(t, 0.3, return_probs=True)
    for (b, i, h), p in r["probs"].items():
        assert np.all(p >= 0)
        assert abs(p.sum() - 1.0) < 1e-12
        # and lse is the log-normaliser: exp(z - lse) sums to one (recomputed from the logits)
        assert len(p) == ref.visible_keys(int(t["seq_lens"][b]), 2, i, True)


@pytest.mark.parametrize("tree", [False, True])
def test_softmax_mass_of_the_oracle_lse_is_one(tree):
    """softmax_mass recomputes the absorbed logits itself; fed the lse of the non-absorbed route it
    must give exactly one per row, fed lse + d it must give e^{-d}, and counting keys the row does
    not see (a wrong mask) must show as mass above one."""
    t = _tiny(seed=5, S=3, lens=(9, 13))
    scale = 0.4
    parents = np.array([[-1, 0, 0], [-1, -1, 1]], dtype=np.int32) if tree else None
    r = _nonabsorbed(t, scale, tree=parents)
    q_lat = ref.absorb_q_reference(t["q_nope"], t["w_uk"])
    rows = [(b, i, h) for b in range(2) for i in range(3) for h in range(4)]
    kw = dict(softmax_scale=scale, page_size=t["page"], tree=parents)
    m = ref.softmax_mass(q_lat, t["q_pe"], t["pool"], t["block_table"], t["seq_lens"], r["lse"], rows, **kw)
    assert np.max(np.abs(m - 1.0)) < 1e-12
    m2 = ref.softmax_mass(q_lat, t["q_pe"], t["pool"], t["block_table"], t["seq_lens"], r["lse"] + 0.25, rows, **kw)
    np.testing.assert_allclose(m2, np.exp(-0.25), rtol=1e-12)
    if not tree:
        wide = ref.softmax_mass(q_lat, t["q_pe"], t["pool"], t["block_table"], t["seq_lens"], r["lse"], rows,
                                softmax_scale=scale, page_size=t["page"], causal=False)
        first = [k for k, (b, i, h) in enumerate(rows) if i == 0]
        assert np.all(wide[first] > 1.0 + 1e-6)


def test_softmax_mass_single_key_by_hand():
    t = _tiny(seed=6, B=1, S=1, lens=(1,))
    row = t["pool"][t["block_table"][0, 0], 0]
    q_lat = ref.absorb_q_reference(t["q_nope"], t["w_uk"])
    z = 0.9 * (q_lat[0, 0, 2] @ row[:16] + t["q_pe"][0, 0, 2] @ row[16:])
    lse = np.zeros((1, 1, 4))
    lse[0, 0, 2] = 1.5
    m = ref.softmax_mass(q_lat, t["q_pe"], t["pool"], t["block_table"], t["seq_lens"], lse, [(0, 0, 2)],
                         softmax_scale=0.9, page_size=t["page"])
    assert abs(m[0] - math.exp(z - 1.5)) < 1e-12
    empty = ref.softmax_mass(q_lat, t["q_pe"], t["pool"], t["block_table"], np.array([0]), lse, [(0, 0, 2)],
                             softmax_scale=0.9, page_size=t["page"])
    assert np.isnan(empty[0])


def test_single_key_returns_that_key():
    """L = 1: p = [1], o_lat = c_0, out = W_UV^T c_0, lse = the one logit."""
    t = _tiny(seed=4, B=1, S=1, lens=(1,))
    scale = 0.7
    r = _nonabsorbed(t, scale)
    row = t["pool"][t["block_table"][0, 0], 0]
    c0, k0 = row[:16], row[16:]
    np.testing.assert_array_equal(r["o_lat"][0, 0], np.broadcast_to(c0, (4, 16)))
    for h in range(4):
        z = scale * (t["q_nope"][0, 0, h] @ (t["w_uk"][h].T @ c0) + t["q_pe"][0, 0, h] @ k0)
        assert abs(r["lse"][0, 0, h] - z) < 1e-12
        np.testing.assert_allclose(r["out"][0, 0, h], t["w_uv"][h].T @ c0, rtol=1e-12, atol=1e-12)


def test_zero_query_gives_mean_of_latent():
    """q_nope = q_pe = 0: every logit is 0, p is uniform, o_lat is the mean latent, lse = ln n."""
    t = _tiny(seed=5, S=1)
    t["q_nope"][:] = 0
    t["q_pe"][:] = 0
    r = _nonabsorbed(t, 1.0)
    for b in range(2):
        L = int(t["seq_lens"][b])
        rows = np.array([t["pool"][t["block_table"][b, j // 4], j % 4] for j in range(L)])
        np.testing.assert_allclose(r["o_lat"][b, 0], np.broadcast_to(rows[:, :16].mean(0), (4, 16)), rtol=1e-12,
                                   atol=1e-13)
        np.testing.assert_allclose(r["lse"][b, 0], math.log(L), rtol=1e-13)


def test_identity_weights_reduce_to_sdpa():
    """W_UK[h] = W_UV[h] = [I_128; 0] -> MQA with q=[q_nope|q_pe], k=[c[:128]|k_pe], v=c[:128].

    torch's scaled_dot_product_attention (fp64, CPU) with its default scale
    1/sqrt(192) and an explicit bottom-right causal mask must give ``out``.
    """
    w = gen.small_workload(2, 2, ragged=(65, 150), dtype="f32", paged=True)
    x = gen.generate(w, 7)
    eye = np.zeros((128, 512, 128))
    eye[:, np.arange(128), np.arange(128)] = 1.0
    r = ref.mla_decode_nonabsorbed(x.q_nope, x.q_pe, eye, eye, x.pool, x.block_table, x.seq_lens,
                                   softmax_scale=w.softmax_scale)
    for b in range(2):
        L = int(x.seq_lens[b])
        rows = ref.gather_rows(x.pool, x.block_table[b], L, 64)
        q = torch.from_numpy(np.concatenate([x.q_nope[b], x.q_pe[b]], -1).astype(np.float64))  # (S,H,192)
        k = torch.from_numpy(np.concatenate([rows[:, :128], rows[:, 512:]], -1))  # (L,192)
        v = torch.from_numpy(rows[:, :128].copy())
        q = q.permute(1, 0, 2)  # (H,S,192)
        kk = k.unsqueeze(0).expand(128, L, 192).contiguous()
        vv = v.unsqueeze(0).expand(128, L, 128).contiguous()
        mask = torch.zeros(2, L, dtype=torch.bool)
        for i in range(2):
            mask[i, :L - 2 + i + 1] = True
        o = torch.nn.functional.scaled_dot_product_attention(q, kk, vv, attn_mask=mask)  # (H,S,128)
        np.testing.assert_allclose(r["out"][b], o.permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)
        assert abs(w.softmax_scale - 1 / math.sqrt(192)) < 1e-15


def test_causal_two_tokens_equal_two_single_calls():
    t = _tiny(seed=6)
    r2 = _nonabsorbed(t, 0.5)
    for i in range(2):
        t1 = dict(t)
        t1["q_nope"] = t["q_nope"][:, i:i + 1]
        t1["q_pe"] = t["q_pe"][:, i:i + 1]
        t1["seq_lens"] = t["seq_lens"] - 2 + i + 1
        r1 = _nonabsorbed(t1, 0.5)
        for key in ("o_lat", "lse", "out"):
            np.testing.assert_allclose(r2[key][:, i], r1[key][:, 0], rtol=1e-13, atol=1e-14)


def test_paging_is_invisible():
    """Same tokens, contiguous vs permuted pages: bitwise equal results."""
    a = _tiny(seed=8, paged=False)
    b = dict(a)
    rng = np.random.default_rng(99)
    P = a["pool"].shape[0]
    perm = rng.permutation(P)  # new page id of old page p is perm[p]
    pool2 = np.empty_like(a["pool"])
    pool2[perm] = a["pool"]
    bt2 = np.where(a["block_table"] >= 0, perm[np.maximum(a["block_table"], 0)], -1)
    b["pool"], b["block_table"] = pool2, bt2
    ra, rb = _nonabsorbed(a, 0.4), _nonabsorbed(b, 0.4)
    for key in ("o_lat", "lse", "out"):
        np.testing.assert_array_equal(ra[key], rb[key])


def test_lse_merge_of_two_key_halves():
    """Attention over keys [0,a) and [a,n) merged by o = Σ e^(lse_k - lse) o_k, lse = log Σ e^lse_k."""
    t = _tiny(seed=9, B=1, S=1, lens=(16,), paged=False)
    q_lat = ref.absorb_q_reference(t["q_nope"], t["w_uk"])
    full = ref.latent_attention_reference(q_lat, t["q_pe"], t["pool"], t["block_table"], t["seq_lens"],
                                          softmax_scale=0.6, page_size=4, causal=False)
    # first 8 tokens = pages 0,1 ; last 8 tokens = pages 2,3
    lo = ref.latent_attention_reference(q_lat, t["q_pe"], t["pool"], t["block_table"][:, :2], np.array([8]),
                                        softmax_scale=0.6, page_size=4, causal=False)
    hi = ref.latent_attention_reference(q_lat, t["q_pe"], t["pool"], t["block_table"][:, 2:], np.array([8]),
                                        softmax_scale=0.6, page_size=4, causal=False)
    lse = np.logaddexp(lo["lse"], hi["lse"])
    o = np.exp(lo["lse"] - lse)[..., None] * lo["o_lat"] + np.exp(hi["lse"] - lse)[..., None] * hi["o_lat"]
    np.testing.assert_allclose(lse, full["lse"], rtol=1e-13)
    np.testing.assert_allclose(o, full["o_lat"], rtol=1e-12, atol=1e-14)


def test_empty_key_set():
    """L = 0: o_lat = 0, out = 0, lse = -inf (empty sum)."""
    t = _tiny(seed=10, B=2, S=1, lens=(0, 3))
    t["block_table"][0, :] = -1
    r = _nonabsorbed(t, 1.0)
    assert np.all(r["o_lat"][0] == 0) and np.all(r["out"][0] == 0) and np.all(np.isneginf(r["lse"][0]))
    assert np.all(np.isfinite(r["lse"][1]))


def test_brute_force_tiny():
    """Pure-Python loops over every (b, i, h, j), the absorbed form, math.fsum."""
    t = _tiny(seed=12, B=1, S=2, H=2, Dc=3, Dr=2, Dh=2, lens=(5,), page=2)
    scale = 0.9
    r = _nonabsorbed(t, scale)
    Wk, Wv, qn, qp = t["w_uk"], t["w_uv"], t["q_nope"], t["q_pe"]
    L = 5
    rows = [t["pool"][t["block_table"][0, j // 2], j % 2] for j in range(L)]
    for i in range(2):
        n = L - 2 + i + 1
        for h in range(2):
            qlat = [math.fsum(Wk[h, c, d] * qn[0, i, h, d] for d in range(2)) for c in range(3)]
            z = [scale * (math.fsum(qlat[c] * rows[j][c] for c in range(3)) +
                          math.fsum(qp[0, i, h, r_] * rows[j][3 + r_] for r_ in range(2))) for j in range(n)]
            mx = max(z)
            e = [math.exp(v - mx) for v in z]
            s = math.fsum(e)
            olat = [math.fsum(e[j] / s * rows[j][c] for j in range(n)) for c in range(3)]
            out = [math.fsum(olat[c] * Wv[h, c, v] for c in range(3)) for v in range(2)]
            np.testing.assert_allclose(r["o_lat"][0, i, h], olat, rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(r["out"][0, i, h], out, rtol=1e-12, atol=1e-14)
            assert abs(r["lse"][0, i, h] - (mx + math.log(s))) < 1e-12


def test_projection_references_are_matmuls():
    """absorb / out-projection references against an independent library contraction (torch.einsum, fp64)."""
    rng = np.random.default_rng(13)
    q = rng.standard_normal((3, 2, 4, 8))
    w = rng.standard_normal((4, 16, 8))
    o = rng.standard_normal((3, 2, 4, 16))
    np.testing.assert_allclose(ref.absorb_q_reference(q, w),
                               torch.einsum("bshd,hcd->bshc", torch.from_numpy(q), torch.from_numpy(w)).numpy(),
                               rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(ref.out_proj_reference(o, w),
                               torch.einsum("bshc,hcd->bshd", torch.from_numpy(o), torch.from_numpy(w)).numpy(),
                               rtol=1e-13, atol=1e-13)


def test_planted_mistakes_are_caught():
    """A dropped RoPE term or a wrong scale in a copy of the oracle breaks the SDPA pin."""
    w = gen.small_workload(1, 1, cache_len=70, dtype="f32", paged=False)
    x = gen.generate(w, 5)
    eye = np.zeros((128, 512, 128))
    eye[:, np.arange(128), np.arange(128)] = 1.0
    good = ref.mla_decode_nonabsorbed(x.q_nope, x.q_pe, eye, eye, x.pool, x.block_table, x.seq_lens,
                                      softmax_scale=w.softmax_scale)["out"]
    no_rope = ref.mla_decode_nonabsorbed(x.q_nope, np.zeros_like(x.q_pe), eye, eye, x.pool, x.block_table,
                                         x.seq_lens, softmax_scale=w.softmax_scale)["out"]
    wrong_scale = ref.mla_decode_nonabsorbed(x.q_nope, x.q_pe, eye, eye, x.pool, x.block_table, x.seq_lens,
                                             softmax_scale=1 / math.sqrt(128))["out"]
    assert _rel(no_rope, good) > 1e-3
    assert _rel(wrong_scale, good) > 1e-3


def test_three_orders_of_the_second_absorption_agree():
    """[note] §三: W_O[score(W_UV c)] (order 1), W_O[W_UV(score c)] (order 2) and (W_O W_UV)(score c)
    (order 3, the fused (h, k, e) weight formed with a library einsum) give the same output."""
    t = _tiny(seed=21)
    rng = np.random.default_rng(22)
    H, Dc, Dv = t["w_uv"].shape
    w_o = rng.standard_normal((H, Dv, 10)) / math.sqrt(H * Dv)
    r = _nonabsorbed(t, 0.7)  # order 1: per-head V, then attention
    y1 = ref.o_proj_reference(r["out"], w_o)
    y2 = ref.o_proj_reference(ref.out_proj_reference(r["o_lat"], t["w_uv"]), w_o)  # order 2
    w_ouv = torch.einsum("hkv,hve->hke", torch.from_numpy(t["w_uv"]), torch.from_numpy(w_o)).numpy()
    y3 = torch.einsum("bshk,hke->bse", torch.from_numpy(r["o_lat"]), torch.from_numpy(w_ouv)).numpy()  # order 3
    np.testing.assert_allclose(y1, y3, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(y2, y3, rtol=1e-11, atol=1e-12)
    # a dropped head in the sum (a plausible indexing mistake) is caught
    y_bad = ref.o_proj_reference(r["out"][:, :, 1:], w_o[1:])
    assert not np.allclose(y_bad, y3, rtol=1e-6)
