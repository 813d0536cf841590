"""Pins of the fp64 prefill oracle (multi-head form) against things other than itself.

* the up-projection agrees with the absorbed identities the pages rest on: q . (C W_UK)_j equals
  (W_UK q) . c_j (absorb_q_reference), and sum_j p_j (C W_UV)_j equals W_UV^T sum_j p_j c_j
  (out_proj_reference) — izhida answer "专家", absorption note §二 / §三;
* W = [I; 0] makes K and V the first d_h latent columns;
* per-head attention equals torch's scaled_dot_product_attention in fp64 (a library routine):
  with its own causal flag for a whole prompt (S = L), with an explicit bottom-right mask for a
  chunk (S < L), and without a mask; lse equals torch.logsumexp of the masked scaled logits;
* the two steps together equal the non-absorbed decode reference (pinned on its own);
* tiny inputs against a brute-force pure-Python evaluation;
* an off-by-one causal rule or dropped RoPE term planted into the oracle breaks the SDPA pin.
"""
import math

import numpy as np
import pytest
import torch

from oracle import mla_decode as ref
from oracle import mla_prefill as pf


def _tiny(seed=0, B=2, S=None, H=3, Dc=16, Dr=4, Dh=8, lens=(9, 13), page=4):
    """Distinct dims so a transposed operand breaks shapes; S defaults to the whole prompt."""
    rng = np.random.default_rng(seed)
    lens = np.array(lens, dtype=np.int32)
    S = int(lens.min()) if S is None else S
    npg = [-(-int(L) // page) for L in lens]
    P = sum(npg)
    order = rng.permutation(P)
    bt = np.full((B, max(npg)), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        bt[b, :npg[b]] = order[off:off + npg[b]]
        off += npg[b]
    return dict(q_nope=rng.standard_normal((B, S, H, Dh)), q_pe=rng.standard_normal((B, S, H, Dr)),
                w_uk=rng.standard_normal((H, Dc, Dh)) / math.sqrt(Dc), w_uv=rng.standard_normal((H, Dc, Dh)) / math.sqrt(Dc),
                pool=rng.standard_normal((P, page, Dc + Dr)), block_table=bt, seq_lens=lens, page=page, Dc=Dc, S=S)


def _prefill(t, scale, causal=True):
    K, V, kpe = pf.kv_up_reference(t["pool"], t["block_table"], t["seq_lens"], t["w_uk"], t["w_uv"],
                                   page_size=t["page"])
    return pf.mha_attention_reference(t["q_nope"], t["q_pe"], K, V, kpe, t["seq_lens"], softmax_scale=scale,
                                      causal=causal)


def test_kv_up_identity_weights():
    t = _tiny(seed=1)
    H, Dc, Dh = t["w_uk"].shape
    eye = np.zeros((H, Dc, Dh))
    eye[:, np.arange(Dh), np.arange(Dh)] = 1.0
    K, V, kpe = pf.kv_up_reference(t["pool"], t["block_table"], t["seq_lens"], eye, eye, page_size=t["page"])
    for b, L in enumerate(t["seq_lens"]):
        rows = np.stack([t["pool"][t["block_table"][b, j // t["page"]], j % t["page"]] for j in range(L)])
        for h in range(H):
            np.testing.assert_array_equal(K[b, h, :L], rows[:, :Dh])
            np.testing.assert_array_equal(V[b, h, :L], rows[:, :Dh])
        np.testing.assert_array_equal(kpe[b, :L], rows[:, Dc:])
        assert np.all(np.isnan(K[b, :, L:])) and np.all(np.isnan(kpe[b, L:]))


def test_kv_up_matches_absorbed_identities():
    """q . K_j = (W_UK q) . c_j and sum_j p_j V_j = W_UV^T sum_j p_j c_j for every head."""
    t = _tiny(seed=2)
    K, V, _ = pf.kv_up_reference(t["pool"], t["block_table"], t["seq_lens"], t["w_uk"], t["w_uv"], page_size=t["page"])
    rng = np.random.default_rng(3)
    H, Dc, Dh = t["w_uk"].shape
    for b, L in enumerate(t["seq_lens"]):
        C = ref.gather_rows(t["pool"], t["block_table"][b], int(L), t["page"])[:, :Dc]
        q = rng.standard_normal((1, 1, H, Dh))
        q_lat = ref.absorb_q_reference(q, t["w_uk"])[0, 0]  # (H, Dc)
        p = rng.random((H, L))
        o_lat = (p @ C)[None, None]  # (1,1,H,Dc): sum_j p_j c_j per head
        via_latent = ref.out_proj_reference(o_lat, t["w_uv"])[0, 0]
        for h in range(H):
            np.testing.assert_allclose(K[b, h, :L] @ q[0, 0, h], C @ q_lat[h], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(p[h] @ V[b, h, :L], via_latent[h], rtol=1e-12, atol=1e-12)


def _sdpa(t, scale, mask):
    """torch SDPA (fp64) per sequence: q = [q_nope | q_pe], k = [K | kpe], v = V; mask builder or flag."""
    K, V, kpe = pf.kv_up_reference(t["pool"], t["block_table"], t["seq_lens"], t["w_uk"], t["w_uv"], page_size=t["page"])
    outs, lses = [], []
    for b, L in enumerate(t["seq_lens"]):
        L = int(L)
        q = torch.from_numpy(np.concatenate([t["q_nope"][b], t["q_pe"][b]], -1)).permute(1, 0, 2)  # (H,S,d)
        H = q.shape[0]
        k = torch.from_numpy(np.concatenate([K[b, :, :L], np.broadcast_to(kpe[b, :L], (H, L, kpe.shape[-1]))], -1))
        v = torch.from_numpy(V[b, :, :L].copy())
        m = mask(t["S"], L)
        if m == "is_causal":
            o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=scale)
            mm = torch.ones(t["S"], L, dtype=torch.bool).tril()
        else:
            o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=m, scale=scale)
            mm = m
        z = (q @ k.transpose(1, 2)) * scale
        lses.append(torch.logsumexp(z.masked_fill(~mm, -math.inf), -1).permute(1, 0).numpy())
        outs.append(o.permute(1, 0, 2).numpy())
    return np.stack(outs), np.stack(lses)


def _bottom_right(S, L):
    return torch.ones(S, L, dtype=torch.bool).tril(diagonal=L - S)


@pytest.mark.parametrize("case", ["whole_prompt", "chunk", "non_causal"])
def test_mha_matches_sdpa(case):
    if case == "whole_prompt":  # S = L for every sequence: torch's own causal flag
        t, causal, mask = _tiny(seed=4, lens=(11, 11)), True, (lambda S, L: "is_causal")
    elif case == "chunk":  # the last S of L tokens are new
        t, causal, mask = _tiny(seed=5, lens=(9, 14), S=5), True, _bottom_right
    else:
        t, causal, mask = _tiny(seed=6, lens=(9, 14), S=5), False, (lambda S, L: torch.ones(S, L, dtype=torch.bool))
    scale = 1 / math.sqrt(t["q_nope"].shape[-1] + t["q_pe"].shape[-1])
    r = _prefill(t, scale, causal)
    o, lse = _sdpa(t, scale, mask)
    np.testing.assert_allclose(r["out"], o, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(r["lse"], lse, rtol=1e-12, atol=1e-12)


def test_two_steps_equal_nonabsorbed_decode_reference():
    t = _tiny(seed=7, lens=(10, 13), S=6)
    r = _prefill(t, 0.45)
    d = ref.mla_decode_nonabsorbed(t["q_nope"], t["q_pe"], t["w_uk"], t["w_uv"], t["pool"], t["block_table"],
                                   t["seq_lens"], softmax_scale=0.45, page_size=t["page"])
    np.testing.assert_allclose(r["out"], d["out"], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(r["lse"], d["lse"], rtol=1e-13, atol=1e-13)


def test_brute_force_tiny():
    """Pure-Python loops, math.fsum, a whole prompt of 5 tokens."""
    t = _tiny(seed=8, B=1, H=2, Dc=3, Dr=2, Dh=2, lens=(5,), page=2)
    scale = 0.8
    r = _prefill(t, scale)
    rows = [t["pool"][t["block_table"][0, j // 2], j % 2] for j in range(5)]
    Wk, Wv, qn, qp = t["w_uk"], t["w_uv"], t["q_nope"], t["q_pe"]
    for h in range(2):
        Kh = [[math.fsum(rows[j][c] * Wk[h, c, d] for c in range(3)) for d in range(2)] for j in range(5)]
        Vh = [[math.fsum(rows[j][c] * Wv[h, c, d] for c in range(3)) for d in range(2)] for j in range(5)]
        for i in range(5):
            z = [scale * (math.fsum(qn[0, i, h, d] * Kh[j][d] for d in range(2)) +
                          math.fsum(qp[0, i, h, e] * rows[j][3 + e] for e in range(2))) for j in range(i + 1)]
            mx = max(z)
            w = [math.exp(v - mx) for v in z]
            s = math.fsum(w)
            out = [math.fsum(w[j] / s * Vh[j][d] for j in range(i + 1)) for d in range(2)]
            np.testing.assert_allclose(r["out"][0, i, h], out, rtol=1e-12, atol=1e-14)
            assert abs(r["lse"][0, i, h] - (mx + math.log(s))) < 1e-12


def test_planted_mistakes_are_caught(monkeypatch):
    """An off-by-one causal rule, or a dropped RoPE term, put into the oracle breaks the SDPA pin."""
    t = _tiny(seed=9, lens=(11, 11))
    scale = 0.5
    o, _ = _sdpa(t, scale, lambda S, L: "is_causal")
    assert np.allclose(_prefill(t, scale)["out"], o, rtol=1e-10, atol=1e-12)

    good = pf.visible_keys
    monkeypatch.setattr(pf, "visible_keys", lambda L, S, i, causal: good(L, S, i, causal) - 1 if causal else L)
    assert not np.allclose(_prefill(t, scale)["out"], o, rtol=1e-6, atol=1e-8, equal_nan=False)
    monkeypatch.setattr(pf, "visible_keys", good)

    t2 = dict(t)
    t2["q_pe"] = np.zeros_like(t["q_pe"])
    assert not np.allclose(_prefill(t2, scale)["out"], o, rtol=1e-6, atol=1e-8)
