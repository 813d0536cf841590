"""Pins of the tree-masked verify in the fp64 oracle.

* the ancestor matrix of a hand-drawn tree, written out by hand; parents outside [-1, j) raise;
* a chain tree (parent j - 1) gives exactly the causal result;
* every node equals a plain single-query decode over the committed keys followed by its own
  root-to-node path, gathered into a fresh contiguous cache (brute force, another route);
* the cache row of a non-ancestor does not change a node's output; an ancestor's row does;
* torch's scaled_dot_product_attention with the hand-written mask of the hand-drawn tree
  (identity up-projections reduce the method to MQA);
* the absorbed route agrees with the non-absorbed one under the tree mask;
* a planted mistake (ancestors without the node itself, or descendants instead of ancestors)
  fails the brute-force pin.
"""
import math

import numpy as np
import pytest
import torch

from oracle import mla_decode as ref
from tests.test_oracle import _tiny

# hand-drawn tree of 6 nodes: 0 <- 1 <- 3, 0 <- 2, and a second root 4 <- 5
PARENTS = [-1, 0, 0, 1, -1, 4]
ANCESTORS = np.array([  # row i: nodes node i sees (itself and its ancestors)
    [1, 0, 0, 0, 0, 0],
    [1, 1, 0, 0, 0, 0],
    [1, 0, 1, 0, 0, 0],
    [1, 1, 0, 1, 0, 0],
    [0, 0, 0, 0, 1, 0],
    [0, 0, 0, 0, 1, 1],
], dtype=bool)


def test_ancestor_matrix_by_hand():
    np.testing.assert_array_equal(ref.tree_ancestors(PARENTS), ANCESTORS)
    np.testing.assert_array_equal(ref.tree_ancestors([-1, -1, -1]), np.eye(3, dtype=bool))
    for bad in ([0], [-1, 1], [-1, 2, 0], [-2]):
        with pytest.raises(ValueError):
            ref.tree_ancestors(bad)


def _case(seed, S, lens, **kw):
    return _tiny(seed=seed, B=len(lens), S=S, lens=lens, **kw)


def _run(t, scale, tree=None, causal=True):
    return ref.mla_decode_nonabsorbed(t["q_nope"], t["q_pe"], t["w_uk"], t["w_uv"], t["pool"], t["block_table"],
                                      t["seq_lens"], softmax_scale=scale, page_size=t["page"], causal=causal,
                                      tree=tree)


def test_chain_tree_is_causal():
    S = 5
    t = _case(11, S, (9, 23))
    chain = np.tile(np.arange(-1, S - 1), (2, 1))
    a, b = _run(t, 0.4, tree=chain), _run(t, 0.4, causal=True)
    for key in ("o_lat", "lse", "out"):
        np.testing.assert_array_equal(a[key], b[key])


def _path_decode(t, b, i, parents, scale):
    """Node i of sequence b as a single-query decode over [committed keys | its root-to-node path]."""
    L, S, page = int(t["seq_lens"][b]), len(parents), t["page"]
    rows = ref.gather_rows(t["pool"], t["block_table"][b], L, page)
    path = []
    j = i
    while j >= 0:
        path.append(j)
        j = parents[j]
    keys = np.concatenate([rows[:L - S], rows[[L - S + j for j in sorted(path)]]])
    n = keys.shape[0]
    npg = -(-n // page)
    pool = np.zeros((npg, page, keys.shape[1]))
    pool.reshape(-1, keys.shape[1])[:n] = keys
    one = ref.mla_decode_nonabsorbed(t["q_nope"][b:b + 1, i:i + 1], t["q_pe"][b:b + 1, i:i + 1], t["w_uk"],
                                     t["w_uv"], pool, np.arange(npg, dtype=np.int32)[None], np.array([n]),
                                     softmax_scale=scale, page_size=page, causal=False)
    return {k: v[0, 0] for k, v in one.items()}


def _check_paths(t, tree, scale):
    r = _run(t, scale, tree=tree)
    for b in range(tree.shape[0]):
        for i in range(tree.shape[1]):
            want = _path_decode(t, b, i, list(tree[b]), scale)
            for key in ("o_lat", "lse", "out"):
                np.testing.assert_allclose(r[key][b, i], want[key], rtol=1e-12, atol=1e-13)


def test_each_node_is_a_decode_over_its_path():
    tree = np.array([PARENTS, [-1, 0, 1, 2, 1, 1]])
    t = _case(12, 6, (17, 6))  # the second sequence has no committed key at all
    _check_paths(t, tree, 0.45)


def test_non_ancestor_rows_do_not_matter():
    S, L = 6, 14
    t = _case(13, S, (L,))
    tree = np.array([PARENTS])
    base = _run(t, 0.5, tree=tree)
    i = 3  # ancestors 0, 1, 3; non-ancestors 2, 4, 5
    for j, matters in ((2, False), (4, False), (5, False), (0, True), (1, True), (3, True)):
        pos = L - S + j
        t2 = dict(t)
        t2["pool"] = t["pool"].copy()
        t2["pool"][t["block_table"][0, pos // t["page"]], pos % t["page"]] += 3.0
        r = _run(t2, 0.5, tree=tree)
        same = all(np.array_equal(r[k][0, i], base[k][0, i]) for k in ("o_lat", "lse", "out"))
        assert same != matters, (j, matters)


def test_identity_weights_reduce_to_sdpa_with_the_hand_written_mask():
    rng = np.random.default_rng(14)
    S, L, H, Dc, Dr, Dh, page = 6, 11, 3, 16, 4, 8, 4
    npg = -(-L // page)
    pool = rng.standard_normal((npg, page, Dc + Dr))
    bt = np.arange(npg, dtype=np.int32)[None]
    q_nope, q_pe = rng.standard_normal((1, S, H, Dh)), rng.standard_normal((1, S, H, Dr))
    eye = np.zeros((H, Dc, Dh))
    eye[:, np.arange(Dh), np.arange(Dh)] = 1.0
    scale = 1 / math.sqrt(Dh + Dr)
    r = ref.mla_decode_nonabsorbed(q_nope, q_pe, eye, eye, pool, bt, np.array([L]), softmax_scale=scale,
                                   page_size=page, tree=np.array([PARENTS]))
    rows = pool.reshape(-1, Dc + Dr)[:L]
    q = torch.from_numpy(np.concatenate([q_nope[0], q_pe[0]], -1)).permute(1, 0, 2)  # (H,S,Dh+Dr)
    k = torch.from_numpy(np.concatenate([rows[:, :Dh], rows[:, Dc:]], -1)).expand(H, L, Dh + Dr).contiguous()
    v = torch.from_numpy(rows[:, :Dh].copy()).expand(H, L, Dh).contiguous()
    mask = torch.zeros(S, L, dtype=torch.bool)
    mask[:, :L - S] = True
    mask[:, L - S:] = torch.from_numpy(ANCESTORS)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)  # default scale 1/sqrt(Dh+Dr)
    np.testing.assert_allclose(r["out"][0], o.permute(1, 0, 2).numpy(), rtol=1e-11, atol=1e-12)


def test_absorbed_equals_nonabsorbed_under_a_tree():
    tree = np.array([PARENTS, [-1, -1, 1, 2, 0, 4]])
    t = _case(15, 6, (21, 9))
    r = _run(t, 0.35, tree=tree)
    q_lat = ref.absorb_q_reference(t["q_nope"], t["w_uk"])
    att = ref.latent_attention_reference(q_lat, t["q_pe"], t["pool"], t["block_table"], t["seq_lens"],
                                         softmax_scale=0.35, page_size=t["page"], tree=tree)
    np.testing.assert_allclose(att["o_lat"], r["o_lat"], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(att["lse"], r["lse"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ref.out_proj_reference(att["o_lat"], t["w_uv"]), r["out"], rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("mistake", ["no_self", "descendants"])
def test_planted_mistakes_are_caught(monkeypatch, mistake):
    good = ref.tree_ancestors
    if mistake == "no_self":
        monkeypatch.setattr(ref, "tree_ancestors", lambda p: good(p) & ~np.eye(len(p), dtype=bool))
    else:
        monkeypatch.setattr(ref, "tree_ancestors", lambda p: good(p).T)
    t = _case(16, 6, (15,))
    with pytest.raises(AssertionError):
        _check_paths(t, np.array([PARENTS]), 0.5)
