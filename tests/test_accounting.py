"""The cost model behind bench.py's roofline figures (deepseek_mla_latent_amd/accounting.py) against
the oracle's own per-call costs (oracle/flops.py, pinned to the pages in tests/test_flops.py), closed
forms for the fused attention + out-projection call, and brute-force pair counts for draft trees."""
import numpy as np
import pytest

from deepseek_mla_latent_amd import accounting
from oracle import flops
from oracle import mla_decode as ref

H, DC, DR, DH = 128, 512, 64, 128


@pytest.mark.parametrize("lens,S,causal,dt", [([4096] * 32, 1, True, "bf16"), ([1, 63, 64, 65, 700], 1, True, "bf16"),
                                              ([5, 130, 2], 2, True, "f32"), ([5, 130, 2], 2, False, "bf16")])
def test_three_calls_match_the_oracle_costs(lens, S, causal, dt):
    e = 2 if dt == "bf16" else 4
    absorb, attn, out = accounting.path_costs(lens, S, dt, causal=causal)
    T = len(lens) * S
    assert (absorb.bytes, absorb.flops) == flops.absorb_q_cost(tokens=T, heads=H, d_c=DC, d_h=DH, e=e)
    assert (attn.bytes, attn.flops) == flops.decode_attn_cost(seq_lens=lens, q_len=S, heads=H, d_c=DC, d_r=DR, e=e,
                                                              causal=causal)
    assert (out.bytes, out.flops) == flops.out_proj_cost(tokens=T, heads=H, d_c=DC, d_h=DH, e=e)


def test_headline_figures():
    """b32_t4096: 164,126,848 attention bytes, 36.5 GFLOP; the fused call 173,547,648 bytes."""
    absorb, attn, out = accounting.path_costs([4096] * 32, 1, "bf16")
    assert attn.bytes == 164_126_848 and attn.flops == 2 * H * (DC + DR + DC) * 32 * 4096
    _, fused = accounting.path_costs([4096] * 32, 1, "bf16", fused=True)
    assert fused.bytes == 173_547_648


@pytest.mark.parametrize("lens,S", [([4096] * 32, 1), ([3, 70, 129], 2), ([0, 64], 3)])
def test_fused_call_is_attention_reads_plus_the_projection(lens, S):
    """The fused call moves what the attention reads (no o_lat / lse written) plus W_UV and the
    output, and computes both calls' FLOPs."""
    T = len(lens) * S
    _, attn, out = accounting.path_costs(lens, S, "bf16")
    _, fused = accounting.path_costs(lens, S, "bf16", fused=True)
    assert fused.bytes == attn.bytes - T * H * (DC + 1) * 4 + H * DC * DH * 2 + T * H * DH * 2
    assert fused.flops == attn.flops + out.flops


def _tree_pairs_brute(lens, parents):
    pairs = 0
    for L, par in zip(lens, parents):
        anc = ref.tree_ancestors(np.where((par >= -1) & (par < np.arange(len(par))), par, -1))
        for i in range(len(par)):
            pairs += np.asarray(ref.visible_key_index(int(L), len(par), i, True, anc)).size
    return pairs


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tree_pairs_match_the_oracle_visibility(seed):
    """visible_pairs under a draft tree counts exactly the keys the oracle lets each node see,
    including sequences shorter than their tree."""
    rng = np.random.default_rng(seed)
    S = 8
    lens = [int(x) for x in rng.integers(1, 200, size=4)] + [S - 3]
    parents = np.stack([[rng.integers(-1, j) if j else -1 for j in range(S)] for _ in lens]).astype(np.int64)
    assert accounting.visible_pairs(lens, S, tree=parents) == _tree_pairs_brute(lens, parents)
