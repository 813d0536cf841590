"""Pins of the oracle's FLOP / byte counter against numbers and closed forms the pages print.

The counter (``oracle/flops.py``) sums per-step costs built from index
extents; these tests compare it with the *printed* results of the absorption
note and the izhida answer, so a dropped step, a wrong index or a wrong
convention changes a printed number and fails here.
"""
import itertools
import json
import os
import random
from fractions import Fraction

import pytest

from oracle import flops

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")))


def test_linear_flops_counts_every_operation():
    """§一.1: D multiplies + (D-1) adds per output, +1 add with a bias; counted by brute force."""
    for B, S, D, O in [(1, 1, 1, 1), (2, 3, 4, 5), (1, 2, 7, 3)]:
        ops_nobias = ops_bias = 0
        for _ in range(B * S * O):
            acc_terms = 0
            for _d in range(D):
                ops_nobias += 1  # multiply
                ops_bias += 1
                if acc_terms:
                    ops_nobias += 1  # add into the running sum
                    ops_bias += 1
                acc_terms += 1
            ops_bias += 1  # bias add
        assert flops.linear_flops(B, S, D, O, bias=False) == ops_nobias == B * S * O * (2 * D - 1)
        assert flops.linear_flops(B, S, D, O, bias=True) == ops_bias == 2 * B * S * D * O


def test_chain_order_difference_closed_form():
    """§一.2: order1 - order2 = 2[mn(p-q) + pq(m-n)], and the stated sign rule."""
    rng = random.Random(0)
    for _ in range(200):
        m, n, p, q = (rng.randint(1, 300) for _ in range(4))
        diff = flops.chain_flops(1, m, n, p, q) - flops.chain_flops(2, m, n, p, q)
        assert diff == 2 * (m * n * (p - q) + p * q * (m - n))
        if p < q and m < n:
            assert diff < 0
        if p > q and m > n:
            assert diff > 0


def test_first_absorption_general_difference():
    """§二.4.1: order1 - order2 = 2bhdk(t-s) + 2bhst(d-k)."""
    for b, s, t, h, d, k, q in itertools.product([1, 3], [1, 2, 5], [1, 7, 4096], [1, 128], [8, 128], [16, 512],
                                                 [1536]):
        got = flops.first_absorption_flops(1, b=b, s=s, t=t, h=h, d=d, k=k, q=q) - \
            flops.first_absorption_flops(2, b=b, s=s, t=t, h=h, d=d, k=k, q=q)
        assert got == 2 * b * h * d * k * (t - s) + 2 * b * h * s * t * (d - k)


def test_first_absorption_printed_values():
    """§二.4.1 / §二.4.2 printed numbers at d=128, k=512, h=128, q=1536."""
    g = GOLDEN["first_absorption"]
    dims = dict(d=g["dims"]["d"], k=g["dims"]["k"], h=g["dims"]["h"], q=g["dims"]["q"])
    f = flops.first_absorption_flops
    for s in [1, 2, 17, 4096]:  # prefill: t = s, b = 1
        assert f(1, b=1, s=s, t=s, **dims) - f(2, b=1, s=s, t=s, **dims) == g[
            "order1_minus_order2_prefill_b1_t_eq_s_coeff_s2"] * s * s
    dec = g["order1_minus_order2_decode_b1_s1"]
    unsimp = g["order1_minus_order2_decode_b1_s1_unsimplified"]
    for t in [1, 2, 3, 512, 4096, 131072]:  # decode: s = 1, b = 1
        diff = f(1, b=1, s=1, t=t, **dims) - f(2, b=1, s=1, t=t, **dims)
        assert diff == dec["coeff_t"] * t + dec["const"]
        assert diff == unsimp["coeff_t_minus_1"] * (t - 1) + unsimp["coeff_t"] * t
        # absorbed order is cheaper exactly from t = 2 on
        assert (diff > 0) == (t >= 2)
    o23 = g["order2_minus_order3"]
    o23u = g["order2_minus_order3_unsimplified"]
    for b, s in [(1, 1), (32, 1), (64, 2), (3, 7)]:
        for t in [1, 4096]:
            diff = f(2, b=b, s=s, t=t, **dims) - f(3, b=b, s=s, t=t, **dims)
            assert diff == o23["coeff_bs"] * b * s + o23["const"]
            assert diff == o23u["coeff_bs_minus_512"] * (b * s - 512) + o23u["coeff_bs"] * b * s
            assert diff < 0


def test_second_absorption_values():
    """§三.4.1 general difference and §三.4.2 printed numbers at v=128, k=512, h=128, e=7168."""
    f = flops.second_absorption_flops
    for b, s, t in itertools.product([1, 4], [1, 2], [1, 9, 4096]):
        for h, v, k, e in [(128, 128, 512, 7168), (3, 5, 7, 11)]:
            d12 = f(1, b=b, s=s, t=t, h=h, v=v, k=k, e=e) - f(2, b=b, s=s, t=t, h=h, v=v, k=k, e=e)
            assert d12 == 2 * b * h * v * k * (t - s) + 2 * b * h * s * t * (v - k)
            d23 = f(2, b=b, s=s, t=t, h=h, v=v, k=k, e=e) - f(3, b=b, s=s, t=t, h=h, v=v, k=k, e=e)
            assert d23 == 2 * h * v * k * (b * s - e) + 2 * b * h * s * e * (v - k)
    g = GOLDEN["second_absorption"]
    dims = g["dims"]
    for b, s in [(1, 1), (32, 1), (64, 2)]:
        d23 = f(2, b=b, s=s, t=100, **dims) - f(3, b=b, s=s, t=100, **dims)
        assert d23 == g["order2_minus_order3"]["coeff_bs"] * b * s + g["order2_minus_order3"]["const"]
        u = g["order2_minus_order3_unsimplified"]
        assert d23 == u["coeff_bs_minus_7168"] * (b * s - 7168) + u["coeff_bs"] * b * s
    # §三.4.1: with v = d the second absorption's order1-order2 equals the first's
    a = flops.first_absorption_flops(1, b=1, s=1, t=4096, h=128, d=128, k=512, q=1536) - \
        flops.first_absorption_flops(2, b=1, s=1, t=4096, h=128, d=128, k=512, q=1536)
    c = f(1, b=1, s=1, t=4096, h=128, v=128, k=512, e=7168) - f(2, b=1, s=1, t=4096, h=128, v=128, k=512, e=7168)
    assert a == c


def test_fused_weight_element_counts():
    """§二.4.2: (h,q,k) has 100663296 elements; (q,h,d)+(k,h,d) has 33554432, about 33%."""
    g = GOLDEN["first_absorption"]
    h, q, k, d = 128, 1536, 512, 128
    fused = flops.step_flops("hqk", h=h, q=q, k=k) // 2
    separate = flops.step_flops("qhd", q=q, h=h, d=d) // 2 + flops.step_flops("khd", k=k, h=h, d=d) // 2
    assert fused == g["fused_query_weight_elements"]
    assert separate == g["separate_query_key_weight_elements"]
    assert round(100 * separate / fused) == 33


def test_decode_macs_per_layer():
    """izhida answer "DeepSeek": 128×(512+64+512)×4K = 557056K = 544M MAC per layer, ×60 = 31.875G."""
    g = GOLDEN["decode_macs"]
    macs = flops.decode_attention_macs(heads=g["heads"], kv_lora_rank=g["kv_lora_rank"], rope_dim=g["rope_dim"],
                                       context=g["context"])
    assert macs == g["macs_per_layer_in_K"] * 1024
    assert macs == g["macs_per_layer_in_M"] * 2 ** 20 == 570425344
    assert Fraction(macs * g["layers"], 2 ** 30) == Fraction(g["macs_all_layers_in_G"])
    ratio = flops.mla_to_gqa_cache_ratio(kv_lora_rank=512, rope_dim=64, groups=8, head_dim=128)
    assert ratio == Fraction(*g["mla_over_gqa8_cache"])


def test_projection_weight_elements():
    """izhida answer "DeepSeek", 3rd paragraph: (3+10)·2^25 materialised vs (3+1+1+10)·2^23."""
    g = GOLDEN["weights"]
    dm = g["dims"]
    kw = dict(n_h=dm["n_h"], d_h=dm["d_h"], d_c=dm["d_c"], d_cq=dm["d_cq"], d=dm["d"])
    mat = flops.projection_weight_elements(materialised=True, **kw)
    sep = flops.projection_weight_elements(materialised=False, **kw)
    assert mat == g["materialised"]["multiplier"] * 2 ** g["materialised"]["power_of_two"]
    assert sep == g["not_materialised"]["multiplier"] * 2 ** g["not_materialised"]["power_of_two"]


def test_cache_bytes_per_token():
    """Perplexity post, "Одноузловое против многоузлового": 70,272 B per token (61 layers, bf16)."""
    g = GOLDEN["cache_bytes"]
    assert flops.latent_cache_bytes_per_token(layers=g["layers"], kv_lora_rank=512, rope_dim=64,
                                              elem_bytes=g["elem_bytes"]) == g["bytes_per_token"]


def test_decode_attention_cost_matches_mac_count():
    """The attention call's algorithmic FLOPs are 2 × the izhida MAC count for every visible pair."""
    nb, fl = flops.decode_attn_cost(seq_lens=[4096], q_len=1, heads=128, d_c=512, d_r=64, e=2)
    assert fl == 2 * 570425344
    # cache part of the bytes: 1152 B per cached token per layer = the 70,272 B/token over 61 layers
    assert (70272 // 61) == 1152
    assert nb >= 4096 * 1152
    # causal S=2: query 0 sees L-1 keys, query 1 sees L
    _, fl2 = flops.decode_attn_cost(seq_lens=[100], q_len=2, heads=128, d_c=512, d_r=64, e=2)
    assert fl2 == 2 * 128 * 1088 * (99 + 100)


@pytest.mark.parametrize("order", [1, 2, 3])
def test_step_lists_touch_the_right_shapes(order):
    """Each step's index set is the union of its two operand shapes as §二.1-3 list them."""
    shapes = {"Wuq": "qhd", "cq": "bsq", "Wuk": "khd", "ckv": "btk"}
    first = flops.FIRST_ABSORPTION[order]
    if order == 1:
        assert set(first[0]) == set(shapes["Wuq"]) | set(shapes["cq"])
        assert set(first[1]) == set(shapes["Wuk"]) | set(shapes["ckv"])
    if order == 3:
        assert set(first[0]) == set(shapes["Wuq"]) | set(shapes["Wuk"])
    assert set(first[-1]) >= set("bhst")
