"""Pin the closed-form size model (oracle/sizes.py) to the numbers the pages print."""
import json
import os

import pytest

from oracle import sizes as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")
with open(GOLDEN) as f:
    NUMBERS = {n["id"]: n for n in json.load(f)["numbers"]}

DSV2 = S.Model("DeepSeek-V2", 60, S.Layer(128, 128, 128, 512, 64))
SW_MODEL = S.Model("32-head 36-layer", 36, S.Layer(32, 32, 128))


def computed():
    u = S.in_unit
    l8, l70, v3, l2 = S.LLAMA3_8B, S.LLAMA3_70B, S.DEEPSEEK_V3, S.LLAMA2_7B
    dsv2_mha_elems = 2 * 5120
    v3_mha = S.with_kv_heads(v3, v3.layer.q_heads)
    per_layer = lambda m: S.elements_per_token(m.layer)
    return {
        "dsv2_mla_no_rope_elems": S.elements_per_token(S.Layer(128, 128, 128, 512, 0)),
        "dsv2_mla_rope_elems": per_layer(DSV2),
        "dsv2_rope_overhead": DSV2.layer.rope / DSV2.layer.latent,
        "dsv2_mha_elems": dsv2_mha_elems,
        "dsv2_ratio_rope": dsv2_mha_elems / per_layer(DSV2),
        "dsv2_ratio_no_rope": dsv2_mha_elems / 512,
        "dsv2_60layer_mla_bytes_per_token": u(S.cache_bytes(DSV2), "KiB"),
        "dsv2_60layer_mha_bytes_per_token": dsv2_mha_elems * 60 * 2 / 1e6,
        "llama2_7b_mha_elems": per_layer(l2),
        "llama2_7b_gqa8_elems": S.elements_per_token(S.Layer(32, 8, 128)),
        "llama2_7b_mqa_elems": per_layer(S.with_kv_heads(l2, 1)),
        "llama2_7b_mla_elems": S.elements_per_token(S.Layer(32, 32, 128, 512, 0)),
        "upprojection_gflops": S.naive_upprojection_flops(4096, 512, 4096) / 1e9,
        "a6000_head_threshold": S.mla_compute_bound_head_threshold(155e12, 768e9),
        "llama3_8b_mha_bytes_per_token": S.cache_bytes(S.with_kv_heads(l8, 32)),
        "llama3_8b_gqa_bytes_per_token": S.cache_bytes(l8),
        "llama3_70b_gqa_bytes_per_token": S.cache_bytes(l70),
        "llama3_8b_128k_gib": u(S.cache_bytes(l8, 131072), "GiB"),
        "llama3_70b_128k_gib": u(S.cache_bytes(l70, 131072), "GiB"),
        "llama3_8b_mqa_kib_per_token": u(S.cache_bytes(S.with_kv_heads(l8, 1)), "KiB"),
        "dsv3_bytes_per_token": S.cache_bytes(v3),
        "dsv3_kib_per_token": u(S.cache_bytes(v3), "KiB"),
        "dsv3_as_mha_mib_per_token": u(S.cache_bytes(v3_mha), "MiB"),
        "dsv3_mha_ratio": S.cache_bytes(v3_mha) / S.cache_bytes(v3),
        "dsv3_128k_gib": u(S.cache_bytes(v3, 131072), "GiB"),
        "dsv3_61_layer_elems": per_layer(v3) * v3.depth,
        "llama3_8b_all_layer_elems": per_layer(l8) * l8.depth,
        "mla_bytes_per_cached_token": S.row_bytes(v3.layer),
        "mla_flops_per_cached_token": S.row_flops(v3.layer),
        "mla_intensity": S.intensity(v3.layer),
        "gqa_bytes_per_cached_token": S.row_bytes(l8.layer),
        "gqa_flops_per_cached_token": S.row_flops(l8.layer),
        "llama3_8b_intensity": S.intensity(l8.layer),
        "llama3_70b_intensity": S.intensity(l70.layer),
        "mha_intensity": S.intensity(S.with_kv_heads(l8, 32).layer),
        "dsv3_128k_layer_read_mb": S.row_bytes(v3.layer) * 131072 / 1e6,
        "llama3_70b_32k_gib": u(S.cache_bytes(l70, 32768), "GiB"),
        "fp8_llama3_8b_kib": u(S.cache_bytes(l8, elem_bytes=1), "KiB"),
        "fp8_llama3_70b_kib": u(S.cache_bytes(l70, elem_bytes=1), "KiB"),
        "fp8_dsv3_kib": u(S.cache_bytes(v3, elem_bytes=1), "KiB"),
        "mla_mha_read_ratio_s20": S.mla_mha_read_ratio(20),
        "mla_mha_read_ratio_limit": S.mla_mha_read_ratio(10 ** 9),
        "shippingwang_kb_per_token_layer": u(S.row_bytes(SW_MODEL.layer), "KiB"),
        "shippingwang_kb_per_token": u(S.cache_bytes(SW_MODEL), "KiB"),
        "shippingwang_32k_gb": S.cache_bytes(SW_MODEL, 32768) / 1e9,
    }


COMPUTED = computed()


@pytest.mark.parametrize("nid", sorted(NUMBERS))
def test_page_number(nid):
    n = NUMBERS[nid]
    got = COMPUTED[nid]
    want = n["value"]
    if n["tol"] == 0:
        assert got == want, (nid, got, want, n["source"])
    else:
        assert abs(got - want) <= n["tol"] * abs(want), (nid, got, want, n["source"])


def test_every_golden_number_is_checked():
    assert set(NUMBERS) == set(COMPUTED)


def test_mi355x_head_threshold_derived():
    # The same head-count rule with MI355X spec numbers (2.5 PFLOP/s dense bf16,
    # 8 TB/s) puts the threshold above DeepSeek's 128 heads: HBM binds.
    t = S.mla_compute_bound_head_threshold(2.5e15, 8e12)
    assert abs(t - 156.25) < 1e-9 and t > 128


def test_mla_intensity_is_heads_times_dims():
    # 2*n_h*(576+512)/1152 for any n_h: intensity scales with the head count
    for nh in (16, 32, 64, 128):
        assert S.intensity(S.Layer(nh, nh, 128, 512, 64)) == pytest.approx(nh * 2 * 1088 / 1152)


def test_head_sharing_schemes_are_one_formula():
    # MHA, GQA and MQA differ only in the KV head count: elements per token
    # per layer are 2 n_kv d_h, and decode intensity is n_h / n_kv = g
    for n_kv in (1, 2, 4, 8, 32):
        layer = S.Layer(32, n_kv, 128)
        assert S.elements_per_token(layer) == 2 * n_kv * 128
        assert S.intensity(layer) == pytest.approx(32 / n_kv)
