"""Pin the closed-form size model (oracle/sizes.py) to the numbers the pages print."""
import json
import os

import pytest

from oracle import sizes as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")
with open(GOLDEN) as f:
    NUMBERS = {n["id"]: n for n in json.load(f)["numbers"]}

DSV2 = S.AttnModel("DeepSeek-V2", 60, 128, 128, 128, "mla", 512, 64)
SW_MODEL = S.AttnModel("32-head 36-layer", 36, 32, 32, 128, "mha")


def computed():
    KIB, MIB, GIB = S.KIB, S.MIB, S.GIB
    l8, l70, v3, l2 = S.LLAMA3_8B, S.LLAMA3_70B, S.DEEPSEEK_V3, S.LLAMA2_7B
    dsv2_mha_elems = 2 * 5120
    v3_mha = S.as_type(v3, "mha")
    return {
        "dsv2_mla_no_rope_elems": S.kv_elems_per_token_per_layer(
            S.AttnModel("x", 1, 128, 128, 128, "mla", 512, 0)),
        "dsv2_mla_rope_elems": S.kv_elems_per_token_per_layer(DSV2),
        "dsv2_rope_overhead": DSV2.qk_rope_dim / DSV2.kv_lora_rank,
        "dsv2_mha_elems": dsv2_mha_elems,
        "dsv2_ratio_rope": dsv2_mha_elems / S.kv_elems_per_token_per_layer(DSV2),
        "dsv2_ratio_no_rope": dsv2_mha_elems / 512,
        "dsv2_60layer_mla_bytes_per_token": S.kv_bytes_per_token(DSV2) / KIB,
        "dsv2_60layer_mha_bytes_per_token": dsv2_mha_elems * 60 * 2 / 1e6,
        "llama2_7b_mha_elems": S.kv_elems_per_token_per_layer(l2),
        "llama2_7b_gqa8_elems": S.kv_elems_per_token_per_layer(
            S.AttnModel("l2-gqa8", 32, 32, 8, 128, "gqa")),
        "llama2_7b_mqa_elems": S.kv_elems_per_token_per_layer(S.as_type(l2, "mqa")),
        "llama2_7b_mla_elems": S.kv_elems_per_token_per_layer(
            S.AttnModel("l2-mla", 32, 32, 32, 128, "mla", 512, 0)),
        "upprojection_gflops": S.naive_upprojection_flops(4096, 512, 4096) / 1e9,
        "a6000_head_threshold": S.mla_compute_bound_head_threshold(155e12, 768e9),
        "llama3_8b_mha_bytes_per_token": S.kv_bytes_per_token(S.as_type(l8, "mha")),
        "llama3_8b_gqa_bytes_per_token": S.kv_bytes_per_token(l8),
        "llama3_70b_gqa_bytes_per_token": S.kv_bytes_per_token(l70),
        "llama3_8b_128k_gib": S.kv_bytes(l8, 131072) / GIB,
        "llama3_70b_128k_gib": S.kv_bytes(l70, 131072) / GIB,
        "llama3_8b_mqa_kib_per_token": S.kv_bytes_per_token(S.as_type(l8, "mqa")) / KIB,
        "dsv3_bytes_per_token": S.kv_bytes_per_token(v3),
        "dsv3_kib_per_token": S.kv_bytes_per_token(v3) / KIB,
        "dsv3_as_mha_mib_per_token": S.kv_bytes_per_token(v3_mha) / MIB,
        "dsv3_mha_ratio": S.kv_bytes_per_token(v3_mha) / S.kv_bytes_per_token(v3),
        "dsv3_128k_gib": S.kv_bytes(v3, 131072) / GIB,
        "dsv3_61_layer_elems": S.kv_elems_per_token_per_layer(v3) * v3.layers,
        "llama3_8b_all_layer_elems": S.kv_elems_per_token_per_layer(l8) * l8.layers,
        "mla_bytes_per_cached_token": S.decode_bytes_per_cached_token(v3),
        "mla_flops_per_cached_token": S.decode_flops_per_cached_token(v3),
        "mla_intensity": S.decode_intensity(v3),
        "gqa_bytes_per_cached_token": S.decode_bytes_per_cached_token(l8),
        "gqa_flops_per_cached_token": S.decode_flops_per_cached_token(l8),
        "llama3_8b_intensity": S.decode_intensity(l8),
        "llama3_70b_intensity": S.decode_intensity(l70),
        "mha_intensity": S.decode_intensity(S.as_type(l8, "mha")),
        "dsv3_128k_layer_read_mb": S.decode_bytes_per_cached_token(v3) * 131072 / 1e6,
        "llama3_70b_32k_gib": S.kv_bytes(l70, 32768) / GIB,
        "fp8_llama3_8b_kib": S.kv_bytes_per_token(l8, 1) / KIB,
        "fp8_llama3_70b_kib": S.kv_bytes_per_token(l70, 1) / KIB,
        "fp8_dsv3_kib": S.kv_bytes_per_token(v3, 1) / KIB,
        "mla_mha_read_ratio_s20": S.mla_mha_read_ratio(20),
        "mla_mha_read_ratio_limit": S.mla_mha_read_ratio(10 ** 9),
        "shippingwang_kb_per_token_layer": S.decode_bytes_per_cached_token(SW_MODEL) / KIB,
        "shippingwang_kb_per_token": S.kv_bytes_per_token(SW_MODEL) / KIB,
        "shippingwang_32k_gb": S.kv_bytes(SW_MODEL, 32768) / 1e9,
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
        m = S.AttnModel("x", 1, nh, nh, 128, "mla", 512, 64)
        assert S.decode_intensity(m) == pytest.approx(nh * 2 * 1088 / 1152)
