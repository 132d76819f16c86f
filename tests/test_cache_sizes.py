"""Closed-form cache sizes printed on the pages (tests/golden/cache_sizes.json)."""
import json
import os

import pytest

from oracle import cache_cost as cc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "cache_sizes.json")
ITEMS = json.load(open(GOLDEN))["items"]

COMPUTE = {
    "mha_v3_elems_per_token_layer": lambda: cc.kv_elems_per_token_layer(128, 128),
    "mla_elems_per_token_layer": lambda: cc.mla_elems_per_token_layer(512, 64),
    "llama2_7b_bytes_per_token": lambda: cc.kv_bytes_per_token(32, 32, 128, 2),
    "llama2_7b_bytes_8k_sequence": lambda: cc.kv_bytes_per_token(32, 32, 128, 2) * 8192,
    "llama2_7b_bytes_8k_batch16": lambda: cc.kv_bytes_per_token(32, 32, 128, 2) * 8192 * 16,
    "mha_32x128_elems_per_token_layer": lambda: cc.kv_elems_per_token_layer(32, 128),
    "mha_32x128_bytes_per_token_layer_fp16": lambda: cc.kv_elems_per_token_layer(32, 128) * 2,
    "llama3_8b_bytes_per_token": lambda: cc.kv_bytes_per_token(32, 8, 128, 2),
    "llama3_vs_llama2_cache_ratio": lambda: cc.kv_bytes_per_token(32, 32, 128, 2) / cc.kv_bytes_per_token(32, 8, 128, 2),
    "deepseek_v2_bytes_per_token": lambda: cc.mla_bytes_per_token(60, 512, 64, 2),
    "mla_equivalent_gqa_groups": lambda: cc.equivalent_gqa_groups(512, 64, 128),
    "gqla_llama3_8b_mqa_absorb_fraction": lambda: cc.mla_elems_per_token_layer(512, 64) / cc.kv_elems_per_token_layer(8, 128),
}


@pytest.mark.parametrize("item", ITEMS, ids=[i["id"] for i in ITEMS])
def test_page_number(item):
    assert COMPUTE[item["id"]]() == item["value"]


def test_every_golden_item_is_checked():
    assert set(COMPUTE) == {i["id"] for i in ITEMS}


def test_units_as_printed():
    # 512 KB, 4 GB, 64 GB, 16 KB, 128 KB and 67.5 KB with KB = 1024 B as the calculator states.
    assert cc.kv_bytes_per_token(32, 32, 128, 2) / 1024 == 512
    assert cc.kv_bytes_per_token(32, 32, 128, 2) * 8192 / 2 ** 30 == 4
    assert cc.kv_bytes_per_token(32, 8, 128, 2) / 1024 == 128
    assert cc.mla_bytes_per_token(60, 512, 64, 2) / 1024 == 67.5
