"""Pins for oracle/memory.py against the figures the pages print (tests/golden/page_figures.json)."""
import json
import os

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def test_transformer_cache_65b_matches_86gb():
    f = GOLD["transformer_cache_65b_512k_8bit"]
    a = f["assumed"]
    b = oracle.transformer_kv_cache_bytes(a["n_tokens"], a["n_layers"], a["kv_width"], a["bytes_per_elem"])
    assert round(b / 1e9) == f["value_gb"]


def test_per_token_saving_tends_to_layer_count():
    L = GOLD["per_token_saving_65b"]["assumed"]["n_layers"]
    n = 1 << 30
    ratio = (oracle.transformer_kv_cache_bytes(n, L, 1024, 2)
             / oracle.yoco_kv_cache_bytes(n, L, 1024, 2, window=1024))
    assert abs(ratio - GOLD["per_token_saving_65b"]["value"]) / ratio < 1e-3
    # and with a short context the constant self-decoder caches still show
    assert oracle.yoco_kv_cache_bytes(2048, L, 1024, 2, 1024) > 2 * 2048 * 1024 * 2


def test_tokens_per_gb_ratio_is_layer_count():
    f = GOLD["tokens_per_gb_65b"]
    L = GOLD["per_token_saving_65b"]["assumed"]["n_layers"]
    per_token_yoco = oracle.yoco_kv_cache_bytes(1 << 30, L, 2048, 2, 1024) / (1 << 30)
    per_token_tf = oracle.transformer_kv_cache_bytes(1, L, 2048, 2)
    assert abs((per_token_tf / per_token_yoco) - f["yoco_tokens"] / f["gqa_tokens"]) < 0.1
