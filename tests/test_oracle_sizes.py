"""Pins for the oracle's byte accounting against the numbers the pages print
(tests/golden/page_values.json holds each value with its page and section)."""
import json
import os

import pytest

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))
MiB, GiB = 2 ** 20, 2 ** 30


@pytest.mark.parametrize("c", GOLD["bits_per_weight"], ids=lambda c: f"b{c['bits']}g{c['group']}s{c['scale_bytes']}z{c['zp_bits']}")
def test_bits_per_weight(c):
    g = c["group"]
    bpw = oracle.quant_bytes(g, c["bits"], g, c["scale_bytes"], c["zp_bits"]) * 8 / g
    if "value" in c:
        assert bpw == c["value"]
    else:
        assert abs(bpw - c["value_approx"]) <= c["tol"]


def test_activation_vs_weight_traffic():
    c = GOLD["activation_vs_weight"]
    act = oracle.quant_bytes(c["hidden"], 16, 1e30, 0, 0)   # plain fp16, no scales
    assert act == c["act_bytes_per_token_layer"]
    assert act * c["tokens"] == c["act_bytes_32_tokens"]
    wb = c["weight_n"] * c["weight_k"] * c["weight_bits"] / 8
    assert c["weight_bytes_min"] < wb < c["weight_bytes_max"]
    assert round(wb / (act * c["tokens"])) == c["ratio_approx"]


@pytest.mark.parametrize("c", GOLD["kv_cache"], ids=lambda c: c["what"])
def test_kv_cache_bytes(c):
    b = oracle.kv_bytes(c["layers"], c["kv_heads"], c["head_dim"], c["tokens"], c["bytes_per_elem"])
    if "bytes" in c:
        assert b == c["bytes"]
    else:
        assert abs(b - c["bytes_approx"]) <= c["tol"]


@pytest.mark.parametrize("c", GOLD["kv_quantized"], ids=lambda c: c["what"])
def test_quantized_kv_bytes(c):
    b = oracle.quant_bytes(c["numel"], c["bits"], c["group"], c["scale_bytes"], c["zp_bits"])
    if "bytes" in c:
        assert b == c["bytes"]
    else:
        assert b == c["bytes_approx"]
    if "data_bytes" in c:
        assert oracle.quant_bytes(c["numel"], c["bits"], 1e30, 0, 0) == c["data_bytes"]
        assert b - c["data_bytes"] == c["scale_total_bytes"]
    if "n_groups_approx" in c:
        assert abs(c["numel"] / c["group"] / c["n_groups_approx"] - 1) < 0.01
    # the printed MB totals: 288 MB, 272 MB, 36 MB
    assert b / MiB in (288, 272, 36) or b / GiB == 4.5


def test_moe_weight_budget():
    c = GOLD["moe_weights"]
    total = c["shared_params"] + c["expert_params"] * c["experts"]
    assert abs(total - c["total_params"]) < 1e3
    assert abs(oracle.quant_bytes(total, 16, 1e30, 0, 0) - c["fp16_bytes"]) < 1e3
    experts = oracle.quant_bytes(c["expert_params"] * c["experts"], 4, 1e30, 0, 0)
    shared = oracle.quant_bytes(c["shared_params"], 8, 1e30, 0, 0)
    assert abs(experts - c["experts_int4_bytes"]) < 1e3
    assert abs(shared - c["shared_int8_bytes"]) < 1e3
    assert abs(experts + shared - c["mixed_bytes"]) < 1e3


def test_moe_budget_function_defaults():
    c = GOLD["moe_budget_defaults"]
    shared = c["shared_b"] * c["s_bits"] / 8
    expert = c["expert_b"] * c["resident_experts"] * c["e_bits"] / 8
    kv = oracle.kv_bytes(c["layers"], c["kv_heads"], c["head_dim"], c["seq_len"], c["kv_bits"] / 8) / 1e9
    assert shared == c["shared_gb"] and abs(expert - c["expert_gb"]) < 1e-12
    assert abs(shared + expert + kv + c["workspace_gb"] + c["runtime_gb"] - 12.37) < 0.005
