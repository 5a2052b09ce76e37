"""Byte accounting of the compressed layout against the figures the
FlashOptim digest prints (tests/golden/flashoptim_figures.json), and the
parameter counts of the synthetic model shapes."""
import json
import os

import pytest

from compressed_adamw_state_amd import workloads as W

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "flashoptim_figures.json")))
GIB = 2.0 ** 30


def per_param(optimizer="adamw"):
    b = W.state_bytes(32 * 1000, optimizer)        # whole groups: exact per-param figure
    return {k: v / (32 * 1000) for k, v in b.items()}


def test_bytes_per_param():
    pp = per_param()
    state = sum(pp.values())
    assert state == 5.125                               # theta' 2 + rho 1 + m 1 + v 1 + 2/16
    assert round(state) == GOLD["flash_adamw_bytes_per_param_grad_release"]["value"]
    assert round(state + 2) == GOLD["flash_adamw_bytes_per_param"]["value"]   # + bf16 grad
    assert 4 + 4 + 4 + 4 == GOLD["adamw_bytes_per_param_standard"]["value"]
    assert 16 * 7 == GOLD["adamw_7b_total_gb"]["value"]
    assert 2 * 7 == GOLD["grad_release_saving_7b_gb"]["value"]
    ck = GOLD["checkpoint_bytes_per_param"]
    assert 4 + 4 + 4 == ck["standard"] and round(state) == ck["flash"]
    assert ck["standard"] * 70 == GOLD["checkpoint_70b_gb"]["standard"]
    assert ck["flash"] * 70 == GOLD["checkpoint_70b_gb"]["flash"]
    # m, v: 8 bytes fp32 -> 1 + 1 + 2 * 2/32 bytes
    comp = (8 - (pp["m_code"] + pp["v_code"] + pp["m_scale"] + pp["v_scale"])) / 8
    assert round(100 * comp) == GOLD["state_quant_compression_pct"]["value"]


def test_llama31_8b_table4():
    tensors = W.WORKLOADS["llama31_8b"].tensors
    n = sum(t.numel for t in tensors)
    assert n == 8_030_261_248 and len(tensors) == 291
    tot = {"theta_bf16": 0, "rho": 0, "m_code": 0, "m_scale": 0, "v_code": 0, "v_scale": 0}
    for t in tensors:
        for k, v in W.state_bytes(t.numel).items():
            tot[k] += v
    g = GOLD["llama31_8b_table4_gib"]
    assert round(4 * n / GIB, 1) == g["params_ref"]
    assert round(tot["theta_bf16"] / GIB, 1) == g["params_flash"]
    assert round(8 * n / GIB, 1) == g["opt_state_ref"]
    flash_state = tot["rho"] + tot["m_code"] + tot["v_code"] + tot["m_scale"] + tot["v_scale"]
    assert round(flash_state / GIB, 1) == g["opt_state_flash"]


@pytest.mark.parametrize("name,count,numel", [
    ("flat1m", 1, 1 << 20),
    ("gpt2_small", 148, 124_439_808),
    ("resnet50", 161, 25_557_032),
    ("llama31_8b", 291, 8_030_261_248),
    ("llama2_13b", 363, 13_015_864_320),
])
def test_workload_shapes(name, count, numel):
    w = W.WORKLOADS[name]
    assert len(w.tensors) == count and w.numel == numel


def test_tail_groups():
    # only ResNet-50's fc.bias (1000 = 31*32 + 8) has a partial group
    tails = {name: [t.name for t in w.tensors if t.numel % 32]
             for name, w in W.WORKLOADS.items()}
    assert tails["resnet50"] == ["fc.bias"]
    assert all(not v for k, v in tails.items() if k != "resnet50")
