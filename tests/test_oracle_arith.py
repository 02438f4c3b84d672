"""The oracle's byte arithmetic against the values the pages print."""
import json
import os

import pytest

from oracle import arith as A

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "pages_arithmetic.json")))

GLM = dict(H=6144, I=2048, k=8)
DSV3 = dict(H=7168, I=2048, k=8, layers=58, experts=256)


def computed():
    glm_read = A.expert_read_per_token(8, 6144, 2048, 1.0)
    glm_a2a = A.a2a_bytes_per_token(6144, 2, 8)
    all_layers = A.a2a_bytes_per_token_all_layers(6144, 2, 8, 75)
    nic = A.nic_bytes_per_second(800)
    dsv3_e = A.expert_params(7168, 2048)
    red = A.redundant_expert_bytes(58, 7168, 2048, 1.0)
    return {
        "glm_expert_params": A.expert_params(6144, 2048),
        "glm_expert_fp8_bytes": A.expert_bytes(6144, 2048, 1.0),
        "glm_read_per_token_fp8": glm_read,
        "glm_a2a_bytes": glm_a2a,
        "glm_read_comm_ratio": A.read_to_comm_ratio(glm_read, glm_a2a),
        "glm_a2a_75_layers": all_layers,
        "nvlink_time_us": A.transfer_seconds(all_layers, 1.8e12) * 1e6,
        "nic_time_us": A.transfer_seconds(all_layers, nic) * 1e6,
        "nic_vs_decode_budget_pct":
            100 * A.transfer_seconds(all_layers, nic) / 20e-3,
        "imbalance_2x_idle": A.idle_fraction(2.0),
        "imbalance_2p5x_idle": A.idle_fraction(2.5),
        "imbalance_moe_share": 0.55 * 2.5,
        "imbalance_step_growth": A.step_growth(0.55, 2.5),
        "dsv3_expert_params": dsv3_e,
        "dsv3_routed_params": A.routed_params(58, 256, 7168, 2048),
        "dsv3_routed_share": A.routed_params(58, 256, 7168, 2048) / 671e9,
        "dsv3_card_bytes_ep8": A.per_card_expert_bytes(58, 256, 8, 7168, 2048, 1.0),
        "dsv3_card_bytes_ep32": A.per_card_expert_bytes(58, 256, 32, 7168, 2048, 1.0),
        "dsv3_dispatch_fp8_bytes": A.a2a_bytes_per_token(7168, 1, 8),
        "dsv3_combine_bf16_bytes": A.a2a_bytes_per_token(7168, 2, 8),
        "fp8_dispatch_saving": A.dispatch_combine_saving(8, 7168, 1, 2),
        "experts_per_card_redundant": A.experts_per_card(256, 8, 8),
        "redundant_expert_gb": red,
        "redundant_expert_gib": red / 2**30,
        "redundant_8_gib": 8 * A.redundant_expert_bytes(58, 7168, 2048, 1.0) / 2**30,
    }


@pytest.mark.parametrize("case", GOLD["cases"], ids=lambda c: c["name"])
def test_printed_value(case):
    got = computed()[case["name"]]
    want = case["value"]
    if case["rel"] == 0.0:
        assert got == pytest.approx(want, rel=1e-12, abs=1e-12), case["cite"]
    else:
        assert abs(got - want) <= case["rel"] * abs(want), (got, case["cite"])


def test_exact_integers():
    # the unrounded values behind the printed ones
    assert A.expert_params(6144, 2048) == 37_748_736
    assert A.expert_params(7168, 2048) == 44_040_192
    assert A.a2a_bytes_per_token(6144, 2, 8) == 98_304
    assert A.a2a_bytes_per_token_all_layers(6144, 2, 8, 75) == 14_745_600
    assert A.read_to_comm_ratio(8 * 37_748_736, 98_304) == 3072.0
