"""Load-balancing policy of the oracle against the printed output of the
power-law load simulation (6.4 Data parallelism and expert parallelism,
section 5.2) and the redundant-slot count of section 5.3."""
import json
import os

import pytest

from oracle import arith, eplb

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "eplb_simulation.json")))


@pytest.fixture(scope="module")
def counts():
    return eplb.simulate_expert_counts(seed=0, experts=256, top_k=8,
                                       tokens=4096, skew=0.4)


def test_simulated_counts_summary(counts):
    assert max(counts) == GOLD["hottest"]
    assert min(counts) == GOLD["coldest"]
    assert sum(counts) / len(counts) == GOLD["average"]
    assert sum(counts) == 4096 * 8


def test_printed_table(counts):
    rows = eplb.imbalance_table(counts)
    for got, want in zip(rows, GOLD["rows"]):
        ep, per, c, r0, r1 = got
        assert (ep, per) == (want["ep"], want["experts_per_gpu"])
        assert round(c, 2) == want["contiguous"]
        assert round(r0, 2) == want["rebalance"]
        assert round(r1, 2) == want["redundant"]


def test_placement_fills_every_slot(counts):
    for ep, red in [(8, 8), (32, 32), (8, 0)]:
        rep = eplb.plan_replicas(counts, red)
        assert sum(rep) == 256 + red
        held, load = eplb.place_replicas(counts, rep, ep)
        assert all(len(h) == arith.experts_per_card(256, red, ep)
                   for h in held)
        assert sum(load) == pytest.approx(sum(counts))
        # every replica placed exactly once
        flat = sorted(x for h in held for x in h)
        assert flat == sorted((e, r) for e in range(256)
                              for r in range(rep[e]))


def test_replicas_go_to_highest_load_per_replica():
    assert eplb.plan_replicas([10, 30, 20], 3) == [1, 3, 2]
    assert eplb.plan_replicas([5, 5], 1) == [2, 1]


def test_balancedness_both_directions():
    load = [4.0, 2.0, 2.0, 0.0]
    assert eplb.busiest_over_mean(load) == 2.0
    assert eplb.mean_over_busiest(load) == 0.5
