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


# ------------------------------------------- one rank's map under a plan
HAND = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "eplb_hand.json")))


def test_hand_worked_plan_placement_and_maps():
    """The hand-worked 4-expert, 2-rank, 2-redundant case: plan, placement,
    both ranks' maps and their dispatch of four tokens, all written out."""
    import numpy as np
    from oracle import moe as omoe
    rep = eplb.plan_replicas(HAND["load"], HAND["redundant"])
    assert rep == HAND["replicas"]
    held, load = eplb.place_replicas(HAND["load"], rep, HAND["ep"])
    assert [[list(x) for x in h] for h in held] == HAND["held"]
    assert load == HAND["rank_load"]
    ids = np.asarray(HAND["ids"], dtype=np.int32)
    for g in range(HAND["ep"]):
        l2p, rc, P = eplb.rank_map(held, rep, g)
        assert P == HAND["slots_per_rank"]
        assert l2p.tolist() == HAND["l2p"][g]
        assert rc.tolist() == HAND["replicas"]
        d = omoe.dispatch(ids, 0, 4, l2p, rc, P)
        assert d.offsets.tolist() == HAND["offsets"][g]
        assert d.row_token.tolist() == HAND["row_token"][g]
        assert d.pair_row.tolist() == HAND["pair_row"][g]


@pytest.mark.parametrize("ep,red", [(8, 8), (32, 32), (8, 24)])
def test_rank_maps_of_the_simulated_step(ep, red):
    """Every rank's map from the oracle's own plan of the section 5.2
    simulated step (seed 0; the step whose printed summary the tests above
    pin): each (token, expert) pair is local on exactly one rank, each rank
    holds (E + R) / EP physical experts, and replica r of an expert with n
    pairs and R replicas receives ceil((n - r) / R) rows."""
    import numpy as np
    from oracle import moe as omoe
    picks, counts = eplb.simulate_routing(seed=0, experts=256, top_k=8,
                                          tokens=4096, skew=0.4)
    assert max(counts) == GOLD["hottest"] and min(counts) == GOLD["coldest"]
    ids = np.asarray(picks, dtype=np.int32)
    rep = eplb.plan_replicas(counts, red)
    held, _ = eplb.place_replicas(counts, rep, ep)
    seen = np.zeros(ids.shape, dtype=np.int64)
    rows = 0
    for g in range(ep):
        l2p, rc, P = eplb.rank_map(held, rep, g)
        assert P == arith.experts_per_card(256, red, ep)
        d = omoe.dispatch(ids, 0, 256, l2p, rc, P)
        seen += d.pair_row >= 0
        rows += d.N
        # physical ids follow (expert, replica) order
        slots = sorted(held[g])
        for p, (e, r) in enumerate(slots):
            n, R = counts[e], rep[e]
            assert d.phys_counts[p] == -(-(n - r) // R)
            assert l2p[e, r] == p
    assert np.all(seen == 1)
    assert rows == 4096 * 8
