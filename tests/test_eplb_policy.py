"""The library's load-balancing policy (host C++ behind the C ABI) against
the oracle and the printed output of the power-law load simulation of
"6.4 Data parallelism and expert parallelism", section 5.2, plus the slot
count of section 5.3.  CPU only: these entry points are host code."""
import ctypes
import json
import os

import numpy as np
import pytest

import expert_moe_fp32_amd as m
from expert_moe_fp32_amd import _lib as L
from oracle import arith, eplb
from oracle import moe as omoe

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "eplb_simulation.json")))


@pytest.fixture(scope="module")
def counts():
    return eplb.simulate_expert_counts(seed=0, experts=256, top_k=8,
                                       tokens=4096, skew=0.4)


@pytest.mark.parametrize("ep,red", [(8, 0), (8, 8), (32, 0), (32, 32),
                                    (64, 0), (64, 64), (256, 0), (256, 256),
                                    (8, 24)])
def test_plan_matches_oracle(counts, ep, red):
    rep, se, sr, rl = m.moe_eplb_plan(counts, ep, red)
    want_rep = eplb.plan_replicas(counts, red)
    assert rep == want_rep
    held, load = eplb.place_replicas(counts, want_rep, ep)
    for g in range(ep):
        assert list(zip(se[g], sr[g])) == sorted(held[g])
    assert rl == load                    # same doubles, same order of adds


def test_plan_reproduces_printed_table(counts):
    for row in GOLD["rows"]:
        ep = row["ep"]
        for red, col in ((0, "rebalance"), (ep, "redundant")):
            _, _, _, rl = m.moe_eplb_plan(counts, ep, red)
            assert round(eplb.busiest_over_mean(rl), 2) == row[col], (ep, red)


def test_slots_per_rank_closed_form(counts):
    # the page's serving command: 256 experts + 8 redundant over EP = 8
    _, se, _, _ = m.moe_eplb_plan(counts, 8, 8)
    assert all(len(s) == 33 for s in se)
    assert arith.experts_per_card(256, 8, 8) == 33


def test_plan_ties_and_small_cases():
    # equal per-replica loads: the lower expert id gets the redundant slot
    rep, se, sr, rl = m.moe_eplb_plan([5, 5], 1, 1)
    assert rep == [2, 1]
    # highest load per replica, recomputed after every grant
    rep, _, _, _ = m.moe_eplb_plan([10, 30, 20], 3, 3)
    assert rep == [1, 3, 2]
    # zero load everywhere: still one replica each, ranks filled in order
    rep, se, sr, rl = m.moe_eplb_plan([0, 0, 0, 0], 2, 0)
    assert rep == [1, 1, 1, 1] and rl == [0.0, 0.0]
    assert sorted(se[0] + se[1]) == [0, 1, 2, 3]


def test_rank_maps_match_oracle(counts):
    ep, red = 8, 8
    rep, se, sr, _ = m.moe_eplb_plan(counts, ep, red)
    held, _ = eplb.place_replicas(counts, rep, ep)
    for g in range(ep):
        l2p, rc, P = m.moe_eplb_rank_map(rep, se, sr, red, g)
        wl2p, wrc, wP = eplb.rank_map(held, rep, g)
        assert P == wP == 33
        assert np.array_equal(np.asarray(l2p), wl2p)
        assert np.array_equal(np.asarray(rc), wrc)


def test_rank_maps_split_every_pair_once():
    """Under a group-wide placement every (token, expert) pair is local on
    exactly one rank, and a hot expert's pairs split over its replicas."""
    rng = np.random.default_rng(3)
    E, k, T, ep, red = 32, 4, 300, 4, 4
    pop = 1.0 / np.arange(1, E + 1) ** 1.2
    ids = np.stack([rng.choice(E, size=k, replace=False, p=pop / pop.sum())
                    for _ in range(T)]).astype(np.int64)
    load = np.bincount(ids.ravel(), minlength=E)
    rep, se, sr, _ = m.moe_eplb_plan(load.tolist(), ep, red)
    seen = np.zeros((T, k), dtype=np.int64)
    rows = 0
    for g in range(ep):
        l2p, rc, P = m.moe_eplb_rank_map(rep, se, sr, red, g)
        d = omoe.dispatch(ids, 0, E, np.asarray(l2p), np.asarray(rc), P)
        seen += d.pair_row >= 0
        rows += int(d.offsets[-1])
        for p in range(P):               # replica r of e gets ceil((n-r)/R)
            e, r = se[g][p], sr[g][p]
            assert d.phys_counts[p] == eplb.replica_share(int(load[e]), rep[e])[r]
    assert np.all(seen == 1)
    assert rows == T * k


def test_window_load_oracle_pin():
    hist = [[1, 0, 2], [0, 5, 0], [3, 3, 3], [7, 0, 1]]
    assert eplb.window_load(hist, 2).tolist() == [10, 3, 4]
    assert eplb.window_load(hist, 10).tolist() == [11, 8, 6]
    assert eplb.window_load(hist[:1], 3).tolist() == [1, 0, 2]


def test_invalid_arguments():
    lib = L.lib()
    E = 4
    ld = (ctypes.c_int64 * E)(1, 2, 3, 4)
    rep = (ctypes.c_int32 * E)()
    se = (ctypes.c_int32 * 8)()
    sr = (ctypes.c_int32 * 8)()
    rl = (ctypes.c_double * 4)()
    a = lambda x: ctypes.addressof(x)
    # (E + redundant) not divisible by ep
    assert lib.moe_eplb_plan(a(ld), E, 3, 0, a(rep), a(se), a(sr), a(rl)) == \
        L.MOE_ERR_INVALID_ARGUMENT
    assert lib.moe_eplb_plan(None, E, 2, 0, a(rep), a(se), a(sr), a(rl)) == \
        L.MOE_ERR_INVALID_ARGUMENT
    neg = (ctypes.c_int64 * E)(1, -2, 3, 4)
    assert lib.moe_eplb_plan(a(neg), E, 2, 0, a(rep), a(se), a(sr), a(rl)) == \
        L.MOE_ERR_INVALID_ARGUMENT
    assert lib.moe_eplb_plan(a(ld), E, 2, 2, a(rep), a(se), a(sr), a(rl)) == L.MOE_OK
    # max_replicas below a replica count; rank out of range
    l2p = (ctypes.c_int32 * (E * 2))()
    rc = (ctypes.c_int32 * E)()
    P = ctypes.c_int32()
    assert lib.moe_eplb_rank_map(a(rep), a(se), a(sr), E, 2, 2, 0, 1, a(l2p),
                                 a(rc), a(P)) == L.MOE_ERR_INVALID_ARGUMENT
    assert lib.moe_eplb_rank_map(a(rep), a(se), a(sr), E, 2, 2, 2, 2, a(l2p),
                                 a(rc), a(P)) == L.MOE_ERR_INVALID_ARGUMENT
    assert lib.moe_eplb_rank_map(a(rep), a(se), a(sr), E, 2, 2, 1, 2, a(l2p),
                                 a(rc), a(P)) == L.MOE_OK
    assert P.value == 3
    # the window record validates before touching the device
    assert lib.moe_eplb_record_load(None, E, 4, 0, None, None, None) == \
        L.MOE_ERR_INVALID_ARGUMENT
