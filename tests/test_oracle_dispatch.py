"""Local share, replica remap and expert-contiguous permutation of the oracle
(dispatch of 6.4 Data parallelism and expert parallelism, section 3.1, step 2;
replicas of section 5.3)."""
import numpy as np
import pytest

from oracle import eplb, moe


def test_hand_example():
    # 4 tokens, top-2 over 4 experts, rank owns experts [1, 3)
    ids = np.array([[1, 0], [2, 1], [3, 2], [1, 2]])
    l2p, rep = moe.identity_map(2)
    d = moe.dispatch(ids, 1, 2, l2p, rep, 2)
    # expert 1 (local 0): pairs (0,0), (1,1), (3,0); expert 2: (1,0), (2,1), (3,1)
    assert d.offsets.tolist() == [0, 3, 6]
    assert d.row_token.tolist() == [0, 1, 3, 1, 2, 3]
    assert d.row_slot.tolist() == [0, 1, 0, 0, 1, 1]
    assert d.pair_row.tolist() == [[0, -1], [3, 1], [-1, 4], [2, 5]]


def test_hand_example_with_replicas():
    # one local expert with two replicas: pairs alternate, round robin
    ids = np.array([[0], [0], [0], [0], [0]])
    l2p = np.array([[1, 0]])
    rep = np.array([2])
    d = moe.dispatch(ids, 0, 1, l2p, rep, 2)
    # n = 0,2,4 -> physical 1 (positions 0,1,2); n = 1,3 -> physical 0
    assert d.offsets.tolist() == [0, 2, 5]
    assert d.row_token.tolist() == [1, 3, 0, 2, 4]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_permutation_invariants(seed):
    rng = np.random.default_rng(seed)
    T, E, k, e0, L = 300, 64, 6, 16, 16
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ids, _, counts = moe.route_topk(logits, k)
    l2p, rep = moe.identity_map(L)
    d = moe.dispatch(ids, e0, L, l2p, rep, L)
    local = (ids >= e0) & (ids < e0 + L)
    assert d.N == local.sum()
    assert np.array_equal(d.phys_counts, counts[e0:e0 + L])
    # bijection between local pairs and rows
    rows = d.pair_row[local]
    assert sorted(rows.tolist()) == list(range(d.N))
    assert np.all(d.pair_row[~local] == -1)
    for r in range(d.N):
        t, j = d.row_token[r], d.row_slot[r]
        assert d.pair_row[t, j] == r
    # segments hold their expert's tokens in increasing token order
    for p in range(L):
        seg = d.row_token[d.offsets[p]:d.offsets[p + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all(ids[seg, d.row_slot[d.offsets[p]:d.offsets[p + 1]]]
                      == e0 + p)


def test_replica_counts_match_closed_form():
    rng = np.random.default_rng(9)
    T, E, k, L = 500, 32, 4, 32
    bias = (-1.2 * np.log(rng.permutation(E) + 1.0)).astype(np.float32)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ids, _, counts = moe.route_topk(logits, k, bias)
    l2p, rep, P = eplb.hottest_replica_map(counts[:L], 8)
    assert P == 40
    d = moe.dispatch(ids, 0, L, l2p, rep, P)
    for e in range(L):
        shares = eplb.replica_share(int(counts[e]), int(rep[e]))
        for r in range(rep[e]):
            assert d.phys_counts[l2p[e, r]] == shares[r]
    assert d.phys_counts.sum() == counts[:L].sum()
    # brute force of the round robin: list the expert's tokens in order
    for e in range(L):
        toks = [t for t in range(T) if e in ids[t]]
        for r in range(rep[e]):
            p = l2p[e, r]
            seg = d.row_token[d.offsets[p]:d.offsets[p + 1]].tolist()
            assert seg == toks[r::rep[e]]


def test_hottest_map_picks_by_count_then_id():
    l2p, rep, P = eplb.hottest_replica_map([5, 9, 9, 1, 7], 3)
    assert P == 8
    assert l2p[:, 1].tolist() == [-1, 5, 6, -1, 7]
    assert rep.tolist() == [1, 2, 2, 1, 2]
