"""Routing of the oracle: top-k selection, gate weights and expert counts
(6.4 Data parallelism and expert parallelism, section 3.1, step 1)."""
import math

import numpy as np
import pytest
from scipy.special import softmax

from oracle import moe


def select_by_scanning(row, k):
    """Brute force: k passes over the scores, first maximum wins."""
    taken = []
    for _ in range(k):
        best = None
        for e, v in enumerate(row):
            if e in taken:
                continue
            if best is None or v > row[best]:
                best = e
        taken.append(best)
    return taken


def test_closed_form_example():
    # scores ln1..ln4: the two largest are experts 3 and 2, weights 4/7, 3/7
    logits = np.log(np.array([[1.0, 2.0, 3.0, 4.0]])).astype(np.float32)
    ids, w, counts = moe.route_topk(logits, 2)
    assert ids.tolist() == [[3, 2]]
    e = np.exp(logits[0, [3, 2]].astype(np.float64))
    assert w[0] == pytest.approx([4 / 7, 3 / 7], rel=1e-6)
    assert w[0] == pytest.approx(e / e.sum(), rel=1e-15)
    assert counts.tolist() == [0, 0, 1, 1]


@pytest.mark.parametrize("T,E,k", [(64, 8, 2), (40, 256, 8), (16, 5, 5)])
def test_selection_equals_brute_force(T, E, k):
    rng = np.random.default_rng(T * E + k)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    # quantise a share of the rows so exact ties are common
    logits[::3] = np.round(logits[::3] * 2) / 2
    ids, w, counts = moe.route_topk(logits, k)
    for t in range(T):
        assert ids[t].tolist() == select_by_scanning(logits[t].tolist(), k)
    assert counts.sum() == T * k
    assert np.array_equal(counts, np.bincount(ids.ravel(), minlength=E))


def test_ties_and_signed_zero():
    logits = np.array([[0.5, 1.0, 1.0, 0.5],
                       [-0.0, 0.0, -1.0, -0.0],
                       [0.0, -0.0, 0.0, -2.0]], dtype=np.float32)
    ids, w, _ = moe.route_topk(logits, 3)
    assert ids.tolist() == [[1, 2, 0], [0, 1, 3], [0, 1, 2]]
    assert w[1] == pytest.approx([1 / 3] * 3, rel=1e-15)


def test_weights_sum_to_one_and_decrease():
    rng = np.random.default_rng(1)
    logits = rng.standard_normal((500, 64)).astype(np.float32) * 3
    _, w, _ = moe.route_topk(logits, 6)
    assert np.allclose(w.sum(1), 1.0, atol=1e-14)
    assert np.all(np.diff(w, axis=1) <= 0)


def test_k_equals_E_is_plain_softmax():
    rng = np.random.default_rng(2)
    logits = rng.standard_normal((20, 7)).astype(np.float32)
    ids, w, _ = moe.route_topk(logits, 7)
    sm = softmax(logits.astype(np.float64), axis=1)
    assert np.allclose(np.take_along_axis(sm, ids, 1), w, rtol=1e-13)


def test_bias_enters_scores_in_float32():
    logits = np.array([[1.0, 1.0, 0.9]], dtype=np.float32)
    bias = np.array([0.0, -0.05, 0.2], dtype=np.float32)
    ids, w, _ = moe.route_topk(logits, 2, bias)
    assert ids.tolist() == [[2, 0]]
    s = (logits + bias).astype(np.float32)[0].astype(np.float64)
    assert w[0, 0] == pytest.approx(1 / (1 + math.exp(s[0] - s[2])), rel=1e-14)


def test_bias_normalisation_constant_is_irrelevant():
    rng = np.random.default_rng(4)
    logits = rng.standard_normal((64, 32)).astype(np.float32)
    rank = rng.permutation(32)
    b1 = (-1.2 * np.log(rank + 1.0)).astype(np.float32)
    # the Zipf constant shifts every score by the same amount
    b2 = (b1.astype(np.float64) - 3.0).astype(np.float32)
    i1, w1, _ = moe.route_topk(logits, 4, b1)
    i2, w2, _ = moe.route_topk(logits, 4, b2)
    # float32 rounding of the shifted scores may break exact ties differently;
    # with continuous logits there are none
    assert np.array_equal(i1, i2)
    assert np.allclose(w1, w2, atol=1e-6)
