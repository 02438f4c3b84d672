"""The oracle's expert FFN, combine and whole layer, pinned to a hand-worked
SwiGLU, to invariants of dispatch + combine, and to a dense brute force."""
import json
import math
import os

import numpy as np
import pytest

from oracle import eplb, moe
from synth import make_workload

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_swiglu_hand_worked():
    g = json.load(open(os.path.join(GOLD, "swiglu_hand.json")))
    y = moe.swiglu(np.array(g["x"]), np.array(g["wg"]), np.array(g["wu"]),
                   np.array(g["wd"]), lambda h: h)
    assert np.allclose(y, np.array(g["y_over_ln3"]) * math.log(3.0),
                       rtol=1e-14, atol=1e-14)


def test_silu_odd_part_and_values():
    z = np.linspace(-20, 20, 4001)
    assert np.allclose(moe.silu(z) - moe.silu(-z), z, atol=1e-13)
    assert moe.silu(np.array([0.0]))[0] == 0.0
    assert moe.silu(np.array([math.log(3.0)]))[0] == pytest.approx(
        0.75 * math.log(3.0), rel=1e-15)


def test_bf16_rounding_matches_library():
    import torch
    rng = np.random.default_rng(0)
    v = (rng.standard_normal(100000) * 10).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(moe.round_to_bf16(v.astype(np.float64)), ref)
    # exact midpoints between bf16 neighbours go to the even significand
    assert moe.round_to_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    assert moe.round_to_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6


def test_identity_experts_scale_by_local_weight_sum():
    """dispatch then combine with y = x returns sum_local(w) * x; with every
    expert local that is x itself."""
    rng = np.random.default_rng(3)
    T, E, k, H = 96, 16, 4, 40
    x = rng.standard_normal((T, H))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ids, w, _ = moe.route_topk(logits, k)
    for e0, L in [(0, 16), (4, 8), (12, 4)]:
        l2p, rep = moe.identity_map(L)
        d = moe.dispatch(ids, e0, L, l2p, rep, L)
        y = x[d.row_token]                       # identity experts
        out = moe.combine(y, d.pair_row, w, None, T, H)
        local = (ids >= e0) & (ids < e0 + L)
        scale = (w * local).sum(1)
        assert np.allclose(out, scale[:, None] * x, rtol=1e-13, atol=1e-13)
        if L == E:
            assert np.allclose(out, x, rtol=1e-13, atol=1e-13)


def _tiny(name="tiny", **kw):
    base = dict(T=24, H=32, I=16)
    base.update(kw)
    return make_workload(name, seed=5, **base)


@pytest.mark.parametrize("kw", [
    dict(),                                          # all 8 experts local
    dict(E=16, num_local=4, expert_begin=8, k=3),   # a partial share
    dict(k=8),                                       # k = E
    dict(k=1, E=1, num_local=1),                     # one dense expert
])
def test_sparse_equals_dense_masked_f32(kw):
    wl = _tiny(**kw)
    ex = moe.expert_set_from_workload(wl)
    res = moe.layer_from_workload(wl, ex)
    dense = moe.dense_masked_forward(wl.logits, wl.bias, wl.x, wl.act, wl.k,
                                     wl.expert_begin, wl.num_local, ex)
    assert np.allclose(res.out, dense, rtol=1e-12, atol=1e-12)


def test_sparse_equals_dense_masked_bf16_shared_bias():
    wl = make_workload("skewed", seed=2, T=20, H=48, I=24, E=16, num_local=8,
                       k=3)
    ex = moe.expert_set_from_workload(wl)
    res = moe.layer_from_workload(wl, ex)
    dense = moe.dense_masked_forward(wl.logits, wl.bias, wl.x, wl.act, wl.k,
                                     wl.expert_begin, wl.num_local, ex)
    assert np.allclose(res.out, dense, rtol=1e-12, atol=1e-12)


def test_sparse_equals_dense_masked_fp8():
    wl = make_workload("fp8", seed=4, T=12, H=256, I=128, E=8, num_local=4,
                       k=2)
    ex = moe.expert_set_from_workload(wl)
    res = moe.layer_from_workload(wl, ex)
    dense = moe.dense_masked_forward(wl.logits, wl.bias, wl.x, wl.act, wl.k,
                                     wl.expert_begin, wl.num_local, ex)
    assert np.allclose(res.out, dense, rtol=1e-12, atol=1e-12)


def test_single_expert_k1_is_dense_swiglu():
    wl = _tiny(k=1, E=1, num_local=1)
    ex = moe.expert_set_from_workload(wl)
    res = moe.layer_from_workload(wl, ex)
    assert np.all(res.weights == 1.0)
    wg, wu, wd = ex.experts[0]
    y = moe.swiglu(wl.x.astype(np.float64), wg, wu, wd, moe.round_to_f32)
    assert np.allclose(res.out, y, rtol=1e-14, atol=1e-14)


def test_rank_shares_sum_to_the_whole_layer():
    """Summing the outputs of every EP rank's share (shared expert counted
    once) gives the layer with all experts local: the expert-parallel split
    of 'Expert Parallel and All-to-All Backends' loses nothing."""
    full = make_workload("prefill", seed=1, T=16, H=32, I=16, E=16,
                         num_local=16, k=4)
    ex_full = moe.expert_set_from_workload(full)
    whole = moe.layer_from_workload(full, ex_full).out
    total = np.zeros_like(whole)
    ep = 4
    for r in range(ep):
        L = 16 // ep
        sub = moe.ExpertSet(fmt=ex_full.fmt,
                            experts=ex_full.experts[r * L:(r + 1) * L],
                            shared=ex_full.shared if r == 0 else None)
        res = moe.layer_forward(full.logits, full.bias, full.x, full.act,
                                full.k, r * L, L, sub)
        total += res.out
    assert np.allclose(total, whole, rtol=1e-12, atol=1e-12)


def test_redundant_replicas_do_not_change_the_output():
    wl = make_workload("skewed", seed=3, T=40, H=32, I=16, E=32,
                       num_local=16, k=4)
    ex = moe.expert_set_from_workload(wl)
    a = moe.layer_from_workload(wl, ex)
    l2p, rep, P = eplb.hottest_replica_map(a.disp.logical_counts, 8)
    b = moe.layer_from_workload(wl, ex, l2p=l2p, rep_count=rep, P=P)
    assert P == 24
    assert np.array_equal(a.ids, b.ids)
    assert np.allclose(a.out, b.out, rtol=1e-13, atol=1e-13)
    assert b.disp.phys_counts.max() < a.disp.phys_counts.max()


def test_token_subset_matches_full_evaluation():
    wl = make_workload("prefill", seed=8, T=30, H=32, I=16, E=16,
                       num_local=8, k=4)
    ex = moe.expert_set_from_workload(wl)
    full = moe.layer_from_workload(wl, ex)
    sub = [0, 7, 29]
    part = moe.layer_from_workload(wl, ex, token_subset=sub)
    assert np.array_equal(part.out[sub], full.out[sub])


def test_worker_threads_give_the_same_layer():
    """Experts evaluated on worker threads: the same arithmetic, so the
    same bits, for the plain and the FP8-detail paths."""
    wl = make_workload("prefill", seed=9, T=40, H=64, I=32, E=16,
                       num_local=8, k=4)
    a = moe.layer_from_workload(wl)
    b = moe.layer_from_workload(wl, workers=3)
    assert np.array_equal(a.out, b.out)
    f = make_workload("fp8", seed=9, T=24, H=256, I=128, E=8, num_local=4,
                      k=2)
    a = moe.layer_from_workload(f, fp8_detail=True)
    b = moe.layer_from_workload(f, fp8_detail=True, workers=2)
    assert np.array_equal(a.out, b.out)
    assert np.array_equal(a.out_allow, b.out_allow)
    assert np.array_equal(a.fp8_routed.v_lo, b.fp8_routed.v_lo,
                          equal_nan=True)
