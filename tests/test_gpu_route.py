"""Router top-k on the GPU against the oracle: ids and counts bit-exact,
weights within 1e-6."""
import numpy as np
import pytest

from oracle import moe as omoe
from synth import make_workload

from .helpers import problem_for

pytestmark = pytest.mark.gpu


def run_route(wl, logits=None, bias=None, k=None):
    import torch
    import expert_moe_fp32_amd as m
    logits = wl.logits if logits is None else logits
    bias = wl.bias if bias is None else bias
    p = problem_for(wl)
    if k is not None:
        p.k = k
    T, E = logits.shape
    p.T, p.E = T, E
    kk = p.k
    dl = torch.from_numpy(np.ascontiguousarray(logits)).cuda()
    db = None if bias is None else torch.from_numpy(bias).cuda()
    ids = torch.full((T * kk,), -7, dtype=torch.int32, device="cuda")
    w = torch.zeros(T * kk, dtype=torch.float32, device="cuda")
    counts = torch.full((E,), 123, dtype=torch.int32, device="cuda")
    m.moe_route_topk(p, dl, db, ids, w, counts)
    torch.cuda.synchronize()
    return (ids.cpu().numpy().reshape(T, kk), w.cpu().numpy().reshape(T, kk),
            counts.cpu().numpy())


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "skewed", "fp8"])
def test_route_full_workloads(name):
    wl = make_workload(name, seed=0)
    print(f"route {wl.describe()}", flush=True)
    ids, w, counts = run_route(wl)
    rids, rw, rcounts = omoe.route_topk(wl.logits, wl.k, wl.bias)
    assert np.array_equal(ids, rids)
    assert np.array_equal(counts, rcounts)
    assert np.max(np.abs(w - rw)) <= 1e-6


def test_route_ties_and_signed_zero():
    wl = make_workload("tiny", seed=1, T=256, E=64, num_local=64, k=6)
    rng = np.random.default_rng(5)
    logits = np.round(rng.standard_normal((256, 64)) * 2).astype(np.float32) / 2
    logits[::7, ::3] = -0.0
    logits[1::7, ::5] = 0.0
    logits[3] = 1.0                        # one row all equal
    ids, w, counts = run_route(wl, logits=logits, bias=None)
    rids, rw, rcounts = omoe.route_topk(logits, 6)
    assert np.array_equal(ids, rids)
    assert np.array_equal(counts, rcounts)
    assert np.max(np.abs(w - rw)) <= 1e-6
    assert ids[3].tolist() == [0, 1, 2, 3, 4, 5]


@pytest.mark.parametrize("E,k", [(8, 8), (100, 3), (512, 16), (1024, 1)])
def test_route_shapes(E, k):
    wl = make_workload("tiny", seed=2, T=333, E=E, num_local=min(E, 8), k=k)
    ids, w, counts = run_route(wl)
    rids, rw, rcounts = omoe.route_topk(wl.logits, k)
    assert np.array_equal(ids, rids)
    assert np.array_equal(counts, rcounts)
    assert np.max(np.abs(w - rw)) <= 1e-6


def test_route_is_deterministic():
    wl = make_workload("prefill", seed=3)
    a = run_route(wl)
    b = run_route(wl)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
