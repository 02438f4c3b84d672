"""Load balancing on the GPU: the sliding-window load record against the
oracle's window sum, and the layer under a group-wide placement (section
5.2 of "6.4 Data parallelism and expert parallelism": an expert's replicas
may sit on different ranks) against the oracle, rank by rank."""
import numpy as np
import pytest

import expert_moe_fp32_amd as m
from oracle import eplb, moe as omoe
from synth import make_workload

from .helpers import BARS, check_output
from .test_gpu_dispatch import check_against_oracle, run_dispatch
from .test_gpu_layer import oracle_out, run_layer

pytestmark = pytest.mark.gpu


def test_record_load_window():
    import torch
    E, window, steps = 256, 7, 23
    print(f"record_load E={E} window={window} steps={steps}", flush=True)
    rng = np.random.default_rng(5)
    hist = torch.zeros((window, E), dtype=torch.int32, device="cuda")
    wsum = torch.zeros(E, dtype=torch.int64, device="cuda")
    seen = []
    for s in range(steps):
        c = rng.integers(0, 5000, size=E).astype(np.int32)
        seen.append(c)
        dc = torch.tensor(c, device="cuda")
        m.moe_eplb_record_load(dc, E, window, s, hist, wsum)
        torch.cuda.synchronize()
        assert np.array_equal(wsum.cpu().numpy(), eplb.window_load(seen, window))


def group_plan(wl, ep, red):
    ids, _, _ = omoe.route_topk(wl.logits, wl.k, wl.bias)
    load = np.bincount(ids.ravel(), minlength=wl.E)
    return m.moe_eplb_plan(load.tolist(), ep, red)


@pytest.mark.parametrize("T", [300, 2500])    # one-workgroup / multi-block
def test_dispatch_group_placement(T):
    wl = make_workload("skewed", seed=21, T=T, H=256, I=128, E=64,
                       num_local=64, k=8, shared=False)
    ep, red = 8, 8
    rep, se, sr, _ = group_plan(wl, ep, red)
    total = 0
    for g in (0, 3, 7):
        l2p, rc, P = m.moe_eplb_rank_map(rep, se, sr, red, g)
        print(f"dispatch T={T} rank {g}: P={P}", flush=True)
        got = run_dispatch(wl, l2p=l2p, rep=rc, P=P)
        check_against_oracle(wl, got, l2p=l2p, rep=rc, P=P)
        total += int(got["offsets"][-1])
    assert total > 0


def test_layer_group_placement_ranks_sum_to_layer():
    """Each rank's output matches the oracle under its map, and the ranks'
    float32 outputs add up to the layer over all experts."""
    wl = make_workload("skewed", seed=22, T=320, H=256, I=256, E=32,
                       num_local=32, k=4, shared=False, out="f32")
    ep, red = 4, 4
    rep, se, sr, _ = group_plan(wl, ep, red)
    total = np.zeros((wl.T, wl.H))
    for g in range(ep):
        l2p, rc, P = m.moe_eplb_rank_map(rep, se, sr, red, g)
        print(f"layer rank {g}: P={P} experts {se[g]}", flush=True)
        out, _ = run_layer(wl, l2p=l2p, rep=rc, P=P)
        ref = oracle_out(wl, l2p=np.asarray(l2p), rep=np.asarray(rc), P=P)
        check_output(out, ref.out, wl.out, BARS["bf16"], f"rank {g}")
        total += out
    full = oracle_out(wl)
    check_output(total, full.out, wl.out, BARS["bf16"], "sum over ranks")
