"""The whole layer on the GPU against the oracle, through the C ABI.

Outputs: max|gpu - oracle| beyond the output format's own rounding must stay
within 1e-5 (fp32), 1e-2 (bf16) or 4e-2 (fp8) of the oracle output's RMS.
Reduced shapes span several tiles and ragged tails; full-size workloads are
checked on sampled tokens in the launch configuration the benchmark times."""
import numpy as np
import pytest

from oracle import eplb, moe as omoe
from synth import make_workload

from .helpers import (BARS, check_output, device_layer, out_to_f64,
                      phys_to_logical_from_map, recipe)

pytestmark = pytest.mark.gpu


def run_layer(wl, l2p=None, rep=None, P=None, steps=False):
    import torch
    from expert_moe_fp32_amd.runner import to_dev
    ptl = None if l2p is None else phys_to_logical_from_map(l2p, rep, P)
    dl = device_layer(wl, l2p=l2p, rep=rep, P=P, phys_to_logical=ptl)
    b = dl.buffers()
    dlog = to_dev(wl.logits)
    dbias = None if wl.bias is None else to_dev(wl.bias)
    dx = to_dev(wl.x)
    if steps:
        dl.route(b, dlog, dbias)
        dl.dispatch(b, dx)
        dl.ffn(b, x_shared=dx if wl.shared else None)
        dl.combine(b)
    else:
        dl.forward(b, dlog, dbias, dx)
    torch.cuda.synchronize()
    out = out_to_f64(b, wl)
    counts = b.counts.cpu().numpy()
    del dl, b
    torch.cuda.empty_cache()
    return out, counts


def oracle_out(wl, tokens=None, l2p=None, rep=None, P=None):
    ex = omoe.expert_set_from_workload(wl, lazy=True)
    res = omoe.layer_from_workload(wl, ex, l2p=l2p, rep_count=rep, P=P,
                                   token_subset=tokens)
    return res


def sample_tokens(T, n, seed=0):
    rng = np.random.default_rng(seed)
    s = set(rng.choice(T, size=min(n, T), replace=False).tolist())
    s |= {0, T - 1}
    return np.array(sorted(s))


@pytest.mark.parametrize("name,kw", [
    ("tiny", {}),                                         # fp32, all local
    ("tiny", dict(T=77, E=16, num_local=6, expert_begin=5, k=3)),
    ("prefill", dict(T=300, H=256, I=256, E=16, num_local=8, k=4)),  # tiled
    ("prefill", dict(T=50, H=512, I=256, E=64, num_local=16, k=4)),  # stream
    ("decode", dict(T=64, H=384, I=256, E=32, num_local=8, k=4)),    # stream
    ("decode", dict(T=700, H=256, I=384, E=8, num_local=8, k=2)),    # tiled
    # ring GEMM gate/up, 128 x 128 tiled down (H not a multiple of 256)
    ("prefill", dict(T=400, H=384, I=256, E=8, num_local=8, k=2)),
    # more than 1024 tokens: the multi-block dispatch, whose scan writes the
    # tile list (ring GEMM + 128-row down list; fp32 kernel)
    ("prefill", dict(T=1100, H=384, I=256, E=8, num_local=8, k=2)),
    ("tiny", dict(T=1500, E=16, num_local=8, k=2)),
    # 2048 tokens or more: the combine's streaming (non-temporal) form, here
    # with float32 output
    ("tiny", dict(T=2100, E=16, num_local=8, k=2)),
    # ring GEMM with the shortest reductions it takes (K = 128, one trip of
    # its 4-stage loop: prologue, register prefetch and clamped tail
    # transfers only): down with I = 128, gate/up with H = 128
    ("prefill", dict(T=500, H=256, I=128, E=8, num_local=8, k=2)),
    ("prefill", dict(T=500, H=128, I=256, E=8, num_local=8, k=2)),
])
def test_layer_reduced_shapes(name, kw):
    wl = make_workload(name, seed=11, **kw)
    print(f"layer {wl.describe()}", flush=True)
    out, counts = run_layer(wl)
    ref = oracle_out(wl)
    assert np.array_equal(counts, ref.counts)
    r = check_output(out, ref.out, wl.out, BARS[recipe(wl)], wl.describe())
    print(f"  max|err|/RMS = {r:.3e}")


def test_steps_equal_layer_forward():
    wl = make_workload("prefill", seed=12, T=200, H=256, I=128, E=16,
                       num_local=8, k=4)
    a, _ = run_layer(wl)
    b, _ = run_layer(wl, steps=True)
    assert np.array_equal(a, b)


def test_tokens_without_local_pairs_get_zero_rows():
    wl = make_workload("decode", seed=13, T=40, H=256, I=128, E=64,
                       num_local=4, expert_begin=60, k=2)
    out, _ = run_layer(wl)
    ref = oracle_out(wl)
    none_local = (ref.disp.pair_row < 0).all(axis=1)
    assert none_local.any()
    assert np.all(out[none_local] == 0.0)
    check_output(out, ref.out, wl.out, BARS["bf16"])


def test_full_decode_all_tokens():
    wl = make_workload("decode", seed=0)
    print(f"layer {wl.describe()}", flush=True)
    out, _ = run_layer(wl)
    ref = oracle_out(wl)
    r = check_output(out, ref.out, wl.out, BARS["bf16"], "decode")
    print(f"  max|err|/RMS = {r:.3e}")


@pytest.fixture(scope="module")
def skewed():
    return make_workload("skewed", seed=0)


def test_full_prefill_sampled():
    wl = make_workload("prefill", seed=0)
    print(f"layer {wl.describe()}", flush=True)
    out, _ = run_layer(wl)
    tok = sample_tokens(wl.T, 20)
    ref = oracle_out(wl, tokens=tok)
    r = check_output(out[tok], ref.out[tok], wl.out, BARS["bf16"], "prefill")
    print(f"  max|err|/RMS = {r:.3e}")


def test_full_skewed_with_and_without_replicas(skewed):
    wl = skewed
    print(f"layer {wl.describe()}", flush=True)
    out_a, counts = run_layer(wl)
    local = counts[wl.expert_begin: wl.expert_begin + wl.num_local]
    l2p, rep, P = eplb.hottest_replica_map(local, wl.redundant)
    out_b, _ = run_layer(wl, l2p=l2p, rep=rep, P=P)
    # replicas compute with the same weights in the same order
    assert np.array_equal(out_a, out_b)
    tok = sample_tokens(wl.T, 16, seed=1)
    ref = oracle_out(wl, tokens=tok, l2p=l2p, rep=rep, P=P)
    check_output(out_b[tok], ref.out[tok], wl.out, BARS["bf16"], "skewed")
    base = ref.disp.logical_counts
    print(f"  busiest/mean local expert: a {base.max() / base.mean():.2f}, "
          f"b {ref.disp.phys_counts.max() / ref.disp.phys_counts.mean():.2f}")


def with_hot_expert(wl, e):
    """Every token gets local expert e in its top-k (its logit raised by 20):
    one expert holds all T rows, several tiles of them."""
    logits = wl.logits.copy()
    logits[:, e] += 20.0
    wl._cache["logits"] = logits
    return wl


@pytest.mark.parametrize("name,kw", [
    ("prefill", dict(T=600, H=256, I=256, E=16, num_local=8, k=4)),  # ring GEMM
    ("decode", dict(T=64, H=384, I=256, E=32, num_local=8, k=4)),    # stream
    ("fp8", dict(T=400, H=512, I=1024, E=16, num_local=8, k=4)),     # FP8 ring
])
def test_layer_hot_expert(name, kw):
    wl = with_hot_expert(make_workload(name, seed=17, **kw), 3)
    print(f"layer hot expert 3: {wl.describe()}", flush=True)
    out, counts = run_layer(wl)
    ref = oracle_out(wl)
    assert counts[3] == wl.T
    assert np.array_equal(counts, ref.counts)
    check_output(out, ref.out, wl.out, BARS[recipe(wl)], wl.describe())


@pytest.mark.parametrize("name,kw", [
    ("decode", dict(T=1, H=384, I=256, E=32, num_local=8, k=4)),
    ("prefill", dict(T=1, H=256, I=256, E=16, num_local=8, k=4)),   # + shared
    ("fp8", dict(T=1, H=512, I=512, E=16, num_local=8, k=4)),
])
def test_layer_single_token(name, kw):
    wl = make_workload(name, seed=19, **kw)
    print(f"layer {wl.describe()}", flush=True)
    out, _ = run_layer(wl)
    ref = oracle_out(wl)
    check_output(out, ref.out, wl.out, BARS[recipe(wl)], wl.describe())
