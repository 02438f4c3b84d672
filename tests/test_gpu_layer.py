"""The whole layer on the GPU against the oracle, through the C ABI.

Outputs: max|gpu - oracle| beyond the output format's own rounding must stay
within 1e-5 (fp32), 1e-2 (bf16) or 4e-2 (fp8) of the oracle output's RMS.
Reduced shapes span several tiles and ragged tails; full-size workloads are
checked on sampled tokens in the launch configuration the benchmark times."""
import numpy as np
import pytest

from oracle import eplb, moe as omoe
from synth import make_workload

from .helpers import (BARS, check_output, device_layer, fp8_complete_check,
                      out_to_f64, phys_to_logical_from_map, recipe,
                      sample_tokens)

pytestmark = pytest.mark.gpu


def run_layer(wl, l2p=None, rep=None, P=None, steps=False, layout="kn"):
    import torch
    from expert_moe_fp32_amd.runner import to_dev
    ptl = None if l2p is None else phys_to_logical_from_map(l2p, rep, P)
    dl = device_layer(wl, l2p=l2p, rep=rep, P=P, phys_to_logical=ptl,
                      layout=layout)
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


def oracle_out(wl, tokens=None, l2p=None, rep=None, P=None, workers=0):
    ex = omoe.expert_set_from_workload(wl, lazy=True)
    res = omoe.layer_from_workload(wl, ex, l2p=l2p, rep_count=rep, P=P,
                                   token_subset=tokens, workers=workers)
    return res


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
    # k = 1; k = E (every expert on every token); the largest k, 16 = E
    ("decode", dict(T=64, H=384, I=256, E=32, num_local=8, k=1)),
    ("tiny", dict(T=200, E=8, num_local=8, k=8)),
    ("tiny", dict(T=300, E=16, num_local=16, k=16)),
])
def test_layer_reduced_shapes(name, kw):
    wl = make_workload(name, seed=11, **kw)
    print(f"layer {wl.describe()}", flush=True)
    out, counts = run_layer(wl)
    ref = oracle_out(wl)
    assert np.array_equal(counts, ref.counts)
    r = check_output(out, ref.out, wl.out, BARS[recipe(wl)], wl.describe())
    print(f"  max|err|/RMS = {r:.3e}")


@pytest.mark.parametrize("name,kw", [
    ("tiny", dict(T=100, E=16, num_local=8, k=2)),                  # fp32
    ("decode", dict(T=64, H=384, I=256, E=32, num_local=8, k=4)),   # stream
    ("prefill", dict(T=300, H=256, I=256, E=16, num_local=8, k=4)),  # ring
])
def test_weights_in_either_storage_order(name, kw):
    """The expert matrices handed over in their logical layout (W_gate,
    W_up [H][I], W_down [I][H]; "6.4 Data parallelism and expert
    parallelism", section 2.1) -- the layout every other test uses -- or
    transposed (output-major) give bit-identical layers, both matching the
    oracle."""
    wl = make_workload(name, seed=14, **kw)
    a, _ = run_layer(wl, layout="kn")
    b, _ = run_layer(wl, layout="nk")
    assert np.array_equal(a, b)
    check_output(a, oracle_out(wl).out, wl.out, BARS[recipe(wl)],
                 wl.describe())


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


@pytest.mark.parametrize("out_fmt", ["bf16", "f32"])
def test_full_decode_all_tokens(out_fmt):
    """The decode workload at full size, every token.  With float32 output
    the bar applies to the raw error (no allowance for any rounding of the
    output); with bf16 output beyond the output's own rounding."""
    wl = make_workload("decode", seed=0, out=out_fmt)
    print(f"layer {wl.describe()}", flush=True)
    out, _ = run_layer(wl)
    ref = oracle_out(wl, workers=16)
    r = check_output(out, ref.out, wl.out, BARS["bf16"], "decode",
                     literal=out_fmt == "f32")
    print(f"  max|err|/RMS = {r:.3e}")


def test_full_decode_skewed_all_tokens():
    """A decode batch with the Zipf logit bias (one local expert holds
    several times the mean rows: its rows run as tall tiles whose four
    quarters share one weight stream), every token, float32 output against
    the raw bar."""
    wl = make_workload("decode_skewed", seed=0, out="f32")
    print(f"layer {wl.describe()}", flush=True)
    out, counts = run_layer(wl)
    local = counts[wl.expert_begin: wl.expert_begin + wl.num_local]
    assert local.max() > 32 and local.max() > 4 * local.mean()
    ref = oracle_out(wl, workers=16)
    assert np.array_equal(counts, ref.counts)
    r = check_output(out, ref.out, wl.out, BARS["bf16"], "decode_skewed",
                     literal=True)
    print(f"  busiest {local.max()} rows, mean {local.mean():.1f}; "
          f"max|err|/RMS = {r:.3e}")


@pytest.fixture(scope="module")
def skewed():
    return make_workload("skewed", seed=0)


@pytest.mark.parametrize("out_fmt", ["bf16", "f32"])
def test_full_prefill_sampled(out_fmt):
    """The prefill workload at full size (T = 8192, shared expert) on 256
    sampled tokens (the oracle evaluates every expert on their rows); with
    float32 output against the raw bar."""
    wl = make_workload("prefill", seed=0, out=out_fmt)
    print(f"layer {wl.describe()}", flush=True)
    out, _ = run_layer(wl)
    tok = sample_tokens(wl.T, 256)
    ref = oracle_out(wl, tokens=tok, workers=16)
    r = check_output(out[tok], ref.out[tok], wl.out, BARS["bf16"], "prefill",
                     literal=out_fmt == "f32")
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
    tok = sample_tokens(wl.T, 256, seed=1)
    ref = oracle_out(wl, tokens=tok, l2p=l2p, rep=rep, P=P, workers=16)
    check_output(out_b[tok], ref.out[tok], wl.out, BARS["bf16"], "skewed")
    base = ref.disp.logical_counts
    print(f"  busiest/mean local expert: a {base.max() / base.mean():.2f}, "
          f"b {ref.disp.phys_counts.max() / ref.disp.phys_counts.mean():.2f}")


@pytest.mark.parametrize("T", [96, 1200])   # streaming kernel; LDS-ring GEMM
def test_rank_shares_sum_to_the_all_local_layer(T):
    """Expert parallelism without a cluster: the layer run for each of 8
    rank shares (8 of 64 experts each, expert_begin = 0, 8, ..., 56; the
    shared expert on share 0 only), float32 outputs summed, equals the layer
    with all 64 experts local, and both match the oracle of the all-local
    layer under the literal bar."""
    kw = dict(T=T, H=256, I=128, E=64, k=4, out="f32")
    total = 0.0
    for s in range(8):
        wl = make_workload("prefill", seed=23, num_local=8, expert_begin=8 * s,
                           shared=s == 0, **kw)
        print(f"share {s}: {wl.describe()}", flush=True)
        out, _ = run_layer(wl)
        total = total + out
    full = make_workload("prefill", seed=23, num_local=64, expert_begin=0,
                         shared=True, **kw)
    print(f"all local: {full.describe()}", flush=True)
    out_full, _ = run_layer(full)
    ref = oracle_out(full)
    rms = float(np.sqrt(np.mean(ref.out ** 2)))
    # the shares differ from the whole only in how float32 partial sums group
    assert np.max(np.abs(total - out_full)) <= 1e-5 * rms
    check_output(total, ref.out, "f32", BARS["bf16"], "sum of shares",
                 literal=True)
    check_output(out_full, ref.out, "f32", BARS["bf16"], "all local",
                 literal=True)


@pytest.mark.parametrize("name,kw", [
    ("decode", dict(T=64, H=384, I=256, E=32, num_local=8, k=4)),      # stream
    ("prefill", dict(T=600, H=256, I=256, E=16, num_local=8, k=4)),    # GEMM
    ("fp8", dict(T=200, H=1024, I=512, E=16, num_local=8, k=4)),       # FP8 ring
])
def test_experts_without_rows_are_not_used(name, kw):
    """Local experts 5, 6 and 7 get no tokens (their logits lowered by 100)
    and NaN weights: an expert with no rows owns no tile, so nothing of it
    reaches the output."""
    wl = make_workload(name, seed=29, **kw)
    logits = wl.logits.copy()
    logits[:, wl.expert_begin + 5: wl.expert_begin + 8] -= 100.0
    wl._cache["logits"] = logits
    for p in (5, 6, 7):
        w = wl.expert(p)
        nan = np.uint16(0x7FC0) if wl.wdt == "bf16" else np.float32("nan")
        wl._experts[p] = {key: np.full_like(v, nan) for key, v in w.items()}
    print(f"layer {wl.describe()} (experts 5-7 empty, NaN weights)", flush=True)
    if wl.wdt == "fp8":
        st = fp8_complete_check(wl)
        assert st["codes"] > 0
        return
    out, counts = run_layer(wl)
    loc = counts[wl.expert_begin: wl.expert_begin + wl.num_local]
    assert np.all(loc[5:8] == 0) and np.all(loc[:5] > 0)
    ref = oracle_out(wl)
    check_output(out, ref.out, wl.out, BARS[recipe(wl)], wl.describe())


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
    assert counts[3] == wl.T
    if wl.wdt == "fp8":           # several h codes can be correct
        fp8_complete_check(wl)
        return
    ref = oracle_out(wl)
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
    if wl.wdt == "fp8":
        fp8_complete_check(wl)
        return
    out, _ = run_layer(wl)
    ref = oracle_out(wl)
    check_output(out, ref.out, wl.out, BARS[recipe(wl)], wl.describe())
