"""The layer captured into a HIP graph (the low-latency decode setting of the
infra-guide page, section 6.1: DeepEP's decode kernels run under graphs).

The library allocates nothing, never synchronises and clears with kernels, so
one moe_layer_forward captures whole.  Each test replays the graph several
times with the program's own eager layer calls (other inputs, other buffers)
and synchronisations in between, and checks every replay bit for bit
against the eager result of the same inputs, and that against the oracle."""
import numpy as np
import pytest

from synth import make_workload

from oracle import moe as omoe

from .helpers import (BARS, check_fp8_complete, check_output, device_layer,
                      out_to_f64, recipe, run_fp8_steps)
from .test_gpu_layer import oracle_out

pytestmark = pytest.mark.gpu


def graph_replays(wl, replays=4):
    import torch
    from expert_moe_fp32_amd.runner import to_dev
    dl = device_layer(wl)
    b, b2 = dl.buffers(), dl.buffers()
    dlog, dx = to_dev(wl.logits), to_dev(wl.x)
    dbias = None if wl.bias is None else to_dev(wl.bias)
    # other inputs for the eager calls between replays
    rng = np.random.default_rng(7)
    dlog2 = to_dev(rng.standard_normal(wl.logits.shape).astype(np.float32))
    dl.forward(b, dlog, dbias, dx)
    torch.cuda.synchronize()
    eager = b.out.clone()
    b.out.fill_(0)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dl.forward(b, dlog, dbias, dx)         # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        dl.forward(b, dlog, dbias, dx)
    torch.cuda.synchronize()
    outs = []
    for r in range(replays):
        b.out.fill_(0)
        graph.replay()
        torch.cuda.synchronize()
        outs.append(b.out.clone())
        dl.forward(b2, dlog2, dbias, dx)       # eager work between replays
        torch.cuda.synchronize()
    out_f64 = out_to_f64(b, wl)
    del graph, dl, b, b2
    torch.cuda.empty_cache()
    return eager, outs, out_f64


def check_against_oracle(wl, out_f64, workers=0):
    """bf16: the output bar; FP8: the complete check on the step-by-step
    calls, whose layer forward must equal the graph's eager output."""
    if wl.wdt != "fp8":
        ref = oracle_out(wl, workers=workers)
        check_output(out_f64, ref.out, wl.out, BARS[recipe(wl)], wl.describe())
        return
    got = run_fp8_steps(wl)
    assert np.array_equal(got["out_layer"], out_f64)
    ref = omoe.layer_from_workload(wl, fp8_detail=True, workers=workers)
    print(f"  {check_fp8_complete(wl, got, ref)}", flush=True)


@pytest.mark.parametrize("name,kw", [
    ("lowlat", dict(H=512, I=256, E=64, num_local=8)),  # FP8, 32-row tiles
    ("decode", dict(T=64, H=384, I=256, E=32, num_local=8, k=4)),  # bf16 stream
    ("prefill", dict(T=300, H=256, I=256, E=16, num_local=8, k=4)),  # ring GEMM
])
def test_graph_replays_match_eager(name, kw):
    wl = make_workload(name, seed=41, **kw)
    print(f"graph {wl.describe()}", flush=True)
    eager, outs, out_f64 = graph_replays(wl)
    for r, o in enumerate(outs):
        assert bool((o == eager).all()), f"replay {r} differs from eager"
    check_against_oracle(wl, out_f64)


def test_graph_lowlat_full_size():
    """The low-latency FP8 decode setting at full size (128 tokens, H = 7168,
    I = 2048, 32 of 256 experts, k = 8), every token."""
    wl = make_workload("lowlat", seed=0)
    print(f"graph {wl.describe()}", flush=True)
    eager, outs, out_f64 = graph_replays(wl, replays=3)
    for r, o in enumerate(outs):
        assert bool((o == eager).all()), f"replay {r} differs from eager"
    check_against_oracle(wl, out_f64, workers=16)
