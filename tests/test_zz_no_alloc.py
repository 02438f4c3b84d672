"""moe_layer_forward_noalloc (the layer for callers that cannot allocate:
its workspace is the library's own per-device scratch) against
moe_layer_forward with a caller's workspace, through the C ABI: two calls in
a row, the second on a smaller batch, bit for bit."""
import numpy as np
import pytest

import expert_moe_fp32_amd as m
from expert_moe_fp32_amd import _lib as L
from synth import make_workload

from .helpers import device_layer, problem_for


def test_too_large_a_problem_is_rejected_before_any_device_work():
    # a prefill batch needs far more than the scratch holds; the call
    # returns WORKSPACE without touching a device
    wl = make_workload("prefill", seed=0)
    p = problem_for(wl)
    assert m.moe_layer_workspace_size(p) > L.NOALLOC_SCRATCH_BYTES
    st = m.moe_layer_forward_noalloc(p, 256, None, 256, L.Weights(), None,
                                     None, 256, None, stream=0, check=False)
    assert st == L.MOE_ERR_WORKSPACE


def _forward_pair(dl, wl, T):
    """The same batch (its first T tokens) through both entry points."""
    import torch
    from expert_moe_fp32_amd.runner import to_dev
    p = problem_for(wl, T=T)
    logits = to_dev(np.ascontiguousarray(wl.logits[:T]))
    x = to_dev(np.ascontiguousarray(wl.x[:T]))
    bias = None if wl.bias is None else to_dev(wl.bias)
    H = wl.H
    out_dt = torch.float32 if wl.out == "f32" else torch.int16
    ws = torch.empty(m.moe_layer_workspace_size(p), dtype=torch.uint8,
                     device="cuda")
    ref = torch.empty(T * H, dtype=out_dt, device="cuda")
    got = torch.full((T * H,), 7, dtype=out_dt, device="cuda")
    c_ref = torch.empty(wl.E, dtype=torch.int32, device="cuda")
    c_got = torch.full((wl.E,), -5, dtype=torch.int32, device="cuda")
    m.moe_layer_forward(p, logits, bias, x, dl.weights, None, None, ref,
                        c_ref, ws, ws.numel())
    torch.cuda.synchronize()
    del ws                                     # nothing else holds scratch
    m.moe_layer_forward_noalloc(p, logits, bias, x, dl.weights, None, None,
                                got, c_got)
    torch.cuda.synchronize()
    assert torch.equal(got, ref), f"T={T}: outputs differ"
    assert torch.equal(c_got, c_ref), f"T={T}: expert counts differ"


@pytest.mark.gpu
@pytest.mark.parametrize("name,T2", [("decode", 100), ("lowlat", 50),
                                     ("tiny", 37)])
def test_noalloc_matches_the_workspace_entry_point(name, T2):
    """Full-size decode (56 MiB of scratch), the FP8 low-latency batch and
    the float32 workload, each followed by a smaller batch on the same
    scratch."""
    import torch
    wl = make_workload(name, seed=3)
    print(f"noalloc {wl.describe()} then T={T2}", flush=True)
    dl = device_layer(wl)
    _forward_pair(dl, wl, wl.T)
    _forward_pair(dl, wl, T2)
    del dl
    torch.cuda.empty_cache()
