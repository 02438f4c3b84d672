"""Shared test plumbing: workloads -> C-ABI problems and device layers, and
the output tolerance check."""
from __future__ import annotations

import numpy as np

from oracle import moe as omoe

# Output bars (max |gpu - oracle| as a fraction of the oracle output's RMS),
# applied after allowing the final rounding into the output format (half an
# ulp of that format at the oracle value): bf16 recipe 1e-2, fp8 recipe 4e-2;
# the fp32 recipe 1e-5.
BARS = {"f32": 1e-5, "bf16": 1e-2, "fp8": 4e-2}


def recipe(wl) -> str:
    return "fp8" if wl.wdt == "fp8" else wl.act


def problem_for(wl, num_physical=None, max_replicas=1, T=None):
    import expert_moe_fp32_amd as m
    return m.make_problem(
        T=wl.T if T is None else T, H=wl.H, I=wl.I, E=wl.E, k=wl.k,
        expert_begin=wl.expert_begin, num_local=wl.num_local,
        num_physical=num_physical, max_replicas=max_replicas,
        has_shared=wl.shared, act=wl.act, wdt=wl.wdt, out=wl.out)


def device_layer(wl, l2p=None, rep=None, P=None, phys_to_logical=None,
                 weights=True):
    from expert_moe_fp32_amd.runner import DeviceLayer
    if l2p is not None:
        l2p = np.asarray(l2p, dtype=np.int32)
        max_rep = l2p.shape[1]
        prob = problem_for(wl, num_physical=P, max_replicas=max_rep)
    else:
        prob = problem_for(wl)
    if not weights:
        return DeviceLayer(prob, None, None, l2p=l2p, replica_count=rep)
    experts = [wl.expert(e) for e in range(wl.num_local)]
    return DeviceLayer(prob, experts, wl.shared_expert,
                       phys_to_logical=phys_to_logical, l2p=l2p,
                       replica_count=rep)


def phys_to_logical_from_map(l2p, rep, P):
    out = [-1] * P
    for e in range(len(rep)):
        for r in range(int(rep[e])):
            if int(l2p[e][r]) >= 0:      # -1: replica placed on another rank
                out[int(l2p[e][r])] = e
    return out


def out_to_f64(b, wl) -> np.ndarray:
    t = b.out[: wl.T * wl.H].cpu().numpy()
    if wl.out == "bf16":
        return omoe.bf16_to_f64(t.view(np.uint16)).reshape(wl.T, wl.H)
    return t.astype(np.float64).reshape(wl.T, wl.H)


def check_output(gpu: np.ndarray, ref: np.ndarray, out_fmt: str, bar: float,
                 what: str = ""):
    """max(|gpu - ref| - half_ulp_out(ref)) <= bar * RMS(ref)."""
    rms = float(np.sqrt(np.mean(ref * ref)))
    half = omoe.bf16_half_ulp(ref) if out_fmt == "bf16" else omoe.f32_half_ulp(ref)
    err = np.abs(gpu - ref)
    excess = float(np.max(err - half)) if err.size else 0.0
    raw = float(np.max(err)) if err.size else 0.0
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    assert excess <= bar * rms, (
        f"{what}: max|err| beyond the output rounding = {excess:.3e} > "
        f"{bar} x RMS ({rms:.3e}); raw max|err|/RMS = {raw / rms:.3e}")
    return raw / rms if rms else 0.0
