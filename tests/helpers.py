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
                 weights=True, layout="kn"):
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
    shared = wl.shared_expert
    if layout == "nk":                       # the transposed storage order
        tr = lambda d: {k: np.ascontiguousarray(v.T) for k, v in d.items()}
        experts = [tr(d) for d in experts]
        shared = None if shared is None else tr(shared)
    return DeviceLayer(prob, experts, shared,
                       phys_to_logical=phys_to_logical, l2p=l2p,
                       replica_count=rep, layout=layout)


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
                 what: str = "", literal: bool = False):
    """max(|gpu - ref| - half_ulp_out(ref)) <= bar * RMS(ref); with
    ``literal`` the bar applies to max|gpu - ref| itself (no allowance for
    the output's own rounding)."""
    rms = float(np.sqrt(np.mean(ref * ref)))
    half = omoe.bf16_half_ulp(ref) if out_fmt == "bf16" else omoe.f32_half_ulp(ref)
    err = np.abs(gpu - ref)
    excess = float(np.max(err - half)) if err.size else 0.0
    raw = float(np.max(err)) if err.size else 0.0
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    if literal:
        assert raw <= bar * rms, (
            f"{what}: max|err| = {raw:.3e} > {bar} x RMS ({rms:.3e})")
    assert excess <= bar * rms, (
        f"{what}: max|err| beyond the output rounding = {excess:.3e} > "
        f"{bar} x RMS ({rms:.3e}); raw max|err|/RMS = {raw / rms:.3e}")
    return raw / rms if rms else 0.0


# -------------------------------------------------- FP8: the complete check
def run_fp8_steps(wl, layout="kn"):
    """Route, dispatch, grouped FFN and combine through the C ABI one step at
    a time, and read back what the checks need: the dispatch index, the h
    codes and scales left in the FFN workspace (moe_ffn_intermediate), the
    output, and the layer forward's output on the same inputs."""
    import torch
    import expert_moe_fp32_amd as m
    from expert_moe_fp32_amd.runner import to_dev
    dl = device_layer(wl, layout=layout)
    b = dl.buffers()
    dlog, dx = to_dev(wl.logits), to_dev(wl.x)
    dbias = None if wl.bias is None else to_dev(wl.bias)
    dl.route(b, dlog, dbias)
    dl.dispatch(b, dx)
    xs = xs_sc = None
    if wl.shared:
        # the shared expert's rows: every token's codes and scales, which is
        # the dispatch of an all-local identity share; take them from a
        # second dispatch whose share holds every expert
        xs, xs_sc = shared_fp8_rows(wl, dl, b, dx)
    dl.ffn(b, x_shared=xs, x_shared_scales=xs_sc)
    dl.combine(b)
    torch.cuda.synchronize()
    p = dl.p
    P, T, I = p.num_physical, wl.T, wl.I
    cap = T * min(wl.k, wl.num_local)
    off = b.offsets.cpu().numpy()[: P + 1]
    N = int(off[-1])
    h_ptr, hs_ptr = m.moe_ffn_intermediate(p, b.ws_ffn, b.ws_ffn.numel())
    base = b.ws_ffn.data_ptr()
    rows = cap + (T if wl.shared else 0)
    ws = b.ws_ffn.cpu().numpy()
    h = ws[h_ptr - base: h_ptr - base + rows * I].reshape(rows, I)
    hs = ws[hs_ptr - base: hs_ptr - base + rows * (I // 128) * 4].view(
        np.float32).reshape(rows, I // 128)
    got = dict(offsets=off, row_token=b.row_token.cpu().numpy()[:N],
               h=h.copy(), h_scales=hs.copy(), cap=cap,
               y_perm=b.y_perm.cpu().numpy()[: N * wl.H].reshape(N, wl.H),
               out=out_to_f64(b, wl))
    # the layer forward on the same inputs and weights
    b2 = dl.buffers()
    dl.forward(b2, dlog, dbias, dx)
    torch.cuda.synchronize()
    got["out_layer"] = out_to_f64(b2, wl)
    del dl, b, b2
    torch.cuda.empty_cache()
    return got


def shared_fp8_rows(wl, dl, b, dx):
    """Per-token E4M3 codes and scales of every token row (the shared
    expert's input), from the library's own quantiser inside a dispatch of a
    share that owns all experts with k = 1 (every token is local once, in
    token order)."""
    import torch
    import expert_moe_fp32_amd as m
    T, H = wl.T, wl.H
    pa = m.make_problem(T=T, H=H, I=wl.I, E=1, k=1, num_local=1,
                        act=wl.act, wdt=wl.wdt, out=wl.out)
    ids = torch.zeros(T, dtype=torch.int32, device="cuda")
    w = torch.ones(T, dtype=torch.float32, device="cuda")
    xq = torch.empty(T * H, dtype=torch.uint8, device="cuda")
    xs = torch.empty(T * (H // 128), dtype=torch.float32, device="cuda")
    off = torch.empty(2, dtype=torch.int32, device="cuda")
    rt = torch.empty(T, dtype=torch.int32, device="cuda")
    rw = torch.empty(T, dtype=torch.float32, device="cuda")
    pr = torch.empty(T, dtype=torch.int32, device="cuda")
    ws = torch.empty(m.moe_dispatch_workspace_size(pa), dtype=torch.uint8,
                     device="cuda")
    m.moe_dispatch(pa, dx, ids, w, None, None, xq, xs, off, rt, rw, pr, ws,
                   ws.numel())
    return xq, xs


def check_fp8_complete(wl, got, ref, tokens=None, bar=4e-2):
    """The complete FP8 check (several h codes can be correct):
    * every h code and scale the GPU produced for an evaluated row lies in
      the interval a correct float32 evaluation may give (the oracle's
      Fp8Rows: exact where no rounding boundary is within the bound, one of
      two neighbouring codes where one is);
    * the output is within the oracle's output plus the allowance those
      alternative codes give, plus the output format's rounding, plus
      bar x RMS.
    Returns a dict of the figures."""
    from oracle import fp8 as ofp8
    T = wl.T
    want = np.ones(T, dtype=bool) if tokens is None else np.isin(
        np.arange(T), tokens)
    d = ref.disp
    assert np.array_equal(got["offsets"], d.offsets)
    assert np.array_equal(got["row_token"], d.row_token)
    rows = np.flatnonzero(want[d.row_token])
    stats = dict(codes=0, ambiguous=0, differ=0)

    def check_rows(gh, ghs, det, what):
        s_ok = (det.s_lo <= ghs) & (ghs <= det.s_hi)
        assert s_ok.all(), f"{what}: {np.count_nonzero(~s_ok)} scales outside"
        v = ofp8.e4m3_decode(gh)
        v_ok = (det.v_lo <= v) & (v <= det.v_hi)
        assert v_ok.all(), (
            f"{what}: {np.count_nonzero(~v_ok)} h codes outside the codes a "
            f"float32 evaluation may give")
        own = ofp8.e4m3_decode(ofp8.quantize_rows(
            det.h.astype(np.float32), 128)[0])
        stats["codes"] += v.size
        stats["ambiguous"] += int(np.count_nonzero(det.v_lo != det.v_hi))
        stats["differ"] += int(np.count_nonzero(v != own))

    if rows.size:
        check_rows(got["h"][rows], got["h_scales"][rows],
                   _take_rows(ref.fp8_routed, rows), "routed rows")
    if wl.shared:
        st = np.flatnonzero(want)
        check_rows(got["h"][got["cap"] + st], got["h_scales"][got["cap"] + st],
                   ref.fp8_shared, "shared rows")
    gpu, r = got["out"][want], ref.out[want]
    allow = ref.out_allow[want]
    rms = float(np.sqrt(np.mean(r * r)))
    half = omoe.bf16_half_ulp(r) if wl.out == "bf16" else omoe.f32_half_ulp(r)
    err = np.abs(gpu - r)
    excess = float(np.max(err - half - allow)) / rms
    stats.update(raw=float(np.max(err)) / rms,
                 excess_beyond_rounding=float(np.max(err - half)) / rms,
                 excess_beyond_alternatives=excess,
                 allow_p99=float(np.percentile(allow, 99)) / rms)
    assert np.all(np.isfinite(gpu))
    assert excess <= bar, f"FP8 output beyond the alternatives: {stats}"
    return stats


def _take_rows(det, rows):
    from oracle import moe as _m
    return _m.Fp8Rows(h=det.h[rows], s_lo=det.s_lo[rows], s_hi=det.s_hi[rows],
                      v_lo=det.v_lo[rows], v_hi=det.v_hi[rows],
                      allow=det.allow[rows])


def fp8_complete_check(wl, tokens=None, layout="kn", workers=0):
    """Run the FP8 layer step by step and as one forward (they must agree
    bit for bit) and apply check_fp8_complete against the oracle."""
    print(f"layer {wl.describe()} layout={layout}", flush=True)
    got = run_fp8_steps(wl, layout=layout)
    assert np.array_equal(got["out"], got["out_layer"])
    ref = omoe.layer_from_workload(wl, token_subset=tokens, fp8_detail=True,
                                   workers=workers)
    st = check_fp8_complete(wl, got, ref, tokens)
    print(f"  {st}", flush=True)
    return st


def sample_tokens(T, n, seed=0):
    """n distinct seeded token indices, plus the first and the last."""
    rng = np.random.default_rng(seed)
    s = set(rng.choice(T, size=min(n, T), replace=False).tolist())
    s |= {0, T - 1}
    return np.array(sorted(s))
