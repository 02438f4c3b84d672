"""Benchmark of the EP-rank MoE layer on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode]

One step = one moe_layer_forward (route -> dispatch -> grouped SwiGLU FFN ->
combine) over one batch of synthetic input already resident in HBM.  The
headline workload is the decode share of a GLM-5.3-shaped layer (T=256,
H=6144, I=2048, 32 of 256 experts local, k=8, bf16).  Prints ONE JSON line.

Workloads: tiny, decode, prefill, skewed (prefill shape with a Zipf logit
bias, identity placement), skewed_eplb (the same batch with the 8 hottest
local experts given a second physical copy, placed from the first pass's
expert counts by the library's moe_eplb_hottest_map; the layer then reads 40
physical experts' weights), fp8, lowlat (128-token FP8 decode batch).

--graph captures one layer forward into a HIP graph (torch.cuda.CUDAGraph on
the library's stream argument) and times graph replays; the line then also
carries the eager per-step time.

Besides throughput the line carries:
* roofline: the dominant kernel's algorithmic bytes (or flops) per launch over
  its average duration, timed with HIP events recorded by the library on the
  layer's own stream (moe_layer_forward_timed), against MI355X's published
  peak (HBM 8 TB/s; dense bf16 MFMA 2.5 PFLOP/s);
* cpu_baseline: the float64 CPU oracle timed on this host on a bounded sample
  of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s on 1 MI355X; decode HBM TB/s and prefill TFLOP/s vs peak"
HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}


# HBM bytes per launch of each workload's dominant (gate/up) kernel from two
# rocprofv3 counter passes (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch),
# each scaled by the factor that makes the same counter read the known size
# of the weight-prepack kernel in the same run (profiles/ has the commands
# and the tables).  The figures hold for the kernel source they were taken
# on: when the SHA-256 of its files differs, traffic is reported as null.
TRAFFIC = {
    "decode": dict(
        kernel="k_stream_bf16<0, 2>",
        files=("expert_moe_fp32_amd/csrc/ffn.hip",
               "expert_moe_fp32_amd/csrc/common.h"),
        sha="3d950f29938a63d4", fetch_kib=794521.5, write_kib=988.7,
        fetch_factor=1.9969, write_factor=1.0),
    "prefill": dict(
        kernel="k_gemm_bf16<0, 4, 2, 2, 4>",
        files=("expert_moe_fp32_amd/csrc/gemm_bf16.hip",
               "expert_moe_fp32_amd/csrc/common.h"),
        sha="04112b138a402e5f", fetch_kib=1890216.9, write_kib=65704.0,
        fetch_factor=1.9973, write_factor=1.0),
    "fp8": dict(
        kernel="k_ring_fp8<0, 10>",
        files=("expert_moe_fp32_amd/csrc/ffn_fp8.hip",
               "expert_moe_fp32_amd/csrc/common.h"),
        sha="919aacd5cdd58cb6", fetch_kib=485395.3, write_kib=33232.1,
        fetch_factor=1.9965, write_factor=1.0),
}


def traffic_bytes(workload):
    """Counter-derived HBM bytes per launch, or None (no counters for this
    workload, or the kernel's source changed since they were taken)."""
    import hashlib
    t = TRAFFIC.get(workload)
    if t is None:
        return None
    h = hashlib.sha256()
    for f in t["files"]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest()[:16] != t["sha"]:
        return None
    return int((t["fetch_kib"] * t["fetch_factor"] +
                t["write_kib"] * t["write_factor"]) * 1024)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Hip:
    """hipEvent plumbing through the HIP runtime's C API."""

    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so")
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                               ctypes.c_void_p, ctypes.c_void_p]
        self.h.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self) -> int:
        e = ctypes.c_void_p()
        assert self.h.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def record(self, e, stream):
        assert self.h.hipEventRecord(e, stream) == 0

    def ms(self, a, b) -> float:
        assert self.h.hipEventSynchronize(b) == 0
        t = ctypes.c_float()
        assert self.h.hipEventElapsedTime(ctypes.byref(t), a, b) == 0
        return float(t.value)

    def destroy(self, e):
        self.h.hipEventDestroy(e)


def replica_counts(local_counts, l2p, rep, P):
    """Rows of every physical expert: replica r of an expert with n pairs and
    R replicas gets ceil((n - r) / R) of them (pair n goes to replica n % R)."""
    out = np.zeros(P, dtype=np.int64)
    for e, n in enumerate(local_counts):
        R = int(rep[e]) if rep is not None else 1
        for r in range(R):
            p = int(l2p[e][r]) if l2p is not None else e
            out[p] = max(0, -(-(int(n) - r) // R))
    return out


def kernel_units(wl, counts, P, phys_counts):
    """Algorithmic work of the gate/up and down launches for this batch."""
    H, I = wl.H, wl.I
    wb = {"bf16": 2, "fp8": 1, "f32": 4}[wl.wdt]
    ab = 1 if wl.wdt == "fp8" else (4 if wl.act == "f32" else 2)
    hb = ab
    nonempty = int(np.count_nonzero(phys_counts))
    N = int(np.sum(phys_counts))
    rows_sh = wl.T if wl.shared else 0
    n_w = nonempty + (1 if wl.shared else 0)
    rows = N + rows_sh
    gu_bytes = n_w * 2 * H * I * wb + rows * H * ab + rows * I * hb
    dn_bytes = n_w * I * H * wb + rows * I * hb + rows * H * 4
    gu_flops = rows * 4.0 * H * I
    dn_flops = rows * 2.0 * H * I
    return dict(nonempty=nonempty, N=N, rows=rows, gu_bytes=gu_bytes,
                dn_bytes=dn_bytes, gu_flops=gu_flops, dn_flops=dn_flops,
                weight_bytes=n_w * 3 * H * I * wb)


def cpu_baseline(wl, sample_tokens, l2p=None, rep=None, P=None):
    """The oracle as it stands, on the host cores, over a bounded sample."""
    from oracle import moe as omoe
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    ex = omoe.expert_set_from_workload(wl, lazy=True)
    res = omoe.layer_from_workload(wl, ex, l2p=l2p, rep_count=rep, P=P,
                                   token_subset=sample_tokens)
    dt = time.perf_counter() - t0
    n = len(sample_tokens)
    return res, dict(value=n / dt, unit="tokens/s", cores=int(threads),
                     kind="oracle",
                     sample=f"{n} of {wl.T} tokens of the {wl.name} workload "
                            f"(route + dispatch of all tokens, float64 experts "
                            f"for the sampled ones), {dt:.1f} s")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode",
                    choices=["tiny", "decode", "prefill", "skewed",
                             "skewed_eplb", "fp8", "lowlat"])
    ap.add_argument("--graph", action="store_true",
                    help="time replays of a HIP graph of one step")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true",
                    help="skip the CPU oracle baseline leg")
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="oracle sample size (0 = workload default)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark measures one EP rank's "
                          "share on one GPU; --gpus must be 1"}))
        sys.exit(2)

    import torch
    import expert_moe_fp32_amd as m
    from expert_moe_fp32_amd import _lib as L
    from expert_moe_fp32_amd.runner import DeviceLayer, to_dev
    from synth import make_workload

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    eplb = args.workload == "skewed_eplb"
    wl = make_workload("skewed" if eplb else args.workload, seed=args.seed)
    log(f"bench: {wl.describe()}")
    t0 = time.perf_counter()
    dlog, dx = to_dev(wl.logits), to_dev(wl.x)
    dbias = None if wl.bias is None else to_dev(wl.bias)
    l2p = rep = None
    P = wl.num_local
    phys_to_logical = None
    if eplb:
        # expert counts of this batch (the first pass), then the placement
        prob0 = m.make_problem(T=wl.T, H=wl.H, I=wl.I, E=wl.E, k=wl.k,
                               expert_begin=wl.expert_begin,
                               num_local=wl.num_local, has_shared=wl.shared,
                               act=wl.act, wdt=wl.wdt, out=wl.out)
        ids = torch.empty((wl.T, wl.k), dtype=torch.int32, device="cuda")
        w = torch.empty((wl.T, wl.k), dtype=torch.float32, device="cuda")
        cnt = torch.zeros(wl.E, dtype=torch.int32, device="cuda")
        L.moe_route_topk(prob0, dlog, dbias, ids, w, cnt)
        local = cnt.cpu().numpy()[wl.expert_begin: wl.expert_begin + wl.num_local]
        l2p, rep, P = L.moe_eplb_hottest_map(local, wl.redundant)
        l2p = np.asarray(l2p, dtype=np.int32)
        rep = np.asarray(rep, dtype=np.int32)
        phys_to_logical = [-1] * P
        for e in range(wl.num_local):
            for r in range(int(rep[e])):
                phys_to_logical[int(l2p[e][r])] = e
        del ids, w, cnt
    prob = m.make_problem(T=wl.T, H=wl.H, I=wl.I, E=wl.E, k=wl.k,
                          expert_begin=wl.expert_begin,
                          num_local=wl.num_local, num_physical=P,
                          max_replicas=1 if l2p is None else int(np.shape(l2p)[1]),
                          has_shared=wl.shared,
                          act=wl.act, wdt=wl.wdt, out=wl.out)
    dl = DeviceLayer(prob, [wl.expert(e) for e in range(wl.num_local)],
                     wl.shared_expert, phys_to_logical=phys_to_logical,
                     l2p=l2p, replica_count=rep)
    b = dl.buffers()
    torch.cuda.synchronize()
    log(f"bench: inputs resident in HBM ({time.perf_counter() - t0:.1f} s)")
    stream = torch.cuda.current_stream().cuda_stream
    hip = Hip()

    def step():
        dl.forward(b, dlog, dbias, dx)

    def timed(fn, k):
        e0, e1 = hip.event(), hip.event()
        torch.cuda.synchronize()
        hip.record(e0, torch.cuda.current_stream().cuda_stream)
        for _ in range(k):
            fn()
        hip.record(e1, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        ms = hip.ms(e0, e1) / k
        hip.destroy(e0)
        hip.destroy(e1)
        return ms

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    eager_ms = None
    if args.graph:
        eager_ms = timed(step, args.steps)
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        step = graph.replay
    # ---- timed region: exactly K layer forwards
    e0, e1 = hip.event(), hip.event()
    torch.cuda.synchronize()
    hip.record(e0, stream)
    t_wall = time.perf_counter()
    for _ in range(args.steps):
        step()
    hip.record(e1, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    total_ms = hip.ms(e0, e1)
    ms_per_step = total_ms / args.steps
    log(f"bench: {args.steps} steps, {ms_per_step * 1e3:.1f} us/step "
        f"(wall {wall * 1e6 / args.steps:.1f} us/step)")

    # ---- per-stage durations, on the layer's stream
    reps = max(10, min(args.steps, 50))
    evs = [[hip.event() for _ in range(L.MOE_STAGE_EVENTS)] for _ in range(reps)]
    for r in range(reps):
        L.moe_layer_forward_timed(prob, dlog, dbias, dx, dl.weights, dl.l2p,
                                  dl.rep, b.out, b.counts, b.ws_layer,
                                  b.ws_layer.numel(), evs[r], stream=stream)
    torch.cuda.synchronize()
    stage_ms = {name: float(np.mean([hip.ms(evs[r][i], evs[r][i + 1])
                                     for r in range(reps)]))
                for i, name in enumerate(L.STAGES)}
    for row in evs:
        for e in row:
            hip.destroy(e)

    counts = b.counts.cpu().numpy()
    local_counts = counts[wl.expert_begin: wl.expert_begin + wl.num_local]
    phys_counts = replica_counts(local_counts, l2p, rep, P)
    u = kernel_units(wl, counts, P, phys_counts)
    tokens_per_s = wl.T / (ms_per_step * 1e-3)
    flops = u["gu_flops"] + u["dn_flops"]
    layer_tflops = flops / (ms_per_step * 1e-3) / 1e12
    weight_tbps = u["weight_bytes"] / (ms_per_step * 1e-3) / 1e12
    # dominant kernel: the gate/up launch (2/3 of the weight bytes and flops)
    gu_s = stage_ms["gate_up"] * 1e-3
    dn_s = stage_ms["down"] * 1e-3
    prec = "fp8" if wl.wdt == "fp8" else wl.act
    ridge = MFMA_PEAK_TFLOPS[prec] * 1e12 / (HBM_PEAK_GBPS * 1e9)
    ai = u["gu_flops"] / u["gu_bytes"]
    traffic = traffic_bytes(args.workload)
    if ai < ridge:
        achieved = u["gu_bytes"] / gu_s / 1e9
        roof = dict(bound="hbm", kernel="gate_up", achieved=round(achieved, 1),
                    peak=HBM_PEAK_GBPS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBPS, 4), traffic=traffic,
                    algorithmic_bytes=int(u["gu_bytes"]),
                    avg_us=round(gu_s * 1e6, 2))
    else:
        achieved = u["gu_flops"] / gu_s / 1e12
        roof = dict(bound="mfma", kernel="gate_up", achieved=round(achieved, 1),
                    peak=MFMA_PEAK_TFLOPS[prec], unit="TFLOP/s",
                    frac=round(achieved / MFMA_PEAK_TFLOPS[prec], 4),
                    traffic=traffic, algorithmic_flops=u["gu_flops"],
                    avg_us=round(gu_s * 1e6, 2))

    # whole-layer roofline: the larger of the flop time at the MFMA peak and
    # the time to move the minimum bytes (weights of non-empty experts, x,
    # logits, out) at the HBM peak, over the measured step
    ab = 4 if wl.act == "f32" else 2
    ob = 4 if wl.out == "f32" else 2
    min_bytes = (u["weight_bytes"] + wl.T * wl.H * ab + wl.T * wl.E * 4
                 + wl.T * wl.H * ob)
    t_flop = flops / (MFMA_PEAK_TFLOPS[prec] * 1e12)
    t_mem = min_bytes / (HBM_PEAK_GBPS * 1e9)
    layer_roof = max(t_flop, t_mem) / (ms_per_step * 1e-3)

    result = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": prec,
        "data": "synthetic",
        "config": {"workload": args.workload, "T": wl.T, "H": wl.H, "I": wl.I,
                   "E": wl.E, "k": wl.k, "local_experts": wl.num_local,
                   "shared_expert": wl.shared, "weights": wl.wdt,
                   "activations": wl.act, "out": wl.out, "seed": wl.seed},
        "roofline": roof,
        "layer": {"weight_TBps": round(weight_tbps, 3),
                  "weight_frac_of_hbm_peak": round(weight_tbps * 1e3 / HBM_PEAK_GBPS, 4),
                  "TFLOPps": round(layer_tflops, 2),
                  "mfma_frac": round(layer_tflops / MFMA_PEAK_TFLOPS[prec], 4),
                  "local_rows": u["N"], "nonempty_experts": u["nonempty"],
                  "expert_weight_bytes": u["weight_bytes"],
                  "min_bytes": int(min_bytes),
                  "roofline_frac": round(layer_roof, 4),
                  "roofline_bound": "mfma" if t_flop > t_mem else "hbm"},
        "stages_us": {k: round(v * 1e3, 2) for k, v in stage_ms.items()},
        "down_GBps": round(u["dn_bytes"] / dn_s / 1e9, 1),
    }
    if args.graph:
        result["graph"] = {"replay_us_per_step": round(ms_per_step * 1e3, 2),
                           "eager_us_per_step": round(eager_ms * 1e3, 2)}
    if wl.name == "skewed":
        lc = local_counts.astype(np.float64)
        pc = phys_counts.astype(np.float64)
        result["imbalance"] = {
            "physical_experts": P,
            "busiest_over_mean": round(float(pc.max() / pc.mean()), 3),
            "mean_over_busiest": round(float(pc.mean() / pc.max()), 4),
            "busiest_over_mean_without_replicas": round(float(lc.max() / lc.mean()), 3),
            "empty_local_experts": int(np.count_nonzero(lc == 0)),
        }
    if not args.no_cpu:
        n = args.cpu_tokens or {"tiny": 128, "decode": 256, "prefill": 16,
                                "skewed": 16, "fp8": 16, "lowlat": 8}[wl.name]
        rng = np.random.default_rng(1)
        tok = np.sort(rng.choice(wl.T, size=min(n, wl.T), replace=False))
        log(f"bench: CPU oracle on {len(tok)} tokens ...")
        res, base = cpu_baseline(wl, tok, l2p, rep, P if eplb else None)
        result["cpu_baseline"] = base
        from oracle import moe as omoe
        got = b.out[: wl.T * wl.H].cpu().numpy()
        got = (omoe.bf16_to_f64(got.view(np.uint16)) if wl.out == "bf16"
               else got.astype(np.float64)).reshape(wl.T, wl.H)[tok]
        ref = res.out[tok]
        rms = float(np.sqrt(np.mean(ref * ref)))
        err = np.abs(got - ref)
        half = (omoe.bf16_half_ulp(ref) if wl.out == "bf16"
                else omoe.f32_half_ulp(ref))
        # the tests' measure: error beyond the output format's own rounding
        result["parity_sample"] = {
            "tokens": int(len(tok)),
            "max_err_over_rms": float(np.max(err) / rms),
            "max_err_beyond_out_rounding_over_rms": float(np.max(err - half) / rms),
            "bar": {"f32": 1e-5, "bf16": 1e-2, "fp8": 4e-2}[prec]}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
