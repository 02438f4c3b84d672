"""Benchmark of the EP-rank MoE layer on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode]

One step = one moe_layer_forward (route -> dispatch -> grouped SwiGLU FFN ->
combine) over one batch of synthetic input already resident in HBM.  The
headline workload is the decode share of a GLM-5.3-shaped layer (T=256,
H=6144, I=2048, 32 of 256 experts local, k=8, bf16).  Prints ONE JSON line.

Workloads: tiny, decode, decode_skewed (decode with a Zipf logit bias: one
hot local expert), prefill, skewed (prefill shape with a Zipf logit bias,
identity placement), skewed_eplb (the same batch with the 8 hottest local
experts given a second physical copy, placed from the first pass's expert
counts by the library's moe_eplb_hottest_map; the layer then reads 40
physical experts' weights), fp8, lowlat (128-token FP8 decode batch),
lowlat_skewed (lowlat with a Zipf logit bias).

With the default workload the same run also times the prefill workload (the
metric's other half, TFLOP/s against the MFMA peak) and reports it in a
``prefill`` object of the same line (--no-prefill skips it).

--graph captures one layer forward into a HIP graph (torch.cuda.CUDAGraph on
the library's stream argument) and times graph replays; the line then also
carries the eager per-step time.

Besides throughput the line carries:
* roofline: the dominant kernel's algorithmic bytes (or flops) per launch over
  its average duration, timed with HIP events recorded by the library on the
  layer's own stream (moe_layer_forward_timed), against MI355X's published
  peak (HBM 8 TB/s; dense bf16 MFMA 2.5 PFLOP/s, fp8 5.0);
* permute / combine: the dispatch gather (a standalone moe_dispatch, which
  writes the permuted rows) and the layer's combine in HBM GB/s;
* cpu_baseline: the float64 CPU oracle timed on this host on a bounded
  sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
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
WORKLOADS = ["tiny", "decode", "decode_skewed", "prefill", "skewed",
             "skewed_eplb", "fp8", "lowlat", "lowlat_skewed"]


# Counter figures per launch of each workload's dominant (gate/up) kernel,
# from rocprofv3 --pmc runs of this script (the profile named in each entry
# has the commands and the per-kernel tables).  HBM bytes: FETCH_SIZE and
# WRITE_SIZE (KiB per dispatch), each scaled by the factor that makes the
# same counter read the known size of a streaming kernel with the same
# 16-byte accesses in the same run (bf16: the weight prepack k_pack_bf16;
# FP8: the activation quantiser k_quant_rows_fp8).  MFMA utilisation:
# SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE / 8 (the counter sums the 8
# XCDs) x 1024 SIMDs, i.e. the fraction of the kernel's own cycles the
# matrix cores were busy.  The figures hold for the kernel they were taken
# on: when the SHA-256 of its files differs, they are reported as null (the
# SHA is moved on only where the kernel's gfx950 machine code was compared
# and found unchanged by an edit elsewhere in those files).
COUNTERS = {
    "tiny": {
        "kernel": "k_f32<0>", "profile": "profiles/layer_f32_tiny.md",
        "files": ["expert_moe_fp32_amd/csrc/ffn.hip", "expert_moe_fp32_amd/csrc/common.h"],
        "sha": "a61869c6790dad6e",
        "fetch_kib": 1831.6, "fetch_factor": 1.5784,
        "write_kib": 128.0, "write_factor": 1.0},
    "decode": {
        "kernel": "k_stream_bf16<0, 2>", "profile": "profiles/layer_stream_bf16_decode.md",
        "files": ["expert_moe_fp32_amd/csrc/ffn.hip", "expert_moe_fp32_amd/csrc/common.h"],
        "sha": "a61869c6790dad6e",
        "fetch_kib": 794472.6, "fetch_factor": 1.9976,
        "write_kib": 988.7, "write_factor": 1.0,
        "mfma_util": 0.051},
    "decode_skewed": {
        "kernel": "k_stream_bf16<0, 2>", "profile": "profiles/layer_stream_bf16_decode_skewed.md",
        "files": ["expert_moe_fp32_amd/csrc/ffn.hip", "expert_moe_fp32_amd/csrc/common.h"],
        "sha": "a61869c6790dad6e",
        "fetch_kib": 207722.8, "fetch_factor": 1.9976,
        "write_kib": 875.4, "write_factor": 1.0,
        "mfma_util": 0.052},
    "prefill": {
        "kernel": "k_gemm_bf16<0, 4, 2, 2, 4>", "profile": "profiles/layer_gemm_bf16_prefill.md",
        "files": ["expert_moe_fp32_amd/csrc/gemm_bf16.hip", "expert_moe_fp32_amd/csrc/common.h"],
        "sha": "bb5473dae36f2749",
        "fetch_kib": 1818199.8, "fetch_factor": 1.9979,
        "write_kib": 71848.3, "write_factor": 1.0,
        "mfma_util": 0.586},
    "skewed": {
        "kernel": "k_gemm_bf16<0, 4, 2, 2, 4>", "profile": "profiles/layer_gemm_bf16_skewed.md",
        "files": ["expert_moe_fp32_amd/csrc/gemm_bf16.hip", "expert_moe_fp32_amd/csrc/common.h"],
        "sha": "bb5473dae36f2749",
        "fetch_kib": 1708994.9, "fetch_factor": 1.9979,
        "write_kib": 55172.0, "write_factor": 1.0,
        "mfma_util": 0.469},
    "skewed_eplb": {
        "kernel": "k_gemm_bf16<0, 4, 2, 2, 4>", "profile": "profiles/layer_gemm_bf16_skewed_eplb.md",
        "files": ["expert_moe_fp32_amd/csrc/gemm_bf16.hip", "expert_moe_fp32_amd/csrc/common.h"],
        "sha": "bb5473dae36f2749",
        "fetch_kib": 1991712.3, "fetch_factor": 1.9979,
        "write_kib": 55220.1, "write_factor": 1.0,
        "mfma_util": 0.421},
    "fp8": {
        "kernel": "k_ring_fp8<0, 10>", "profile": "profiles/layer_ring_fp8_fp8.md",
        "files": ["expert_moe_fp32_amd/csrc/ffn_fp8.hip", "expert_moe_fp32_amd/csrc/common.h"],
        "sha": "74796710a92125a6",
        "fetch_kib": 485368.9, "fetch_factor": 1.9987,
        "write_kib": 33232.1, "write_factor": 1.0,
        "mfma_util": 0.295},
    "lowlat": {
        "kernel": "k_wstream_fp8<0>", "profile": "profiles/layer_wstream_fp8_lowlat.md",
        "files": ["expert_moe_fp32_amd/csrc/ffn_fp8.hip", "expert_moe_fp32_amd/csrc/common.h"],
        "sha": "74796710a92125a6",
        "fetch_kib": 452572.8, "fetch_factor": 1.9637,
        "write_kib": 278.1, "write_factor": 1.0,
        "mfma_util": 0.080},
    "lowlat_skewed": {
        "kernel": "k_wstream_fp8<0>", "profile": "profiles/layer_wstream_fp8_lowlat_skewed.md",
        "files": ["expert_moe_fp32_amd/csrc/ffn_fp8.hip", "expert_moe_fp32_amd/csrc/common.h"],
        "sha": "74796710a92125a6",
        "fetch_kib": 162262.5, "fetch_factor": 1.9637,
        "write_kib": 566.7, "write_factor": 1.0},
}


def _source_sha(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counters(workload):
    """(traffic bytes or None, mfma utilisation or None) of the dominant
    kernel: None where no counters were taken or the source changed."""
    t = COUNTERS.get(workload)
    if t is None or _source_sha(t["files"]) != t["sha"]:
        return None, None
    traffic = None
    if "fetch_kib" in t:
        traffic = int((t["fetch_kib"] * t["fetch_factor"] +
                       t["write_kib"] * t["write_factor"]) * 1024)
    return traffic, t.get("mfma_util")


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


def kernel_units(wl, phys_counts):
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
                            f"(float64 NumPy oracle: route + dispatch of all "
                            f"tokens, every expert evaluated on the sampled "
                            f"tokens' rows, one thread per BLAS call), "
                            f"{dt:.1f} s")


class Bench:
    """One workload resident on the device, ready to step."""

    def __init__(self, workload, seed, hip):
        import torch
        import expert_moe_fp32_amd as m
        from expert_moe_fp32_amd import _lib as L
        from expert_moe_fp32_amd.runner import DeviceLayer, to_dev
        from synth import make_workload

        self.name = workload
        self.hip = hip
        self.L = L
        eplb = workload == "skewed_eplb"
        self.eplb = eplb
        wl = make_workload("skewed" if eplb else workload, seed=seed)
        self.wl = wl
        log(f"bench: {wl.describe()}")
        t0 = time.perf_counter()
        self.dlog, self.dx = to_dev(wl.logits), to_dev(wl.x)
        self.dbias = None if wl.bias is None else to_dev(wl.bias)
        l2p = rep = None
        P = wl.num_local
        phys_to_logical = None
        if eplb:
            # expert counts of this batch (the first pass), then the placement
            prob0 = m.make_problem(T=wl.T, H=wl.H, I=wl.I, E=wl.E, k=wl.k,
                                   expert_begin=wl.expert_begin,
                                   num_local=wl.num_local,
                                   has_shared=wl.shared, act=wl.act,
                                   wdt=wl.wdt, out=wl.out)
            ids = torch.empty((wl.T, wl.k), dtype=torch.int32, device="cuda")
            w = torch.empty((wl.T, wl.k), dtype=torch.float32, device="cuda")
            cnt = torch.zeros(wl.E, dtype=torch.int32, device="cuda")
            L.moe_route_topk(prob0, self.dlog, self.dbias, ids, w, cnt)
            local = cnt.cpu().numpy()[wl.expert_begin: wl.expert_begin + wl.num_local]
            l2p, rep, P = L.moe_eplb_hottest_map(local, wl.redundant)
            l2p = np.asarray(l2p, dtype=np.int32)
            rep = np.asarray(rep, dtype=np.int32)
            phys_to_logical = [-1] * P
            for e in range(wl.num_local):
                for r in range(int(rep[e])):
                    phys_to_logical[int(l2p[e][r])] = e
            del ids, w, cnt
        self.l2p, self.rep, self.P = l2p, rep, P
        self.prob = m.make_problem(
            T=wl.T, H=wl.H, I=wl.I, E=wl.E, k=wl.k,
            expert_begin=wl.expert_begin, num_local=wl.num_local,
            num_physical=P,
            max_replicas=1 if l2p is None else int(np.shape(l2p)[1]),
            has_shared=wl.shared, act=wl.act, wdt=wl.wdt, out=wl.out)
        self.dl = DeviceLayer(self.prob,
                              [wl.expert(e) for e in range(wl.num_local)],
                              wl.shared_expert,
                              phys_to_logical=phys_to_logical, l2p=l2p,
                              replica_count=rep)
        self.b = self.dl.buffers()
        torch.cuda.synchronize()
        log(f"bench: inputs resident in HBM ({time.perf_counter() - t0:.1f} s)")
        self.stream = torch.cuda.current_stream().cuda_stream

    def step(self):
        self.dl.forward(self.b, self.dlog, self.dbias, self.dx)

    def timed(self, fn, k):
        """Average ms of k calls of fn, HIP events on the library's stream."""
        import torch
        hip = self.hip
        e0, e1 = hip.event(), hip.event()
        torch.cuda.synchronize()
        hip.record(e0, self.stream)
        for _ in range(k):
            fn()
        hip.record(e1, self.stream)
        torch.cuda.synchronize()
        ms = hip.ms(e0, e1) / k
        hip.destroy(e0)
        hip.destroy(e1)
        return ms

    def stage_ms(self, reps):
        """Per-stage durations from the library's own events."""
        import torch
        L, hip = self.L, self.hip
        evs = [[hip.event() for _ in range(L.MOE_STAGE_EVENTS)]
               for _ in range(reps)]
        for r in range(reps):
            L.moe_layer_forward_timed(self.prob, self.dlog, self.dbias,
                                      self.dx, self.dl.weights, self.dl.l2p,
                                      self.dl.rep, self.b.out, self.b.counts,
                                      self.b.ws_layer, self.b.ws_layer.numel(),
                                      evs[r], stream=self.stream)
        torch.cuda.synchronize()
        out = {name: float(np.mean([hip.ms(evs[r][i], evs[r][i + 1])
                                    for r in range(reps)]))
               for i, name in enumerate(L.STAGES)}
        for row in evs:
            for e in row:
                hip.destroy(e)
        return out

    def permute_ms(self, reps):
        """A standalone moe_dispatch (index + the gather that writes the
        permuted rows), after the route that feeds it."""
        self.dl.route(self.b, self.dlog, self.dbias)
        self.dl.dispatch(self.b, self.dx)
        return self.timed(lambda: self.dl.dispatch(self.b, self.dx), reps)

    def close(self):
        import torch
        del self.dl, self.b, self.dlog, self.dx, self.dbias
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


def measure(bn: Bench, steps, warmup, graph=False):
    """Time exactly `steps` layer forwards (after `warmup`), then the stage
    breakdown, the permute leg and the rooflines."""
    import torch
    wl = bn.wl
    step = bn.step
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    eager_ms = None
    if graph:
        eager_ms = bn.timed(step, steps)
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            step()
        torch.cuda.synchronize()
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        step = g.replay
    # ---- timed region: exactly `steps` layer forwards
    t_wall = time.perf_counter()
    ms_per_step = bn.timed(step, steps)
    wall = time.perf_counter() - t_wall
    log(f"bench: {wl.name}: {steps} steps, {ms_per_step * 1e3:.1f} us/step "
        f"(wall {wall * 1e6 / steps:.1f} us/step)")
    reps = max(10, min(steps, 50))
    stage = bn.stage_ms(reps)
    perm_ms = bn.permute_ms(reps)

    counts = bn.b.counts.cpu().numpy()
    local_counts = counts[wl.expert_begin: wl.expert_begin + wl.num_local]
    phys_counts = replica_counts(local_counts, bn.l2p, bn.rep, bn.P)
    u = kernel_units(wl, phys_counts)
    flops = u["gu_flops"] + u["dn_flops"]
    prec = "fp8" if wl.wdt == "fp8" else wl.act
    peak_tf = MFMA_PEAK_TFLOPS[prec]
    # dominant kernel: the gate/up launch (2/3 of the weight bytes and flops)
    gu_s = stage["gate_up"] * 1e-3
    dn_s = stage["down"] * 1e-3
    ridge = peak_tf * 1e12 / (HBM_PEAK_GBPS * 1e9)
    ai = u["gu_flops"] / u["gu_bytes"]
    traffic, mfma_util = counters(bn.name)
    if ai < ridge:
        achieved = u["gu_bytes"] / gu_s / 1e9
        roof = dict(bound="hbm", kernel="gate_up", achieved=round(achieved, 1),
                    peak=HBM_PEAK_GBPS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBPS, 4), traffic=traffic,
                    algorithmic_bytes=int(u["gu_bytes"]),
                    avg_us=round(gu_s * 1e6, 2), mfma_util=mfma_util)
    else:
        achieved = u["gu_flops"] / gu_s / 1e12
        roof = dict(bound="mfma", kernel="gate_up", achieved=round(achieved, 1),
                    peak=peak_tf, unit="TFLOP/s",
                    frac=round(achieved / peak_tf, 4), traffic=traffic,
                    algorithmic_flops=u["gu_flops"],
                    algorithmic_bytes=int(u["gu_bytes"]),
                    avg_us=round(gu_s * 1e6, 2), mfma_util=mfma_util)
    # whole-layer roofline: the larger of the flop time at the MFMA peak and
    # the time to move the minimum bytes (weights of non-empty experts, x,
    # logits, out) at the HBM peak, over the measured step
    ab = 4 if wl.act == "f32" else 2
    ob = 4 if wl.out == "f32" else 2
    min_bytes = (u["weight_bytes"] + wl.T * wl.H * ab + wl.T * wl.E * 4
                 + wl.T * wl.H * ob)
    t_flop = flops / (peak_tf * 1e12)
    t_mem = min_bytes / (HBM_PEAK_GBPS * 1e9)
    layer_roof = max(t_flop, t_mem) / (ms_per_step * 1e-3)
    step_s = ms_per_step * 1e-3
    # permute: the gather reads N token rows and writes them permuted (FP8:
    # it first quantises all T rows: T*H*2 in, T*H + T*H/32 out; then moves
    # N rows of codes and their scales)
    N, H = u["N"], wl.H
    if wl.wdt == "fp8":
        perm_bytes = (wl.T * H * 2 + wl.T * H * (1 + 4 / 128)
                      + 2 * N * H * (1 + 4 / 128))
    else:
        perm_bytes = 2 * N * H * ab
    # combine: every local row's float32 output (and the shared expert's)
    # read once, the output row written once
    comb_bytes = ((N + (wl.T if wl.shared else 0)) * H * 4 +
                  wl.T * wl.k * 8 + wl.T * H * ob)
    res = {
        "ms_per_step": round(ms_per_step, 5),
        "tokens_per_s": round(wl.T / step_s, 1),
        "roofline": roof,
        "layer": {"weight_TBps": round(u["weight_bytes"] / step_s / 1e12, 3),
                  "weight_frac_of_hbm_peak": round(
                      u["weight_bytes"] / step_s / 1e9 / HBM_PEAK_GBPS, 4),
                  "TFLOPps": round(flops / step_s / 1e12, 2),
                  "mfma_frac": round(flops / step_s / 1e12 / peak_tf, 4),
                  "local_rows": u["N"], "nonempty_experts": u["nonempty"],
                  "expert_weight_bytes": u["weight_bytes"],
                  "min_bytes": int(min_bytes),
                  "roofline_frac": round(layer_roof, 4),
                  "roofline_bound": "mfma" if t_flop > t_mem else "hbm"},
        "stages_us": {k: round(v * 1e3, 2) for k, v in stage.items()},
        "down_GBps": round(u["dn_bytes"] / dn_s / 1e9, 1),
        "permute": {"bytes": int(perm_bytes), "us": round(perm_ms * 1e3, 2),
                    "GBps": round(perm_bytes / (perm_ms * 1e-3) / 1e9, 1),
                    "what": "standalone moe_dispatch: index + gather of the "
                            "local rows into expert order"},
        "combine": {"bytes": int(comb_bytes),
                    "us": round(stage["combine"] * 1e3, 2),
                    "GBps": round(comb_bytes / (stage["combine"] * 1e-3) / 1e9,
                                  1)},
    }
    if eager_ms is not None:
        res["graph"] = {"replay_us_per_step": round(ms_per_step * 1e3, 2),
                        "eager_us_per_step": round(eager_ms * 1e3, 2)}
    if wl.bias_kind == "zipf":
        lc = local_counts.astype(np.float64)
        pc = phys_counts.astype(np.float64)
        res["imbalance"] = {
            "physical_experts": bn.P,
            "busiest_over_mean": round(float(pc.max() / pc.mean()), 3),
            "mean_over_busiest": round(float(pc.mean() / pc.max()), 4),
            "busiest_over_mean_without_replicas": round(float(lc.max() / lc.mean()), 3),
            "empty_local_experts": int(np.count_nonzero(lc == 0)),
            "busiest_rows": int(pc.max()),
        }
    return res, prec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode", choices=WORKLOADS)
    ap.add_argument("--graph", action="store_true",
                    help="time replays of a HIP graph of one step")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true",
                    help="skip the CPU oracle baseline leg")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill leg of the default workload")
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="oracle sample size (0 = workload default)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark measures one EP rank's "
                          "share on one GPU; --gpus must be 1"}))
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    hip = Hip()
    bn = Bench(args.workload, args.seed, hip)
    wl = bn.wl
    res, prec = measure(bn, args.steps, args.warmup, graph=args.graph)
    result = {
        "metric": METRIC,
        "value": res.pop("tokens_per_s"),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": prec,
        "data": "synthetic",
        "config": {"workload": args.workload, "T": wl.T, "H": wl.H, "I": wl.I,
                   "E": wl.E, "k": wl.k, "local_experts": wl.num_local,
                   "shared_expert": wl.shared, "weights": wl.wdt,
                   "activations": wl.act, "out": wl.out, "seed": wl.seed},
    }
    result.update(res)
    if not args.no_cpu:
        n = args.cpu_tokens or {"tiny": 128, "decode": 256,
                                "decode_skewed": 256, "prefill": 16,
                                "skewed": 16, "fp8": 16,
                                "lowlat": 8, "lowlat_skewed": 8}[wl.name]
        rng = np.random.default_rng(1)
        tok = np.sort(rng.choice(wl.T, size=min(n, wl.T), replace=False))
        log(f"bench: CPU oracle on {len(tok)} tokens ...")
        ref, base = cpu_baseline(wl, tok, bn.l2p, bn.rep,
                                 bn.P if bn.eplb else None)
        result["cpu_baseline"] = base
        from oracle import moe as omoe
        got = bn.b.out[: wl.T * wl.H].cpu().numpy()
        got = (omoe.bf16_to_f64(got.view(np.uint16)) if wl.out == "bf16"
               else got.astype(np.float64)).reshape(wl.T, wl.H)[tok]
        r = ref.out[tok]
        rms = float(np.sqrt(np.mean(r * r)))
        err = np.abs(got - r)
        half = (omoe.bf16_half_ulp(r) if wl.out == "bf16"
                else omoe.f32_half_ulp(r))
        # the tests' measure: error beyond the output format's own rounding
        result["parity_sample"] = {
            "tokens": int(len(tok)),
            "max_err_over_rms": float(np.max(err) / rms),
            "max_err_beyond_out_rounding_over_rms": float(np.max(err - half) / rms),
            "bar": {"f32": 1e-5, "bf16": 1e-2, "fp8": 4e-2}[prec]}
    bn.close()
    if args.workload == "decode" and not args.no_prefill:
        # the metric's other half: prefill TFLOP/s, timed the same way
        pb = Bench("prefill", args.seed, hip)
        pres, _ = measure(pb, args.steps, args.warmup)
        pres["workload"] = "prefill"
        pres["T"] = pb.wl.T
        result["prefill"] = pres
        pb.close()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
