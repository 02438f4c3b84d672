"""Device-side plumbing around the C ABI: upload host arrays into torch
device tensors, allocate the caller-owned buffers and workspaces, and call
the entry points on the current stream.

Nothing here computes any part of the layer; it moves memory and passes
pointers.  Host arrays use the stored formats of include/moe.h: float32, or
bf16 bit patterns held in uint16 arrays.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np
import torch

from . import _lib as L


def to_dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    """Copy a host array to the device, keeping its bytes (uint16 bf16
    patterns travel as int16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    elif a.dtype == np.uint8:
        pass
    return torch.from_numpy(a).to(device)


def from_dev_bf16(t: torch.Tensor) -> np.ndarray:
    """bf16 bit patterns of a device tensor as a host uint16 array."""
    return t.cpu().numpy().view(np.uint16)


@dataclasses.dataclass
class LayerBuffers:
    ids: torch.Tensor
    w: torch.Tensor
    counts: torch.Tensor
    offsets: torch.Tensor
    row_token: torch.Tensor
    row_weight: torch.Tensor
    pair_row: torch.Tensor
    x_perm: torch.Tensor
    x_perm_scales: Optional[torch.Tensor]
    y_perm: torch.Tensor
    y_shared: Optional[torch.Tensor]
    out: torch.Tensor
    ws_dispatch: torch.Tensor
    ws_ffn: torch.Tensor
    ws_layer: torch.Tensor


class DeviceLayer:
    """One EP rank's MoE layer with weights resident on the device.

    experts: per physical-expert source, a dict of host arrays wg [H,I],
    wu [H,I], wd [I,H] in the logical layout (float32 for the fp32 and fp8
    recipes -- fp8 weights are quantised on the device by
    moe_quantize_fp8_blocks -- or bf16 bits); ``layout`` "nk" says they are
    stored transposed (wg, wu [I,H], wd [H,I]) instead.
    phys_to_logical maps physical ids to entries of ``experts`` (replicas
    share the source but get their own device copy when copy_replicas)."""

    def __init__(self, problem: L.Problem, experts: Optional[Sequence[dict]],
                 shared: Optional[dict] = None,
                 phys_to_logical: Optional[Sequence[int]] = None,
                 l2p=None, replica_count=None, copy_replicas=True,
                 device="cuda", keep_codes=False, layout="kn"):
        self.p = problem
        self.device = device
        self.layout = L.LAYOUTS[layout]
        self.keep_codes = keep_codes   # fp8: also keep unpacked codes
        P = problem.num_physical
        if phys_to_logical is None:
            phys_to_logical = list(range(P))
        if len(phys_to_logical) != P:
            raise ValueError("phys_to_logical must have num_physical entries")
        self.fp8 = problem.weight_dtype == L.MOE_FP8_E4M3
        self.l2p = None if l2p is None else torch.tensor(
            np.asarray(l2p, dtype=np.int32), device=device)
        self.rep = None if replica_count is None else torch.tensor(
            np.asarray(replica_count, dtype=np.int32), device=device)
        if experts is None:          # routing / dispatch only
            self.keep = [[], None]
            self.weights = L.Weights()
            return
        uploaded = {}
        per_phys: List[dict] = []
        for p, e in enumerate(phys_to_logical):
            if e in uploaded and not copy_replicas:
                per_phys.append(uploaded[e])
                continue
            d = self._upload_expert(experts[e])
            uploaded.setdefault(e, d)
            per_phys.append(d)
        sh = self._upload_expert(shared) if shared is not None else None
        self.keep = [per_phys, sh]
        self.weights = self._tables(per_phys, sh)

    # -------------------------------------------------------- weights
    def _upload_expert(self, e: dict) -> dict:
        out = {}
        for key in ("wg", "wu", "wd"):
            t = to_dev(e[key], self.device)
            rows, cols = t.shape
            # reduction size K and outputs N of this matrix
            K, N = (rows, cols) if self.layout == L.MOE_LAYOUT_KN else (cols, rows)
            if self.fp8:
                codes = torch.empty((rows, cols), dtype=torch.uint8,
                                    device=self.device)
                scales = torch.empty((N // 128, K // 128),
                                     dtype=torch.float32, device=self.device)
                L.moe_quantize_fp8_blocks(t, K, N, 128, self.layout, codes,
                                          scales)
                packed = torch.empty_like(codes)
                L.moe_prepack_weights(codes, K, N, L.MOE_FP8_E4M3,
                                      self.layout, packed)
                if self.keep_codes:
                    out["codes_" + key] = codes
                out[key] = packed
                out["s" + key[1]] = scales
            else:
                prepared = torch.empty_like(t)
                L.moe_prepack_weights(t, K, N, self.p.weight_dtype,
                                      self.layout, prepared)
                out[key] = prepared
            del t
        return out

    def _tables(self, per_phys, sh) -> L.Weights:
        dev = self.device
        self._ptr_tables = []

        def table(key):
            if any(d.get(key) is None for d in per_phys):
                return None
            t = torch.tensor([d[key].data_ptr() for d in per_phys],
                             dtype=torch.int64, device=dev)
            self._ptr_tables.append(t)
            return t.data_ptr()

        s = L.Weights()
        s.w_gate, s.w_up, s.w_down = table("wg"), table("wu"), table("wd")
        s.s_gate, s.s_up, s.s_down = table("sg"), table("su"), table("sd")
        if sh is not None:
            s.sh_gate = sh["wg"].data_ptr()
            s.sh_up = sh["wu"].data_ptr()
            s.sh_down = sh["wd"].data_ptr()
            if self.fp8:
                s.sh_s_gate = sh["sg"].data_ptr()
                s.sh_s_up = sh["su"].data_ptr()
                s.sh_s_down = sh["sd"].data_ptr()
        return s

    def fp8_weights(self, phys: int):
        """Device codes and scales of a physical expert (fp8 recipe)."""
        d = self.keep[0][phys]
        return d

    # -------------------------------------------------------- buffers
    def buffers(self) -> LayerBuffers:
        p, dev = self.p, self.device
        T, H, k = p.T, p.H, p.k
        cap = T * min(p.k, p.num_local)
        act_b = {L.MOE_F32: 4, L.MOE_BF16: 2}[p.act_dtype]
        xb = 1 if self.fp8 else act_b
        out_dt = torch.float32 if p.out_dtype == L.MOE_F32 else torch.int16
        def z(n, dt):
            return torch.empty(max(int(n), 1), dtype=dt, device=dev)
        return LayerBuffers(
            ids=z(T * k, torch.int32), w=z(T * k, torch.float32),
            counts=z(p.E, torch.int32), offsets=z(p.num_physical + 1, torch.int32),
            row_token=z(cap, torch.int32), row_weight=z(cap, torch.float32),
            pair_row=z(T * k, torch.int32),
            x_perm=z(cap * H * xb, torch.uint8),
            x_perm_scales=z(cap * (H // 128), torch.float32) if self.fp8 else None,
            y_perm=z(cap * H, torch.float32),
            y_shared=z(T * H, torch.float32) if p.has_shared else None,
            out=z(T * H, out_dt),
            ws_dispatch=z(L.moe_dispatch_workspace_size(p), torch.uint8),
            ws_ffn=z(L.moe_ffn_workspace_size(p), torch.uint8),
            ws_layer=z(L.moe_layer_workspace_size(p), torch.uint8))

    # -------------------------------------------------------- calls
    def forward(self, b: LayerBuffers, logits, bias, x, counts=True):
        return L.moe_layer_forward(
            self.p, logits, bias, x, self.weights, self.l2p, self.rep, b.out,
            b.counts if counts else None, b.ws_layer, b.ws_layer.numel())

    def route(self, b: LayerBuffers, logits, bias):
        return L.moe_route_topk(self.p, logits, bias, b.ids, b.w, b.counts)

    def dispatch(self, b: LayerBuffers, x):
        return L.moe_dispatch(self.p, x, b.ids, b.w, self.l2p, self.rep,
                              b.x_perm, b.x_perm_scales, b.offsets,
                              b.row_token, b.row_weight, b.pair_row,
                              b.ws_dispatch, b.ws_dispatch.numel())

    def ffn(self, b: LayerBuffers, x_shared=None, x_shared_scales=None):
        return L.moe_grouped_ffn(self.p, b.x_perm, b.x_perm_scales, b.offsets,
                                 x_shared, x_shared_scales, self.weights,
                                 b.y_perm, b.y_shared, b.ws_ffn,
                                 b.ws_ffn.numel())

    def combine(self, b: LayerBuffers):
        return L.moe_combine(self.p, b.y_perm, b.pair_row, b.w, b.y_shared,
                             b.out)
