"""Seeded synthetic workloads for the expert-parallel MoE layer.

The five workloads follow the problem statement of the pages (E routed experts,
k active per token, hidden size H, expert intermediate size I, an optional
always-on shared expert, one EP rank's contiguous share of experts):

* ``tiny``    T=128, H=256, I=128, E=8 (all local), k=2, fp32 everywhere.  The
  shape of the EP=4 / 8-expert / top-2 dispatch figure on the infra-guide page
  ("6.4 Data parallelism and expert parallelism", section 3.1).
* ``decode``  GLM-5.3-like expert shape (H=6144, I=2048, E=256, k=8) from the
  aiinfrainterviews "Expert Parallel and All-to-All Backends" worked example;
  T=256 tokens, the rank owns 32 of the 256 experts; bf16.
* ``prefill`` DeepSeek-V3-like shape (H=7168, I=2048, E=256, k=8, one shared
  expert) from the infra-guide page, section 2.1; T=8192; bf16.
* ``skewed``  ``prefill`` plus a per-expert logit bias ln(1/(rank+1)^1.2) over a
  seeded permutation of the experts (a Zipf popularity law, the same shape of
  skew as the power-law load simulation of the infra-guide page, section 5.2).
* ``fp8``     DeepSeek-V3 shape, T=4096, no shared expert; fp32 master weights
  that each side quantises to OCP E4M3 with one fp32 scale per 128x128 block.
* ``decode_skewed`` ``decode`` plus the Zipf s=1.2 logit bias of ``skewed``:
  a decode batch in which one local expert holds several times the mean
  rows (51-166 of 138-275 local rows over four seeds).
* ``lowlat``  the low-latency decode setting of DeepEP's low-latency kernels as
  the infra-guide page, section 6.1, gives it: 128 tokens a batch, hidden 7168,
  top-8, FP8 dispatch (activations in E4M3 per token per 128 channels) and
  BF16 combine; the expert is DeepSeek-V3's (I=2048, 256 experts, 32 local),
  weights as in ``fp8``.
* ``lowlat_skewed`` ``lowlat`` plus the Zipf s=1.2 logit bias of ``skewed``:
  an FP8 decode batch in which one local expert holds most of the local rows.

Stored layouts (row-major):
* ``logits`` [T, E] float32, ``bias`` [E] float32 or None;
* ``x`` [T, H]: float32 for fp32 workloads, else bf16 bit patterns (uint16);
* per expert ``wg``, ``wu`` [H, I] and ``wd`` [I, H]: the gate/up and down
  matrices in their logical layout (h = silu(x Wg) * (x Wu), y = h Wd), float32
  or bf16 bit patterns.

Normals are drawn in float32 with numpy's PCG64 generator seeded by
``[seed, workload id, tensor id, index]``, then rounded to nearest-even bf16
by integer operations where the workload is bf16.  Those rounded values are
the inputs for every consumer.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

# workload id is part of every seed so two workloads never share a stream
CONFIGS: Dict[str, dict] = {
    "tiny": dict(wid=1, T=128, H=256, I=128, E=8, k=2, expert_begin=0,
                 num_local=8, shared=False, act="f32", wdt="f32", out="f32",
                 bias=None),
    "decode": dict(wid=2, T=256, H=6144, I=2048, E=256, k=8, expert_begin=0,
                   num_local=32, shared=False, act="bf16", wdt="bf16",
                   out="bf16", bias=None),
    "prefill": dict(wid=3, T=8192, H=7168, I=2048, E=256, k=8,
                    expert_begin=0, num_local=32, shared=True, act="bf16",
                    wdt="bf16", out="bf16", bias=None),
    "skewed": dict(wid=4, T=8192, H=7168, I=2048, E=256, k=8,
                   expert_begin=0, num_local=32, shared=True, act="bf16",
                   wdt="bf16", out="bf16", bias="zipf", zipf_s=1.2,
                   redundant=8),
    "fp8": dict(wid=5, T=4096, H=7168, I=2048, E=256, k=8, expert_begin=0,
                num_local=32, shared=False, act="bf16", wdt="fp8", out="bf16",
                bias=None, quant_block=128),
    "lowlat": dict(wid=6, T=128, H=7168, I=2048, E=256, k=8, expert_begin=0,
                   num_local=32, shared=False, act="bf16", wdt="fp8",
                   out="bf16", bias=None, quant_block=128),
    "decode_skewed": dict(wid=7, T=256, H=6144, I=2048, E=256, k=8,
                          expert_begin=0, num_local=32, shared=False,
                          act="bf16", wdt="bf16", out="bf16", bias="zipf",
                          zipf_s=1.2),
    "lowlat_skewed": dict(wid=8, T=128, H=7168, I=2048, E=256, k=8,
                          expert_begin=0, num_local=32, shared=False,
                          act="bf16", wdt="fp8", out="bf16", bias="zipf",
                          zipf_s=1.2, quant_block=128),
}

_TENSOR_LOGITS, _TENSOR_X, _TENSOR_W, _TENSOR_SHARED, _TENSOR_PERM = 1, 2, 3, 4, 5
WEIGHT_STD = 0.02


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); return the bits.

    Finite inputs only (the generators draw normals)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Workload:
    name: str
    T: int
    H: int
    I: int
    E: int
    k: int
    expert_begin: int
    num_local: int
    shared: bool
    act: str
    wdt: str
    out: str
    seed: int
    wid: int
    bias_kind: Optional[str] = None
    zipf_s: float = 1.2
    redundant: int = 0
    quant_block: int = 128
    _experts: Dict[int, dict] = dataclasses.field(default_factory=dict,
                                                  repr=False)
    _cache: Dict[str, object] = dataclasses.field(default_factory=dict,
                                                  repr=False)

    # ---------------------------------------------------------------- rng
    def _rng(self, tensor: int, index: int = 0) -> np.random.Generator:
        return np.random.default_rng([self.seed, self.wid, tensor, index])

    def _normal(self, rng, shape, std=1.0) -> np.ndarray:
        a = rng.standard_normal(int(np.prod(shape)), dtype=np.float32)
        if std != 1.0:
            a *= np.float32(std)
        return a.reshape(shape)

    def _store(self, a: np.ndarray, fmt: str) -> np.ndarray:
        if fmt == "bf16":
            return bf16_bits_from_f32(a)
        return np.ascontiguousarray(a, dtype=np.float32)

    # ------------------------------------------------------------ tensors
    @property
    def logits(self) -> np.ndarray:
        if "logits" not in self._cache:
            self._cache["logits"] = self._normal(self._rng(_TENSOR_LOGITS),
                                                 (self.T, self.E))
        return self._cache["logits"]

    @property
    def bias(self) -> Optional[np.ndarray]:
        """Per-expert logit bias, or None.  ``zipf``: ln of the popularity
        1/(rank+1)^s, rank being a seeded permutation of the expert ids."""
        if self.bias_kind is None:
            return None
        if "bias" not in self._cache:
            rank = self._rng(_TENSOR_PERM).permutation(self.E)
            b = -self.zipf_s * np.log(rank.astype(np.float64) + 1.0)
            self._cache["bias"] = b.astype(np.float32)
        return self._cache["bias"]

    @property
    def x(self) -> np.ndarray:
        if "x" not in self._cache:
            self._cache["x"] = self._store(
                self._normal(self._rng(_TENSOR_X), (self.T, self.H)),
                "bf16" if self.act == "bf16" else "f32")
        return self._cache["x"]

    def _weights(self, tensor: int, index: int) -> dict:
        rng = self._rng(tensor, index)
        fmt = "bf16" if self.wdt == "bf16" else "f32"
        wg = self._store(self._normal(rng, (self.H, self.I), WEIGHT_STD), fmt)
        wu = self._store(self._normal(rng, (self.H, self.I), WEIGHT_STD), fmt)
        wd = self._store(self._normal(rng, (self.I, self.H), WEIGHT_STD), fmt)
        return dict(wg=wg, wu=wu, wd=wd)

    def expert(self, e_local: int) -> dict:
        """Weights of local logical expert ``e_local`` (global id
        expert_begin + e_local): dict(wg [H,I], wu [H,I], wd [I,H])."""
        if not 0 <= e_local < self.num_local:
            raise IndexError(e_local)
        if e_local not in self._experts:
            self._experts[e_local] = self._weights(
                _TENSOR_W, self.expert_begin + e_local)
        return self._experts[e_local]

    def drop_expert(self, e_local: int) -> None:
        self._experts.pop(e_local, None)

    @property
    def shared_expert(self) -> Optional[dict]:
        if not self.shared:
            return None
        if "shared" not in self._cache:
            self._cache["shared"] = self._weights(_TENSOR_SHARED, 0)
        return self._cache["shared"]

    def x_f32(self) -> np.ndarray:
        """The activations as exact float32 values."""
        return bf16_bits_to_f32(self.x) if self.act == "bf16" else self.x

    def describe(self) -> str:
        return (f"{self.name}: T={self.T} H={self.H} I={self.I} E={self.E} "
                f"k={self.k} local=[{self.expert_begin},"
                f"{self.expert_begin + self.num_local}) shared={self.shared} "
                f"act={self.act} w={self.wdt} out={self.out} seed={self.seed}")


def make_workload(name: str, seed: int = 0, **overrides) -> Workload:
    """Build a workload by name; keyword overrides shrink or reshape it (the
    parity tests use reduced T/H/I that still span several tiles)."""
    if name not in CONFIGS:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(CONFIGS)}")
    c = dict(CONFIGS[name])
    c.update(overrides)
    return Workload(name=name, T=c["T"], H=c["H"], I=c["I"], E=c["E"],
                    k=c["k"], expert_begin=c["expert_begin"],
                    num_local=c["num_local"], shared=c["shared"],
                    act=c["act"], wdt=c["wdt"], out=c["out"], seed=seed,
                    wid=c["wid"], bias_kind=c.get("bias"),
                    zipf_s=c.get("zipf_s", 1.2),
                    redundant=c.get("redundant", 0),
                    quant_block=c.get("quant_block", 128))


def all_expert_weights(w: Workload) -> List[dict]:
    return [w.expert(e) for e in range(w.num_local)]
