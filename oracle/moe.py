"""Float64 oracle of the expert-parallel MoE layer on one EP rank's share.

What it follows (pages as titled in the reference text):
* "6.4 Data parallelism and expert parallelism" (infra-guide), section 3.1: the
  four steps of an MoE layer -- route each token to its top-k experts and
  weights; dispatch a copy of the token to the owner of each chosen expert;
  run the experts on the tokens they received; combine the results at the
  token's home, weighted by the route weights.  Section 2.1: an expert is three
  matrices gate, up, down; one shared expert per layer serves every token.
* "Expert Parallel and All-to-All Backends" (aiinfrainterviews), "Why expert
  parallelism exists": each GPU holds whole experts and works only on the
  tokens that selected them; on one GPU the all-to-all becomes a local
  permutation into expert-contiguous order and its inverse.
* "How Expert Parallelism Works for Mixture-of-Experts Models in vLLM"
  (instagit), "MoE Layer Construction": physical experts = logical experts +
  redundant replicas; a logical-to-physical map sends a logical expert's tokens
  to its replicas.

Readings where the pages are silent (each listed in the design notes):
* gating: softmax over all E logits, keep the top k, renormalise the k weights
  to sum to 1 (equal to a softmax over the k selected logits);
* selection is on the float32 logits (plus bias), descending, lower expert id
  first on equal values (+0.0 and -0.0 are equal);
* the expert activation is SwiGLU: h = silu(x Wg) * (x Wu), silu(z) = z/(1+e^-z),
  y = h Wd; no biases;
* a logical expert's n-th local pair in token order goes to replica n mod R at
  position floor(n / R) of that replica's segment; segments are laid out in
  physical-id order and are token-ordered inside;
* h is rounded to the activation format before the down projection (bf16, or
  E4M3 with per-row-per-128 scales, or float32); everything else is exact;
* the shared expert's output is added with weight 1; tokens with no local pair
  and no shared expert produce zero rows.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np

from . import fp8 as _fp8


# ----------------------------------------------------------------- formats
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact float64 (bf16 is the top half of float32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def round_to_bf16(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (8 significant bits,
    ties to even), returned as float64.  Normal range only (|v| > 2^-126)."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)                    # v = m 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0), e - 8)


def round_to_f32(v: np.ndarray) -> np.ndarray:
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def to_f64(a: np.ndarray, fmt: str) -> np.ndarray:
    if fmt == "bf16":
        return bf16_to_f64(a)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


# ----------------------------------------------------------------- routing
def route_topk(logits: np.ndarray, k: int, bias: Optional[np.ndarray] = None):
    """Top-k routing of each token (infra-guide page, section 3.1, step 1).

    logits [T, E] float32; bias [E] float32 or None, added in float32.
    Returns ids [T, k] int32 (slot j = j-th largest score, lower id first on
    ties), weights [T, k] float64 (softmax over E renormalised over the k
    selected = exp(l_j - l_0) / sum_i exp(l_i - l_0)), counts [E] int64 (number
    of (token, slot) pairs per expert over all E)."""
    l32 = np.asarray(logits, dtype=np.float32)
    if bias is not None:
        l32 = (l32 + np.asarray(bias, dtype=np.float32)[None, :]).astype(
            np.float32)
    T, E = l32.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    # a stable sort of the negated scores keeps equal scores in id order;
    # -0.0 and +0.0 compare equal, so they tie as well
    order = np.argsort(-l32, axis=1, kind="stable")
    ids = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(l32, ids, axis=1).astype(np.float64)
    ex = np.exp(sel - sel[:, :1])
    w = ex / ex.sum(axis=1, keepdims=True)
    counts = np.bincount(ids.ravel(), minlength=E).astype(np.int64)
    return ids, w, counts


# ---------------------------------------------------------------- dispatch
@dataclasses.dataclass
class Dispatch:
    offsets: np.ndarray      # [P+1] int64, exclusive scan of physical counts
    phys_counts: np.ndarray  # [P]
    row_token: np.ndarray    # [N] token of each permuted row
    row_slot: np.ndarray     # [N] slot j of each permuted row
    row_phys: np.ndarray     # [N] physical expert of each permuted row
    pair_row: np.ndarray     # [T, k] row of each local pair, -1 otherwise
    logical_counts: np.ndarray  # [num_local] local pairs per logical expert

    @property
    def N(self) -> int:
        return int(self.offsets[-1])


def identity_map(num_local: int):
    """Logical-to-physical map with one replica per expert (P = num_local)."""
    l2p = np.arange(num_local, dtype=np.int32)[:, None]
    return l2p, np.ones(num_local, dtype=np.int32)


def dispatch(ids: np.ndarray, expert_begin: int, num_local: int,
             l2p: np.ndarray, rep_count: np.ndarray, P: int) -> Dispatch:
    """Local share, replica remap and expert-contiguous permutation.

    A pair (t, j) is local when ids[t, j] lies in [expert_begin,
    expert_begin + num_local).  Walking pairs in token order (t ascending; a
    token picks an expert at most once), the n-th pair of local logical expert
    e goes to physical expert l2p[e, n mod R_e] at position floor(n / R_e) of
    that physical expert's segment.  Segments are concatenated in physical-id
    order.

    Under a placement spread over several ranks (section 5.2 of the
    infra-guide page: replicas of one expert may sit on different cards) an
    entry l2p[e, r] = -1 says that replica r of e lives on another rank: the
    pair still counts in e's n, but it is not local here (pair_row -1)."""
    T, k = ids.shape
    rep_count = np.asarray(rep_count)
    n_seen = np.zeros(num_local, dtype=np.int64)
    pair_phys = np.full((T, k), -1, dtype=np.int64)
    pair_pos = np.full((T, k), -1, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j]) - expert_begin
            if 0 <= e < num_local:
                n = n_seen[e]
                n_seen[e] += 1
                R = int(rep_count[e])
                p = int(l2p[e, n % R])
                if p == -1:                 # that replica is on another rank
                    continue
                if not 0 <= p < P:
                    raise ValueError("physical id out of range")
                pair_phys[t, j] = p
                pair_pos[t, j] = n // R
    local = pair_phys >= 0
    phys_counts = np.bincount(pair_phys[local], minlength=P).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(phys_counts)]).astype(np.int64)
    N = int(offsets[-1])
    row_token = np.full(N, -1, dtype=np.int64)
    row_slot = np.full(N, -1, dtype=np.int64)
    row_phys = np.full(N, -1, dtype=np.int64)
    pair_row = np.full((T, k), -1, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            p = pair_phys[t, j]
            if p >= 0:
                r = offsets[p] + pair_pos[t, j]
                if row_token[r] != -1:
                    raise AssertionError("two pairs mapped to one row")
                row_token[r], row_slot[r], row_phys[r] = t, j, p
                pair_row[t, j] = r
    return Dispatch(offsets=offsets, phys_counts=phys_counts,
                    row_token=row_token, row_slot=row_slot, row_phys=row_phys,
                    pair_row=pair_row, logical_counts=n_seen)


# ------------------------------------------------------------------ experts
def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def swiglu(x64: np.ndarray, wg64: np.ndarray, wu64: np.ndarray,
           wd64: np.ndarray, h_round) -> np.ndarray:
    """One expert on the rows of x64 [n, H]: y = round(silu(x Wg) * (x Wu)) Wd,
    with Wg, Wu the H x I matrices and Wd the I x H matrix."""
    g = x64 @ wg64
    u = x64 @ wu64
    h = h_round(silu(g) * u)
    return h @ wd64


# ------------------------- what a correct evaluation of h may differ by (FP8)
U32 = 2.0 ** -24           # unit roundoff of float32
LAMBDA = 4.0               # model standard deviations the bound allows
# The FP8 recipe sums each 128-channel scale block's products as one unit
# (the per-block scales apply to that sum).  gfx950's FP8 matrix instruction
# returns such a 128-product sum with an error that is not float32 rounding
# (only 11 % of the sums come back correctly rounded): mean-zero, with a root
# mean square of 34 u * sum|p| over the block for normal-distributed codes
# and 85 for the down projection's h codes times weight codes (measured
# through the library; tests/test_gpu_fp8.py checks it stays within the
# model).  The model takes 128, so LAMBDA = 4 model deviations is 15 of the
# gate/up data's own.
C_BLOCK = 128.0


def h_eval_bound(x64: np.ndarray, wg64: np.ndarray, wu64: np.ndarray,
                 g: np.ndarray, u: np.ndarray, block: int = 128) -> np.ndarray:
    """Bound on |h_eval - h| for h = silu(x Wg) * (x Wu) evaluated by the FP8
    recipe: each 128-product block sum S_b = sum_{k in b} x_k w_k comes back
    with a mean-zero error of RMS at most C_BLOCK u sum_{k in b} |x_k w_k|,
    independent between blocks, so the errors of g's blocks add like a random
    walk: RMS C_BLOCK u sqrt(sum_b (sum_{k in b} |p_k|)^2); the bound takes
    LAMBDA of those.  The scaled block sums are then multiplied by two scales
    and added in float32 (round to nearest: at most (K/128 + 2) u sum|p|).
    silu(z) = z / (1 + exp(-z)): |silu'| <= 1.1, and its float32 evaluation
    (the exponent's argument rounded, exp to within 2 ulp, one add, one
    divide) has relative error below (|z| + 6) u; the bound takes twice that.
    The product silu(g) * u adds one rounding."""
    K = x64.shape[1]
    nb = K // block
    ax = np.abs(x64)

    def bound(w64):
        aw = np.abs(w64)
        sq = np.zeros((x64.shape[0], w64.shape[1]))
        for b in range(nb):
            sb = ax[:, b * block:(b + 1) * block] @ aw[b * block:(b + 1) * block]
            sq += sb * sb
        return (LAMBDA * C_BLOCK * U32 * np.sqrt(sq) +
                (nb + 2) * U32 * (ax @ aw))

    eg, eu = bound(wg64), bound(wu64)
    sg = silu(g)
    es = 1.1 * eg + 2.0 * (np.abs(g) + 6.0) * U32 * np.abs(sg)
    h = sg * u
    return np.abs(u) * es + np.abs(sg) * eu + es * eu + U32 * np.abs(h)


@dataclasses.dataclass
class Fp8Rows:
    """Per routed (or shared) row of the FP8 recipe: the exact h, the
    interval of scales and E4M3 code values a correct evaluation may produce
    for it (a value near a rounding boundary has two correct codes), and the
    largest change of the dequantised h that choice allows."""
    h: np.ndarray            # [n, I] float64, exact silu(x Wg) * (x Wu)
    s_lo: np.ndarray         # [n, I/128] float32
    s_hi: np.ndarray
    v_lo: np.ndarray         # [n, I] float64 code values
    v_hi: np.ndarray
    allow: np.ndarray        # [n, I] max |dequantised h - oracle's own|


def fp8_rows_detail(x64, wg64, wu64, block: int = 128):
    """h, its code and scale intervals, and the oracle's own rounding of it
    (for ``Fp8Rows`` and the down projection)."""
    g = x64 @ wg64
    u = x64 @ wu64
    h = silu(g) * u
    eps = h_eval_bound(x64, wg64, wu64, g, u, block)
    s_lo, s_hi = _fp8.row_scale_interval(h, eps, block)
    v_lo, v_hi = _fp8.row_code_interval(h, eps, s_lo, s_hi, block)
    slo = np.repeat(s_lo.astype(np.float64), block, axis=1)
    shi = np.repeat(s_hi.astype(np.float64), block, axis=1)
    d_lo = np.minimum(v_lo * slo, v_lo * shi)
    d_hi = np.maximum(v_hi * slo, v_hi * shi)
    own = h_rounder("fp8", "bf16", block)(h)
    allow = np.maximum(d_hi - own, own - d_lo)
    return Fp8Rows(h=h, s_lo=s_lo, s_hi=s_hi, v_lo=v_lo, v_hi=v_hi,
                   allow=allow), own


@dataclasses.dataclass
class ExpertSet:
    """Expert weights in float64, as the layer consumes them.

    ``fmt`` is the activation/weight recipe: "f32", "bf16" or "fp8".  For fp8,
    weights are the exact values of the block-quantised codes.  Either
    ``experts`` holds (wg, wu, wd) per local logical expert, or ``loader(e)``
    produces them on demand (large workloads: one expert at a time)."""
    fmt: str
    experts: Optional[List[tuple]] = None
    shared: Optional[tuple] = None
    quant_block: int = 128
    loader: Optional[object] = None
    shared_loader: Optional[object] = None
    # the workload the weights come from (a copy without cached tensors), so
    # worker threads can make an expert's weights themselves
    source: Optional[object] = None

    def get(self, e: int) -> tuple:
        if self.experts is not None:
            return self.experts[e]
        return self.loader(e)

    def get_shared(self) -> Optional[tuple]:
        if self.shared is not None or self.shared_loader is None:
            return self.shared
        return self.shared_loader()

    @property
    def has_shared(self) -> bool:
        return self.shared is not None or self.shared_loader is not None


def expert_set_from_workload(w, experts: Optional[Sequence[int]] = None,
                             lazy: bool = False) -> ExpertSet:
    """Convert a synthetic workload's stored weights to float64; fp8
    workloads are block-quantised here, by the oracle's own quantiser.  With
    ``lazy`` nothing is converted until an expert is used."""
    conv = _weight_converter(w.wdt, w.quant_block)

    def load(e):
        d = w.expert(e)
        return conv(d["wg"]), conv(d["wu"]), conv(d["wd"])

    def load_shared():
        d = w.shared_expert
        return conv(d["wg"]), conv(d["wu"]), conv(d["wd"])

    source = dataclasses.replace(w, _experts={}, _cache={})
    if lazy:
        return ExpertSet(fmt=w.wdt, quant_block=w.quant_block, loader=load,
                         shared_loader=load_shared if w.shared else None,
                         source=source)
    idx = range(w.num_local) if experts is None else experts
    ex = [None] * w.num_local
    for e in idx:
        ex[e] = load(e)
    sh = load_shared() if w.shared else None
    return ExpertSet(fmt=w.wdt, experts=ex, shared=sh,
                     quant_block=w.quant_block, source=source)


def _weight_converter(wdt: str, block: int):
    if wdt == "fp8":
        def conv(a):
            codes, s = _fp8.quantize_blocks_2d(a, block)
            return _fp8.dequantize_blocks_2d(codes, s, block)
        return conv
    return lambda a: to_f64(a, wdt)


def activation_rows(x_stored: np.ndarray, act: str, wdt: str,
                    block: int = 128) -> np.ndarray:
    """Values of the token rows the experts multiply: exact inputs, or their
    per-token per-128-channel E4M3 quantisation when the weights are fp8."""
    x64 = to_f64(x_stored, act)
    if wdt == "fp8":
        codes, s = _fp8.quantize_rows(x64.astype(np.float32), block)
        return _fp8.dequantize_rows(codes, s, block)
    return x64


def h_rounder(wdt: str, act: str, block: int = 128):
    """Rounding of the intermediate h before the down projection."""
    if wdt == "fp8":
        def q(h):
            codes, s = _fp8.quantize_rows(h.astype(np.float32), block)
            return _fp8.dequantize_rows(codes, s, block)
        return q
    if act == "bf16":
        return round_to_bf16
    return round_to_f32


# ------------------------------------------------------------------ combine
def combine(y_rows: np.ndarray, pair_row: np.ndarray, w: np.ndarray,
            shared_out: Optional[np.ndarray], T: int, H: int) -> np.ndarray:
    """out[t] = sum over slots j (ascending) with a local row of
    w[t, j] * y[pair_row[t, j]], plus the shared expert's output
    (infra-guide page, section 3.1, step 4)."""
    out = np.zeros((T, H), dtype=np.float64)
    k = pair_row.shape[1]
    for j in range(k):
        r = pair_row[:, j]
        m = r >= 0
        out[m] += w[m, j][:, None] * y_rows[r[m]]
    if shared_out is not None:
        out += shared_out
    return out


# ------------------------------------------------------------ whole layer
@dataclasses.dataclass
class LayerResult:
    ids: np.ndarray
    weights: np.ndarray
    counts: np.ndarray
    disp: Dispatch
    y_rows: np.ndarray
    shared_out: Optional[np.ndarray]
    out: np.ndarray
    # FP8 recipe with fp8_detail: per routed row (permuted order) and per
    # shared row, the h intervals; out_allow [T, H] bounds how far a correct
    # choice among the alternative h codes moves each output element
    fp8_routed: Optional[Fp8Rows] = None
    fp8_shared: Optional[Fp8Rows] = None
    out_allow: Optional[np.ndarray] = None


def _eval_expert(weights, xrs, fmt: str, act: str, block: int,
                 detail: bool):
    """One expert on each of the row sets ``xrs``: per set (y, allowance or
    None, Fp8Rows or None)."""
    wg, wu, wd = weights
    out = []
    for xr in xrs:
        if detail:
            det, hq = fp8_rows_detail(xr, wg, wu, block)
            out.append((hq @ wd, det.allow @ np.abs(wd), det))
        else:
            out.append((swiglu(xr, wg, wu, wd, h_rounder(fmt, act, block)),
                        None, None))
    return out


def _expert_job(source, e: int, xrs, act: str, detail: bool):
    """One expert's evaluation from the workload alone: its weights are made
    from the workload's generator (expert -1 is the shared one)."""
    conv = _weight_converter(source.wdt, source.quant_block)
    d = source.expert(e) if e >= 0 else source.shared_expert
    weights = (conv(d["wg"]), conv(d["wu"]), conv(d["wd"]))
    return _eval_expert(weights, xrs, source.wdt, act, source.quant_block,
                        detail)


def _run_experts(jobs, experts: "ExpertSet", act: str, detail: bool,
                 workers: int):
    """Evaluate (expert, row sets) jobs in order; with ``workers`` > 1 and a
    workload behind the expert set, on that many threads (NumPy releases the
    interpreter lock in its array loops; the same arithmetic, one expert per
    thread at a time)."""
    if workers > 1 and experts.source is not None and len(jobs) > 1:
        import concurrent.futures as cf
        with cf.ThreadPoolExecutor(max_workers=min(workers, len(jobs))) as pool:
            futs = [pool.submit(_expert_job, experts.source, e, xrs, act,
                                detail) for e, _, xrs in jobs]
            for (e, parts, _), f in zip(jobs, futs):
                yield e, parts, f.result()
        return
    for e, parts, xrs in jobs:
        weights = experts.get(e) if e >= 0 else experts.get_shared()
        res = _eval_expert(weights, xrs, experts.fmt, act,
                           experts.quant_block, detail)
        del weights
        yield e, parts, res


def layer_forward(logits, bias, x_stored, act: str, k: int, expert_begin: int,
                  num_local: int, experts: ExpertSet, l2p=None, rep_count=None,
                  P: Optional[int] = None, token_subset=None,
                  fp8_detail: bool = False, workers: int = 0) -> LayerResult:
    """The whole layer: route -> dispatch -> experts -> combine.

    ``experts.experts[e]`` are the weights of local logical expert e; all
    replicas of e compute with the same weights.  ``token_subset`` (optional)
    restricts the expert evaluation and the output to those tokens, for
    spot checks of large workloads (routing and dispatch still cover all).
    ``fp8_detail`` (FP8 recipe) also records, for every evaluated row, the
    codes and scales a correct float32 evaluation of h may give
    (``fp8_rows_detail``) and the resulting allowance on the output.
    ``workers`` > 1 evaluates the experts on that many threads (expert sets
    made by ``expert_set_from_workload`` only)."""
    ids, w, counts = route_topk(logits, k, bias)
    if l2p is None:
        l2p, rep_count = identity_map(num_local)
        P = num_local
    d = dispatch(ids, expert_begin, num_local, l2p, rep_count, P)
    T = ids.shape[0]
    H = x_stored.shape[1]
    # logical expert of each physical id
    phys_to_logical = np.full(P, -1, dtype=np.int64)
    for e in range(num_local):
        for r in range(int(rep_count[e])):
            if l2p[e, r] != -1:          # -1: that replica is on another rank
                phys_to_logical[l2p[e, r]] = e
    x_rows = activation_rows(x_stored, act, experts.fmt, experts.quant_block)
    hr = h_rounder(experts.fmt, act, experts.quant_block)
    want = np.ones(T, dtype=bool)
    if token_subset is not None:
        want = np.zeros(T, dtype=bool)
        want[np.asarray(token_subset)] = True
    detail = fp8_detail and experts.fmt == "fp8"
    y_rows = np.zeros((d.N, H), dtype=np.float64)
    y_allow = np.zeros((d.N, H), dtype=np.float64) if detail else None
    rows_detail = {}
    by_expert = {}
    for p in range(P):
        lo, hi = int(d.offsets[p]), int(d.offsets[p + 1])
        if hi == lo:
            continue
        rows = np.arange(lo, hi)
        rows = rows[want[d.row_token[rows]]]
        if rows.size == 0:
            continue
        by_expert.setdefault(int(phys_to_logical[p]), []).append(rows)
    # every logical expert's rows (and the shared expert's, as expert -1)
    jobs = [(e, parts, [x_rows[d.row_token[r]] for r in parts])
            for e, parts in sorted(by_expert.items())]
    if experts.has_shared:
        jobs.append((-1, [np.flatnonzero(want)], [x_rows[want]]))
    shared_out = shared_det = shared_allow = None
    for e, parts, results in _run_experts(jobs, experts, act, detail,
                                          workers):
        if e < 0:
            shared_out = np.zeros((T, H), dtype=np.float64)
            y, allow, shared_det = results[0]
            shared_out[want] = y
            if detail:
                shared_allow = np.zeros((T, H), dtype=np.float64)
                shared_allow[want] = allow
            continue
        for rows, (y, allow, det) in zip(parts, results):
            y_rows[rows] = y
            if detail:
                y_allow[rows] = allow
                rows_detail[tuple(rows[[0, -1]])] = (rows, det)
    pr = d.pair_row.copy()
    pr[~want] = -1
    out = combine(y_rows, pr, w, shared_out, T, H)
    res = LayerResult(ids=ids, weights=w, counts=counts, disp=d,
                      y_rows=y_rows, shared_out=shared_out, out=out)
    if detail:
        # the allowance adds up like the output: |w| times each row's own
        res.out_allow = combine(y_allow, pr, np.abs(w), shared_allow, T, H)
        res.fp8_routed = _gather_rows_detail(rows_detail, d.N)
        res.fp8_shared = shared_det
    return res


def _gather_rows_detail(parts: dict, n_rows: int) -> Fp8Rows:
    """Per-expert pieces of ``Fp8Rows`` placed at their permuted rows (rows
    that were not evaluated stay NaN)."""
    first = next(iter(parts.values()))[1] if parts else None
    if first is None:
        return None
    I_ = first.h.shape[1]
    G = first.s_lo.shape[1]
    out = Fp8Rows(h=np.full((n_rows, I_), np.nan),
                  s_lo=np.full((n_rows, G), np.nan, dtype=np.float32),
                  s_hi=np.full((n_rows, G), np.nan, dtype=np.float32),
                  v_lo=np.full((n_rows, I_), np.nan),
                  v_hi=np.full((n_rows, I_), np.nan),
                  allow=np.full((n_rows, I_), np.nan))
    for rows, det in parts.values():
        for f in ("h", "s_lo", "s_hi", "v_lo", "v_hi", "allow"):
            getattr(out, f)[rows] = getattr(det, f)
    return out


def layer_from_workload(wl, experts: Optional[ExpertSet] = None,
                        l2p=None, rep_count=None, P=None,
                        token_subset=None, fp8_detail=False,
                        workers: int = 0) -> LayerResult:
    if experts is None:
        experts = expert_set_from_workload(wl, lazy=workers > 1)
    return layer_forward(wl.logits, wl.bias, wl.x, wl.act, wl.k,
                         wl.expert_begin, wl.num_local, experts, l2p,
                         rep_count, P, token_subset, fp8_detail, workers)


# ------------------------------------------------------ dense brute force
def dense_masked_forward(logits, bias, x_stored, act: str, k: int,
                         expert_begin: int, num_local: int,
                         experts: ExpertSet) -> np.ndarray:
    """Independent evaluation for tiny inputs: every local expert runs on
    every token, and a routing mask picks the contributions.

    Selection scans the E scores of each token k times in pure Python,
    keeping the first maximum (so the lower id wins a tie); the weights are
    the softmax over all E probabilities of the selected experts divided by
    their sum.  No permutation, histogram or scan is involved."""
    l32 = np.asarray(logits, dtype=np.float32)
    if bias is not None:
        l32 = (l32 + np.asarray(bias, dtype=np.float32)[None, :]).astype(
            np.float32)
    T, E = l32.shape
    x_rows = activation_rows(x_stored, act, experts.fmt, experts.quant_block)
    hr = h_rounder(experts.fmt, act, experts.quant_block)
    H = x_rows.shape[1]
    gate = np.zeros((T, E), dtype=np.float64)
    for t in range(T):
        row = [float(v) for v in l32[t]]
        mx = max(row)
        p = np.array([np.exp(v - mx) for v in row])
        p = p / p.sum()
        taken: List[int] = []
        for _ in range(k):
            best = -1
            for e in range(E):
                if e in taken:
                    continue
                if best < 0 or row[e] > row[best]:
                    best = e
            taken.append(best)
        tot = sum(p[e] for e in taken)
        for e in taken:
            gate[t, e] = p[e] / tot
    out = np.zeros((T, H), dtype=np.float64)
    for e_loc in range(num_local):
        wg, wu, wd = experts.get(e_loc)
        y_all = swiglu(x_rows, wg, wu, wd, hr)
        out += gate[:, expert_begin + e_loc][:, None] * y_all
    if experts.has_shared:
        wg, wu, wd = experts.get_shared()
        out += swiglu(x_rows, wg, wu, wd, hr)
    return out


# ------------------------------------------------------------- tolerances
def bf16_half_ulp(v: np.ndarray) -> np.ndarray:
    """Half a bf16 unit in the last place at |v| (the largest error of a
    correct rounding of v to bf16)."""
    v = np.abs(np.asarray(v, dtype=np.float64))
    _, e = np.frexp(np.where(v == 0, 1.0, v))
    return np.where(v == 0, 0.0, np.ldexp(1.0, e - 9))


def f32_half_ulp(v: np.ndarray) -> np.ndarray:
    v = np.abs(np.asarray(v, dtype=np.float64))
    _, e = np.frexp(np.where(v == 0, 1.0, v))
    return np.where(v == 0, 0.0, np.ldexp(1.0, e - 25))
