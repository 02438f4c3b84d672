"""ctypes binding of libmoe.so (include/moe.h).

Argument marshalling only: every function here forwards to the C entry point
of the same name, passing device pointers of torch tensors and the current
HIP stream.  All arithmetic happens in the library's HIP kernels.  Importing
this module on a machine without the built library raises immediately; there
is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARGUMENT, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, \
    MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16, MOE_FP8_E4M3 = range(3)
DTYPES = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8": MOE_FP8_E4M3}

MOE_LAYOUT_KN, MOE_LAYOUT_NK = range(2)
LAYOUTS = {"kn": MOE_LAYOUT_KN, "nk": MOE_LAYOUT_NK}

EXPORTS = (
    "moe_status_string", "moe_check_problem", "moe_workspace_size",
    "moe_dispatch_workspace_size",
    "moe_ffn_workspace_size", "moe_layer_workspace_size", "moe_route_topk",
    "moe_dispatch", "moe_grouped_ffn", "moe_ffn_intermediate", "moe_combine",
    "moe_layer_forward", "moe_layer_forward_timed",
    "moe_layer_forward_noalloc", "moe_prepack_weights",
    "moe_quantize_fp8_blocks",
    "moe_eplb_hottest_map", "moe_eplb_plan", "moe_eplb_rank_map",
    "moe_eplb_record_load",
)
MOE_STAGE_EVENTS = 8
STAGES = ("route", "dispatch_index", "gather", "tiles", "gate_up", "down",
          "combine")


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class Problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "T", "H", "I", "E", "k", "expert_begin", "num_local", "num_physical",
        "max_replicas", "has_shared", "act_dtype", "weight_dtype",
        "out_dtype", "quant_block")]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down", "sh_gate",
        "sh_up", "sh_down", "sh_s_gate", "sh_s_up", "sh_s_down")]


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load libmoe.so (built by expert_moe_fp32_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m expert_moe_fp32_amd.build` (hipcc, gfx950)")
        # torch brings its own HIP runtime (same soname as the system one the
        # library links against); loading it first makes the library bind to
        # that one copy, so the process holds a single HIP runtime whatever
        # the order of first use
        try:
            import torch  # noqa: F401
        except ImportError:  # pragma: no cover - the binding needs torch
            pass
        L = ctypes.CDLL(LIB_PATH)
        P, V, S, I32 = (ctypes.POINTER(Problem), ctypes.c_void_p,
                        ctypes.c_size_t, ctypes.c_int32)
        sig = {
            "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
            "moe_check_problem": (ctypes.c_int, [P]),
            "moe_workspace_size": (ctypes.c_int, [P, ctypes.POINTER(S)]),
            "moe_dispatch_workspace_size": (ctypes.c_int, [P, ctypes.POINTER(S)]),
            "moe_ffn_workspace_size": (ctypes.c_int, [P, ctypes.POINTER(S)]),
            "moe_layer_workspace_size": (ctypes.c_int, [P, ctypes.POINTER(S)]),
            "moe_route_topk": (ctypes.c_int, [P, V, V, V, V, V, V]),
            "moe_dispatch": (ctypes.c_int, [P, V, V, V, V, V, V, V, V, V, V,
                                            V, V, S, V]),
            "moe_grouped_ffn": (ctypes.c_int, [P, V, V, V, V, V,
                                               ctypes.POINTER(Weights), V, V,
                                               V, S, V]),
            "moe_ffn_intermediate": (ctypes.c_int, [
                P, V, S, ctypes.POINTER(V), ctypes.POINTER(V)]),
            "moe_combine": (ctypes.c_int, [P, V, V, V, V, V, V]),
            "moe_layer_forward": (ctypes.c_int, [P, V, V, V,
                                                 ctypes.POINTER(Weights), V, V,
                                                 V, V, V, S, V]),
            "moe_layer_forward_timed": (ctypes.c_int, [P, V, V, V,
                                                       ctypes.POINTER(Weights),
                                                       V, V, V, V, V, S, V,
                                                       V]),
            "moe_layer_forward_noalloc": (ctypes.c_int, [
                P, V, V, V, ctypes.POINTER(Weights), V, V, V, V, V]),
            "moe_prepack_weights": (ctypes.c_int, [V, I32, I32, I32, I32, V,
                                                   V]),
            "moe_quantize_fp8_blocks": (ctypes.c_int, [V, I32, I32, I32, I32,
                                                       V, V, V]),
            "moe_eplb_hottest_map": (ctypes.c_int, [V, I32, I32, V, V, V]),
            "moe_eplb_plan": (ctypes.c_int, [V, I32, I32, I32, V, V, V, V]),
            "moe_eplb_rank_map": (ctypes.c_int, [V, V, V, I32, I32, I32, I32,
                                                 I32, V, V, V]),
            "moe_eplb_record_load": (ctypes.c_int, [V, I32, I32,
                                                    ctypes.c_int64, V, V, V]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, where)


def ptr(t) -> Optional[int]:
    """Device (or host) address of a torch tensor, an int, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def current_stream() -> Optional[int]:
    import torch
    if not torch.cuda.is_available():
        return None
    return torch.cuda.current_stream().cuda_stream


def make_problem(T, H, I, E, k, expert_begin=0, num_local=None,
                 num_physical=None, max_replicas=1, has_shared=False,
                 act="bf16", wdt="bf16", out="bf16",
                 quant_block=128) -> Problem:
    num_local = E if num_local is None else num_local
    num_physical = num_local if num_physical is None else num_physical
    return Problem(T, H, I, E, k, expert_begin, num_local, num_physical,
                   max_replicas, int(bool(has_shared)), DTYPES[act],
                   DTYPES[wdt], DTYPES[out], quant_block)


# ----------------------------------------------------- the entry points
def moe_check_problem(p: Problem) -> int:
    return lib().moe_check_problem(ctypes.byref(p))


def _ws(fn, p: Problem) -> int:
    n = ctypes.c_size_t(0)
    _check(fn(ctypes.byref(p), ctypes.byref(n)), fn.__name__)
    return n.value


def moe_workspace_size(p: Problem) -> int:
    return _ws(lib().moe_workspace_size, p)


def moe_dispatch_workspace_size(p: Problem) -> int:
    return _ws(lib().moe_dispatch_workspace_size, p)


def moe_ffn_workspace_size(p: Problem) -> int:
    return _ws(lib().moe_ffn_workspace_size, p)


def moe_layer_workspace_size(p: Problem) -> int:
    return _ws(lib().moe_layer_workspace_size, p)


def moe_route_topk(p, logits, bias, topk_ids, topk_w, expert_counts=None,
                   stream=None, check=True) -> int:
    st = lib().moe_route_topk(ctypes.byref(p), ptr(logits), ptr(bias),
                              ptr(topk_ids), ptr(topk_w), ptr(expert_counts),
                              stream if stream is not None else current_stream())
    if check:
        _check(st, "moe_route_topk")
    return st


def moe_dispatch(p, x, topk_ids, topk_w, l2p, replica_count, x_perm,
                 x_perm_scales, offsets, row_token, row_weight, pair_row,
                 workspace, ws_bytes, stream=None, check=True) -> int:
    st = lib().moe_dispatch(
        ctypes.byref(p), ptr(x), ptr(topk_ids), ptr(topk_w), ptr(l2p),
        ptr(replica_count), ptr(x_perm), ptr(x_perm_scales), ptr(offsets),
        ptr(row_token), ptr(row_weight), ptr(pair_row), ptr(workspace),
        ws_bytes, stream if stream is not None else current_stream())
    if check:
        _check(st, "moe_dispatch")
    return st


def moe_grouped_ffn(p, x_perm, x_perm_scales, offsets, x_shared,
                    x_shared_scales, weights: Weights, y_perm, y_shared,
                    workspace, ws_bytes, stream=None, check=True) -> int:
    st = lib().moe_grouped_ffn(
        ctypes.byref(p), ptr(x_perm), ptr(x_perm_scales), ptr(offsets),
        ptr(x_shared), ptr(x_shared_scales), ctypes.byref(weights),
        ptr(y_perm), ptr(y_shared), ptr(workspace), ws_bytes,
        stream if stream is not None else current_stream())
    if check:
        _check(st, "moe_grouped_ffn")
    return st


def moe_ffn_intermediate(p, workspace, ws_bytes):
    """Device addresses (h, h_scales or None) of the expert intermediate
    inside an FFN workspace."""
    h = ctypes.c_void_p()
    hs = ctypes.c_void_p()
    _check(lib().moe_ffn_intermediate(ctypes.byref(p), ptr(workspace),
                                      ws_bytes, ctypes.byref(h),
                                      ctypes.byref(hs)),
           "moe_ffn_intermediate")
    return h.value, hs.value


def moe_combine(p, y_perm, pair_row, topk_w, y_shared, out, stream=None,
                check=True) -> int:
    st = lib().moe_combine(ctypes.byref(p), ptr(y_perm), ptr(pair_row),
                           ptr(topk_w), ptr(y_shared), ptr(out),
                           stream if stream is not None else current_stream())
    if check:
        _check(st, "moe_combine")
    return st


def moe_layer_forward(p, logits, bias, x, weights: Weights, l2p,
                      replica_count, out, expert_counts, workspace, ws_bytes,
                      stream=None, check=True) -> int:
    st = lib().moe_layer_forward(
        ctypes.byref(p), ptr(logits), ptr(bias), ptr(x),
        ctypes.byref(weights), ptr(l2p), ptr(replica_count), ptr(out),
        ptr(expert_counts), ptr(workspace), ws_bytes,
        stream if stream is not None else current_stream())
    if check:
        _check(st, "moe_layer_forward")
    return st


def moe_layer_forward_timed(p, logits, bias, x, weights: Weights, l2p,
                            replica_count, out, expert_counts, workspace,
                            ws_bytes, events, stream=None, check=True) -> int:
    """``events``: sequence of MOE_STAGE_EVENTS hipEvent_t handles (ints)."""
    ev = (ctypes.c_void_p * MOE_STAGE_EVENTS)(*events)
    st = lib().moe_layer_forward_timed(
        ctypes.byref(p), ptr(logits), ptr(bias), ptr(x),
        ctypes.byref(weights), ptr(l2p), ptr(replica_count), ptr(out),
        ptr(expert_counts), ptr(workspace), ws_bytes,
        stream if stream is not None else current_stream(),
        ctypes.addressof(ev))
    if check:
        _check(st, "moe_layer_forward_timed")
    return st


NOALLOC_SCRATCH_BYTES = 64 << 20


def moe_layer_forward_noalloc(p, logits, bias, x, weights: Weights, l2p,
                              replica_count, out, expert_counts, stream=None,
                              check=True) -> int:
    """moe_layer_forward with the library's own device scratch (no
    workspace argument; for callers that cannot allocate)."""
    st = lib().moe_layer_forward_noalloc(
        ctypes.byref(p), ptr(logits), ptr(bias), ptr(x),
        ctypes.byref(weights), ptr(l2p), ptr(replica_count), ptr(out),
        ptr(expert_counts),
        stream if stream is not None else current_stream())
    if check:
        _check(st, "moe_layer_forward_noalloc")
    return st


def moe_prepack_weights(src, K, N, dtype, layout, dst, stream=None,
                        check=True) -> int:
    """Prepare a K x N weight matrix stored ``layout`` (MOE_LAYOUT_KN =
    [K][N], MOE_LAYOUT_NK = [N][K]) into the form moe_weights takes."""
    st = lib().moe_prepack_weights(
        ptr(src), K, N, dtype, layout, ptr(dst),
        stream if stream is not None else current_stream())
    if check:
        _check(st, "moe_prepack_weights")
    return st


def moe_quantize_fp8_blocks(w, K, N, block, layout, codes, scales,
                            stream=None, check=True) -> int:
    st = lib().moe_quantize_fp8_blocks(
        ptr(w), K, N, block, layout, ptr(codes), ptr(scales),
        stream if stream is not None else current_stream())
    if check:
        _check(st, "moe_quantize_fp8_blocks")
    return st


def moe_eplb_hottest_map(local_counts: Sequence[int], redundant: int):
    """Host-side replica map; returns (l2p [L][2], replica_count [L], P) as
    Python lists."""
    L = len(local_counts)
    cnt = (ctypes.c_int32 * L)(*[int(c) for c in local_counts])
    l2p = (ctypes.c_int32 * (2 * L))()
    rep = (ctypes.c_int32 * L)()
    P = ctypes.c_int32(0)
    _check(lib().moe_eplb_hottest_map(ctypes.addressof(cnt), L, redundant,
                                      ctypes.addressof(l2p),
                                      ctypes.addressof(rep),
                                      ctypes.addressof(P)),
           "moe_eplb_hottest_map")
    return ([[l2p[2 * e], l2p[2 * e + 1]] for e in range(L)], list(rep),
            P.value)


def moe_eplb_plan(load: Sequence[int], ep: int, redundant: int):
    """Group-wide replica plan and placement (host).  Returns (replicas [E],
    slot_expert [ep][S], slot_replica [ep][S], rank_load [ep]) as lists."""
    E = len(load)
    if E < 1 or ep < 1 or (E + redundant) % ep:
        raise MoeError(MOE_ERR_INVALID_ARGUMENT, "moe_eplb_plan")
    S = (E + redundant) // ep
    ld = (ctypes.c_int64 * E)(*[int(v) for v in load])
    rep = (ctypes.c_int32 * E)()
    se = (ctypes.c_int32 * (ep * S))()
    sr = (ctypes.c_int32 * (ep * S))()
    rl = (ctypes.c_double * ep)()
    _check(lib().moe_eplb_plan(ctypes.addressof(ld), E, ep, redundant,
                               ctypes.addressof(rep), ctypes.addressof(se),
                               ctypes.addressof(sr), ctypes.addressof(rl)),
           "moe_eplb_plan")
    return (list(rep), [list(se[g * S:(g + 1) * S]) for g in range(ep)],
            [list(sr[g * S:(g + 1) * S]) for g in range(ep)], list(rl))


def moe_eplb_rank_map(replicas, slot_expert, slot_replica, redundant: int,
                      rank: int, max_replicas: Optional[int] = None):
    """One rank's (l2p [E][max_replicas], replica_count [E], P) from a plan."""
    E, ep = len(replicas), len(slot_expert)
    S = len(slot_expert[0]) if ep else 0
    mr = max(replicas) if max_replicas is None else max_replicas
    rep = (ctypes.c_int32 * E)(*replicas)
    se = (ctypes.c_int32 * (ep * S))(*[v for row in slot_expert for v in row])
    sr = (ctypes.c_int32 * (ep * S))(*[v for row in slot_replica for v in row])
    l2p = (ctypes.c_int32 * (E * mr))()
    rc = (ctypes.c_int32 * E)()
    P = ctypes.c_int32(0)
    _check(lib().moe_eplb_rank_map(ctypes.addressof(rep), ctypes.addressof(se),
                                   ctypes.addressof(sr), E, ep, redundant,
                                   rank, mr, ctypes.addressof(l2p),
                                   ctypes.addressof(rc), ctypes.addressof(P)),
           "moe_eplb_rank_map")
    return ([list(l2p[e * mr:(e + 1) * mr]) for e in range(E)], list(rc),
            P.value)


def moe_eplb_record_load(expert_counts, E: int, window: int, step: int,
                         history, window_load, stream=None) -> None:
    """Device sliding-window load record (see include/moe.h)."""
    _check(lib().moe_eplb_record_load(ptr(expert_counts), E, window, step,
                                      ptr(history), ptr(window_load),
                                      current_stream() if stream is None
                                      else stream),
           "moe_eplb_record_load")


# ------------------------------------------------- device weight plumbing
@dataclasses.dataclass
class DeviceWeights:
    """Device copies of expert weights plus the pointer tables the C ABI
    takes.  Keeps every tensor alive for as long as the struct is used."""
    struct: Weights
    keep: list


def device_weights(experts: Sequence[dict], shared: Optional[dict],
                   phys_to_logical: Optional[Sequence[int]] = None,
                   device="cuda") -> DeviceWeights:
    """Upload per-expert weights (dict with wg, wu, wd and optionally sg, su,
    sd scale tensors, all torch tensors, host or device) and build the device
    pointer tables.  ``phys_to_logical[p]`` names the logical expert whose
    tensors physical expert p uses (default: identity)."""
    import torch
    keep = []

    def dev(t):
        if t is None:
            return None
        d = t.to(device, non_blocking=False).contiguous()
        keep.append(d)
        return d

    up = [{k: dev(v) for k, v in e.items()} for e in experts]
    if phys_to_logical is None:
        phys_to_logical = list(range(len(up)))

    def table(key):
        if any(up[e].get(key) is None for e in phys_to_logical):
            return None
        t = torch.tensor([up[e][key].data_ptr() for e in phys_to_logical],
                         dtype=torch.int64, device=device)
        keep.append(t)
        return t.data_ptr()

    s = Weights()
    s.w_gate, s.w_up, s.w_down = table("wg"), table("wu"), table("wd")
    s.s_gate, s.s_up, s.s_down = table("sg"), table("su"), table("sd")
    if shared is not None:
        sh = {k: dev(v) for k, v in shared.items()}
        s.sh_gate, s.sh_up, s.sh_down = (sh["wg"].data_ptr(),
                                         sh["wu"].data_ptr(),
                                         sh["wd"].data_ptr())
        if sh.get("sg") is not None:
            s.sh_s_gate, s.sh_s_up, s.sh_s_down = (sh["sg"].data_ptr(),
                                                   sh["su"].data_ptr(),
                                                   sh["sd"].data_ptr())
    return DeviceWeights(struct=s, keep=keep)
