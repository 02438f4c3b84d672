"""The C ABI without a GPU: the library loads, exports every declared entry
point, and rejects bad arguments with the documented status before touching
a device."""
import ctypes
import os
import re

import pytest

import expert_moe_fp32_amd as m
from expert_moe_fp32_amd import _lib as L
from oracle import eplb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_entry_points():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    return sorted(set(re.findall(r"MOE_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(", src)))


def test_header_lists_the_binding_exports():
    assert declared_entry_points() == sorted(L.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = L.lib()
    for name in declared_entry_points():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_status_strings():
    assert m.status_string(0) == "ok"
    assert "workspace" in m.status_string(3)
    assert m.status_string(99) == "unknown status"


def good(**kw):
    base = dict(T=64, H=256, I=128, E=16, k=4, expert_begin=4, num_local=8,
                act="bf16", wdt="bf16", out="bf16")
    base.update(kw)
    return m.make_problem(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(), L.MOE_OK),
    (dict(T=-1), L.MOE_ERR_INVALID_ARGUMENT),
    (dict(k=0), L.MOE_ERR_INVALID_ARGUMENT),
    (dict(k=17, E=32), L.MOE_ERR_UNSUPPORTED),
    (dict(k=20, E=16), L.MOE_ERR_INVALID_ARGUMENT),
    (dict(expert_begin=10), L.MOE_ERR_INVALID_ARGUMENT),
    (dict(num_local=0), L.MOE_ERR_INVALID_ARGUMENT),
    (dict(num_physical=0), L.MOE_ERR_INVALID_ARGUMENT),
    (dict(num_physical=3), L.MOE_OK),          # group-wide placement share
    (dict(H=200), L.MOE_ERR_UNSUPPORTED),
    (dict(I=96), L.MOE_ERR_UNSUPPORTED),
    (dict(act="f32"), L.MOE_ERR_UNSUPPORTED),
    (dict(out="fp8"), L.MOE_ERR_UNSUPPORTED),
    (dict(act="f32", wdt="f32", out="f32", H=36, I=20), L.MOE_OK),
    (dict(wdt="fp8", quant_block=64), L.MOE_ERR_UNSUPPORTED),
    (dict(wdt="fp8"), L.MOE_OK),
    (dict(wdt="fp8", H=16384 + 128), L.MOE_ERR_UNSUPPORTED),
    (dict(E=2000, k=2, num_local=8), L.MOE_ERR_UNSUPPORTED),
])
def test_problem_validation(kw, status):
    assert m.moe_check_problem(good(**kw)) == status


def test_null_problem_is_rejected():
    assert L.lib().moe_check_problem(None) == L.MOE_ERR_INVALID_ARGUMENT


def test_workspace_sizes_grow_with_tokens():
    a = m.moe_layer_workspace_size(good(T=64))
    b = m.moe_layer_workspace_size(good(T=640))
    assert 0 < a < b
    assert m.moe_dispatch_workspace_size(good()) > 0
    assert m.moe_ffn_workspace_size(good()) > 0
    assert m.moe_layer_workspace_size(good(has_shared=True)) > a


def test_zero_tokens_is_a_no_op():
    p = good(T=0)
    # nothing is enqueued, so no device is needed
    assert m.moe_route_topk(p, None, None, None, None, None, stream=0,
                            check=False) == L.MOE_OK
    assert m.moe_combine(p, None, None, None, None, None, stream=0,
                         check=False) == L.MOE_OK
    assert m.moe_dispatch(p, None, None, None, None, None, None, None, None,
                          None, None, None, None, 0, stream=0,
                          check=False) == L.MOE_OK


def test_missing_pointers_are_rejected():
    p = good()
    assert m.moe_route_topk(p, None, None, None, None, None, stream=0,
                            check=False) == L.MOE_ERR_INVALID_ARGUMENT
    assert m.moe_combine(p, 16, None, 16, None, 16, stream=0,
                         check=False) == L.MOE_ERR_INVALID_ARGUMENT


def test_misaligned_rows_are_rejected():
    """Row arrays move with 16-byte accesses; a pointer off a 16-byte
    boundary is refused on the host before anything is enqueued."""
    p = good()
    assert m.moe_combine(p, 256, 256, 256, None, 256 + 8, stream=0,
                         check=False) == L.MOE_ERR_INVALID_ARGUMENT
    assert m.moe_combine(p, 256 + 4, 256, 256, None, 256, stream=0,
                         check=False) == L.MOE_ERR_INVALID_ARGUMENT
    need = m.moe_dispatch_workspace_size(p)
    st = m.moe_dispatch(p, 256 + 2, 256, 256, None, None, 256, None, 256, 256,
                        256, 256, 256, need, stream=0, check=False)
    assert st == L.MOE_ERR_INVALID_ARGUMENT


def test_small_workspace_is_rejected():
    p = good()
    need = m.moe_dispatch_workspace_size(p)
    st = m.moe_dispatch(p, 256, 256, 256, None, None, 256, None, 256, 256,
                        256, 256, 256, need - 1, stream=0, check=False)
    assert st == L.MOE_ERR_WORKSPACE


def test_map_arguments_must_pair():
    p = good(num_physical=10, max_replicas=2)
    # a replica map is required once P differs from num_local
    st = m.moe_dispatch(p, 256, 256, 256, None, None, 256, None, 256, 256,
                        256, 256, 256, 1 << 20, stream=0, check=False)
    assert st == L.MOE_ERR_INVALID_ARGUMENT


def test_weights_struct_is_checked():
    p = good()
    w = L.Weights()
    st = m.moe_layer_forward(p, 256, None, 256, w, None, None, 256, None, 256,
                             1 << 30, stream=0, check=False)
    assert st == L.MOE_ERR_INVALID_ARGUMENT
    w.w_gate = w.w_up = w.w_down = 256
    ps = good(has_shared=True)
    st = m.moe_layer_forward(ps, 256, None, 256, w, None, None, 256, None, 256,
                             1 << 30, stream=0, check=False)
    assert st == L.MOE_ERR_INVALID_ARGUMENT


def test_fp8_quantiser_checks_shapes():
    KN = L.MOE_LAYOUT_KN
    st = m.moe_quantize_fp8_blocks(256, 100, 128, 128, KN, 256, 256, stream=0,
                                   check=False)
    assert st == L.MOE_ERR_INVALID_ARGUMENT
    st = m.moe_quantize_fp8_blocks(256, 128, 128, 64, KN, 256, 256, stream=0,
                                   check=False)
    assert st == L.MOE_ERR_UNSUPPORTED
    st = m.moe_quantize_fp8_blocks(256, 128, 128, 128, 2, 256, 256, stream=0,
                                   check=False)
    assert st == L.MOE_ERR_INVALID_ARGUMENT          # no such layout
    assert m.moe_quantize_fp8_blocks(None, 0, 0, 128, KN, None, None,
                                     stream=0, check=False) == L.MOE_OK


@pytest.mark.parametrize("counts,red", [
    ([5, 9, 9, 1, 7], 3), ([0] * 8, 8), (list(range(32, 0, -1)), 8),
    ([3, 1, 4, 1, 5, 9, 2, 6, 5, 3, 5, 8, 9, 7, 9, 3], 0)])
def test_hottest_map_matches_oracle(counts, red):
    l2p, rep, P = m.moe_eplb_hottest_map(counts, red)
    ol2p, orep, oP = eplb.hottest_replica_map(counts, red)
    assert P == oP
    assert rep == orep.tolist()
    for e in range(len(counts)):
        assert l2p[e][: rep[e]] == ol2p[e][: rep[e]].tolist()


def test_hottest_map_rejects_bad_arguments():
    with pytest.raises(m.MoeError):
        m.moe_eplb_hottest_map([1, 2], 3)


def test_prepack_checks_arguments():
    KN, NK = L.MOE_LAYOUT_KN, L.MOE_LAYOUT_NK
    # bf16: K (the reduction) a multiple of 32, N a multiple of 16
    assert m.moe_prepack_weights(256, 30, 16, L.MOE_BF16, KN, 512, stream=0,
                                 check=False) == L.MOE_ERR_INVALID_ARGUMENT
    assert m.moe_prepack_weights(256, 32, 24, L.MOE_BF16, NK, 512, stream=0,
                                 check=False) == L.MOE_ERR_INVALID_ARGUMENT
    assert m.moe_prepack_weights(256, 32, 16, 7, KN, 512, stream=0,
                                 check=False) == L.MOE_ERR_UNSUPPORTED
    assert m.moe_prepack_weights(256, 32, 16, L.MOE_BF16, 5, 512, stream=0,
                                 check=False) == L.MOE_ERR_INVALID_ARGUMENT
    assert m.moe_prepack_weights(256, 32, 16, L.MOE_BF16, KN, 256, stream=0,
                                 check=False) == L.MOE_ERR_INVALID_ARGUMENT
    assert m.moe_prepack_weights(None, 32, 0, L.MOE_BF16, KN, None, stream=0,
                                 check=False) == L.MOE_OK


def test_prepack_fp8_checks_arguments():
    KN = L.MOE_LAYOUT_KN
    assert m.moe_prepack_weights(256, 64, 16, L.MOE_FP8_E4M3, KN, 512,
                                 stream=0, check=False) == \
        L.MOE_ERR_INVALID_ARGUMENT
    assert m.moe_prepack_weights(256, 128, 8, L.MOE_FP8_E4M3, KN, 512,
                                 stream=0, check=False) == \
        L.MOE_ERR_INVALID_ARGUMENT


def test_one_workspace_serves_every_entry_point():
    for p in (good(), good(has_shared=True), good(wdt="fp8"),
              good(T=3000, num_physical=12, max_replicas=2)):
        total = m.moe_workspace_size(p)
        assert total == max(m.moe_dispatch_workspace_size(p),
                            m.moe_ffn_workspace_size(p),
                            m.moe_layer_workspace_size(p))


def test_intermediate_lies_inside_the_ffn_workspace():
    for p, hb in ((good(), 2), (good(wdt="fp8"), 1),
                  (good(act="f32", wdt="f32", out="f32"), 4)):
        need = m.moe_ffn_workspace_size(p)
        base = 1 << 20
        h, hs = m.moe_ffn_intermediate(p, base, need)
        cap = p.T * min(p.k, p.num_local)
        assert base <= h and h + cap * p.I * hb <= base + need
        if p.weight_dtype == L.MOE_FP8_E4M3:
            assert hs is not None and h < hs
            assert hs + cap * (p.I // 128) * 4 <= base + need
        else:
            assert hs is None
    with pytest.raises(m.MoeError):
        m.moe_ffn_intermediate(good(), 1 << 20, 16)
