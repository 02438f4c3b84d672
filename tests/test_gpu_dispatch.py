"""Dispatch on the GPU against the oracle: offsets, permutation, pair rows and
the permuted activation rows are bit-exact; two runs are bitwise equal."""
import numpy as np
import pytest

from oracle import eplb, fp8 as ofp8, moe as omoe
from synth import make_workload

from .helpers import device_layer, phys_to_logical_from_map

pytestmark = pytest.mark.gpu


def run_dispatch(wl, l2p=None, rep=None, P=None):
    import torch
    from expert_moe_fp32_amd.runner import to_dev
    ptl = None if l2p is None else phys_to_logical_from_map(l2p, rep, P)
    # dispatch reads no expert weights: none are uploaded
    dl = device_layer(wl, l2p=l2p, rep=rep, P=P, phys_to_logical=ptl,
                      weights=False)
    b = dl.buffers()
    b.pair_row.fill_(-99)
    dlog = to_dev(wl.logits)
    dbias = None if wl.bias is None else to_dev(wl.bias)
    dx = to_dev(wl.x)
    dl.route(b, dlog, dbias)
    dl.dispatch(b, dx)
    torch.cuda.synchronize()
    P = dl.p.num_physical
    off = b.offsets.cpu().numpy()[: P + 1]
    N = int(off[-1])
    res = dict(offsets=off, row_token=b.row_token.cpu().numpy()[:N],
               row_weight=b.row_weight.cpu().numpy()[:N],
               pair_row=b.pair_row.cpu().numpy()[: wl.T * wl.k].reshape(wl.T, wl.k),
               w=b.w.cpu().numpy()[: wl.T * wl.k].reshape(wl.T, wl.k))
    if dl.fp8:
        res["x_perm"] = b.x_perm.cpu().numpy()[: N * wl.H].reshape(N, wl.H)
        res["x_scales"] = b.x_perm_scales.cpu().numpy()[: N * (wl.H // 128)].reshape(
            N, wl.H // 128)
    else:
        eb = 4 if wl.act == "f32" else 2
        raw = b.x_perm.cpu().numpy()[: N * wl.H * eb]
        res["x_perm"] = raw.view(np.float32 if eb == 4 else np.uint16).reshape(N, wl.H)
    del dl, b
    torch.cuda.empty_cache()
    return res


def check_against_oracle(wl, got, l2p=None, rep=None, P=None):
    ids, w, _ = omoe.route_topk(wl.logits, wl.k, wl.bias)
    if l2p is None:
        l2p, rep = omoe.identity_map(wl.num_local)
        P = wl.num_local
    d = omoe.dispatch(ids, wl.expert_begin, wl.num_local, np.asarray(l2p),
                      np.asarray(rep), P)
    assert np.array_equal(got["offsets"], d.offsets)
    assert np.array_equal(got["row_token"], d.row_token)
    assert np.array_equal(got["pair_row"], d.pair_row)
    # row weights are the route weights of the pairs, bit for bit
    assert np.array_equal(got["row_weight"], got["w"][d.row_token, d.row_slot])
    if wl.wdt == "fp8":
        codes, s = ofp8.quantize_rows(wl.x_f32(), 128)
        assert np.array_equal(got["x_perm"], codes[d.row_token])
        assert np.array_equal(got["x_scales"], s[d.row_token])
    else:
        assert np.array_equal(got["x_perm"], wl.x[d.row_token])
    return d


@pytest.mark.parametrize("name,kw", [
    ("tiny", {}),
    ("tiny", dict(T=1000, E=64, num_local=16, expert_begin=16, k=5, H=64, I=64)),
    ("decode", {}),
    ("prefill", dict(H=256, I=128)),
    ("fp8", dict(H=512, I=128)),
    # more than 256 local experts: the multi-block path's per-expert ballot
    # loop, with many blocks (T = 2000) and with one (T = 700)
    ("tiny", dict(T=2000, E=512, num_local=300, expert_begin=100, k=8, H=64,
                  I=64)),
    ("tiny", dict(T=700, E=512, num_local=300, expert_begin=0, k=8, H=64,
                  I=64)),
    # the largest share: 1024 local experts, k = 16
    ("tiny", dict(T=500, E=1024, num_local=1024, expert_begin=0, k=16, H=64,
                  I=64)),
    # just past the single-workgroup kernel's 1024 tokens (a last block of
    # one token), 64 local experts over 20 blocks, a last block of one token
    # at 8193, and 65 local experts (the ballot words past the first)
    ("tiny", dict(T=1025, E=64, num_local=16, expert_begin=8, k=4, H=64,
                  I=64)),
    ("tiny", dict(T=5000, E=128, num_local=64, expert_begin=64, k=8, H=64,
                  I=64)),
    ("tiny", dict(T=8193, E=64, num_local=32, expert_begin=0, k=6, H=64,
                  I=64)),
    ("tiny", dict(T=3000, E=256, num_local=65, expert_begin=0, k=8, H=64,
                  I=64)),
])
def test_dispatch_matches_oracle(name, kw):
    wl = make_workload(name, seed=0, **kw)
    print(f"dispatch {wl.describe()}", flush=True)
    got = run_dispatch(wl)
    check_against_oracle(wl, got)
    again = run_dispatch(wl)
    for key in got:
        assert np.array_equal(got[key], again[key]), key


def test_dispatch_with_redundant_replicas():
    wl = make_workload("skewed", seed=0, H=256, I=128)
    ids, _, counts = omoe.route_topk(wl.logits, wl.k, wl.bias)
    l2p, rep, P = eplb.hottest_replica_map(counts[:wl.num_local], wl.redundant)
    got = run_dispatch(wl, l2p=l2p, rep=rep, P=P)
    d = check_against_oracle(wl, got, l2p, rep, P)
    base = omoe.dispatch(ids, 0, wl.num_local, *omoe.identity_map(wl.num_local),
                         wl.num_local)
    assert d.phys_counts.max() < base.phys_counts.max()


def test_dispatch_edge_cases():
    # every token on one expert, a single token, tokens with no local pair
    wl = make_workload("tiny", seed=0, T=300, E=16, num_local=4,
                       expert_begin=12, k=2, H=64, I=64)
    logits = np.full((300, 16), -5.0, dtype=np.float32)
    logits[:, 13] = 3.0
    logits[:, 2] = 2.0
    logits[::2, 2] = 4.0
    wl._cache["logits"] = logits
    got = run_dispatch(wl)
    d = check_against_oracle(wl, got)
    assert d.phys_counts.tolist() == [0, 300, 0, 0]
    one = make_workload("tiny", seed=1, T=1)
    check_against_oracle(one, run_dispatch(one))
    # the same skew over 3000 tokens (the multi-block kernels)
    big = make_workload("tiny", seed=0, T=3000, E=16, num_local=4,
                        expert_begin=12, k=2, H=64, I=64)
    logits = np.full((3000, 16), -5.0, dtype=np.float32)
    logits[:, 13] = 3.0
    logits[:, 2] = 2.0
    logits[::2, 2] = 4.0
    big._cache["logits"] = logits
    d = check_against_oracle(big, run_dispatch(big))
    assert d.phys_counts.tolist() == [0, 3000, 0, 0]


def test_fp8_quantiser_every_bf16_value():
    """Every finite bf16 value of magnitude <= 448, quantised with a unit
    scale: each 128-channel group leads with +448 or -448, so amax / 448 = 1
    and the codes are the E4M3 rounding of the values themselves.  Every
    rounding boundary of E4M3 is a bf16 value, so this covers all of them,
    the subnormal range, signed zero and the top of the range, bit for bit."""
    pos = np.arange(0, 0x43E1, dtype=np.uint16)          # +0 .. +448
    vals = np.concatenate([pos, pos | np.uint16(0x8000)])
    H, per = 512, 127
    groups = -(-len(vals) // per)
    T = -(-groups // (H // 128))
    g = np.zeros((T * (H // 128), 128), dtype=np.uint16)
    g[:, 0] = 0x43E0                                      # +448
    g[1::2, 0] = 0xC3E0                                   # -448
    flat = np.zeros(g.shape[0] * per, dtype=np.uint16)
    flat[: len(vals)] = vals
    g[:, 1:] = flat.reshape(-1, per)
    wl = make_workload("fp8", seed=3, T=T, H=H, I=128, E=8, num_local=8, k=2)
    wl._cache["x"] = g.reshape(T, H)
    print(f"quantiser: {len(vals)} bf16 values in {T} rows", flush=True)
    got = run_dispatch(wl)
    check_against_oracle(wl, got)
    assert np.all(got["x_scales"] == 1.0)
