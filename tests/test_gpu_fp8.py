"""FP8 recipe on the GPU against the oracle.

* Block-quantised weight codes and scales bit-exact, from either storage
  order of the weights; the packed layout as documented.
* The complete layer check: every h code and scale lies in the set a correct
  evaluation may give (one of two neighbouring codes only where the exact h
  is within the oracle's stated evaluation bound -- float32 steps and the
  matrix instruction's block sums -- of an E4M3 rounding boundary), and the
  output is within 4e-2 x RMS of the oracle's once the output rounding and
  the effect of those alternative codes are allowed for (the FP8 dispatch
  of "6.4 Data parallelism and expert parallelism", section 3.2; weights in
  FP8, section 2.3).
* The block-sum error model behind that bound, measured through the C ABI."""
import numpy as np
import pytest

from oracle import fp8 as ofp8, moe as omoe
from synth import make_workload

from .helpers import fp8_complete_check, run_fp8_steps

pytestmark = pytest.mark.gpu

KN, NK = 0, 1


@pytest.mark.parametrize("layout", [KN, NK])
def test_weight_quantiser_bit_exact(layout):
    import torch
    import expert_moe_fp32_amd as m
    rng = np.random.default_rng(21)
    K, N = 384, 256                             # logical [K][N]
    w = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    w[:128, 128:] = 0.0                         # an all-zero block
    w[200, 7] = 3.0                             # a block with one outlier
    src = w if layout == KN else np.ascontiguousarray(w.T)
    dw = torch.from_numpy(src).cuda()
    codes = torch.empty(src.shape, dtype=torch.uint8, device="cuda")
    scales = torch.empty((N // 128, K // 128), dtype=torch.float32,
                         device="cuda")
    m.moe_quantize_fp8_blocks(dw, K, N, 128, layout, codes, scales)
    torch.cuda.synchronize()
    rc, rs = ofp8.quantize_blocks_2d(w, 128)    # [K][N] codes, [K/128][N/128]
    want_codes = rc if layout == KN else rc.T
    assert np.array_equal(codes.cpu().numpy(), want_codes)
    assert np.array_equal(scales.cpu().numpy(), rs.T)


def packed_fp8_reference(c: np.ndarray) -> np.ndarray:
    """c: logical [K][N] codes.  Block (n/16, k/128) of 2 KiB at
    (n/16)*(K/128) + k/128; lane L = n%16 + 16*((k%128)//32); byte (k%32) of
    its slot at (k%32 >= 16)*1024 + L*16 + k%16."""
    K, N = c.shape
    out = np.empty(K * N, dtype=np.uint8)
    for n in range(N):
        for k in range(K):
            blk = (n // 16) * (K // 128) + k // 128
            L = n % 16 + 16 * ((k % 128) // 32)
            off = ((k % 32) // 16) * 1024 + L * 16 + k % 16
            out[blk * 2048 + off] = c[k, n]
    return out


@pytest.mark.parametrize("layout", [KN, NK])
def test_prepack_fp8_layout(layout):
    import torch
    import expert_moe_fp32_amd as m
    from expert_moe_fp32_amd import _lib as L
    rng = np.random.default_rng(3)
    K, N = 256, 32
    c = rng.integers(0, 256, size=(K, N), dtype=np.uint8)
    src = torch.from_numpy(c if layout == KN else np.ascontiguousarray(c.T)).cuda()
    dst = torch.zeros_like(src)
    m.moe_prepack_weights(src, K, N, L.MOE_FP8_E4M3, layout, dst)
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy().ravel(), packed_fp8_reference(c))


complete_check = fp8_complete_check


@pytest.mark.parametrize("kw", [
    # LDS-ring weight streaming, 160-row tiles (one per expert), ragged;
    # gate/up runs two trips of its 4-stage loop
    dict(T=200, H=1024, I=512, E=16, num_local=8, k=4),
    # register weight streaming (k_wstream_fp8), 32-row tiles (a few rows
    # per expert)
    dict(T=64, H=512, I=512, E=32, num_local=8, k=4),
    # the same kernel with 6 K blocks in gate/up (the last trip of its
    # 4-block loop half past the end) and 2 in down (the prologue clamps
    # its third block to the last one)
    dict(T=64, H=768, I=256, E=32, num_local=8, k=4),
    # the ring with K-block counts that are multiples of its 3-stage trip
    # (6 in gate/up, 3 in down: no partial last trip)
    dict(T=200, H=768, I=384, E=16, num_local=8, k=4),
    # LDS-ring streaming with the shared expert's 300 rows in 160-row tiles
    dict(T=300, H=512, I=512, E=8, num_local=8, k=2, shared=True),
    # 128 x 128 tiled kernel (H not a multiple of 256; many rows per
    # expert), and the ring with a one-K-block down pass (I = 128)
    dict(T=40, H=384, I=128, E=64, num_local=16, k=4),
    dict(T=300, H=256, I=128, E=8, num_local=8, k=2, shared=True),
    # 1,400 rows at I = 256 (where one h code rounded the other way moves an
    # output by a visible part of its RMS) and at I = 512
    dict(T=700, H=256, I=256, E=8, num_local=8, k=2),
    dict(T=700, H=256, I=512, E=8, num_local=8, k=2),
])
def test_fp8_layer_reduced(kw):
    complete_check(make_workload("fp8", seed=31, **kw))


@pytest.mark.parametrize("T,E,shared", [(128, 32, False), (300, 64, False),
                                        (45, 32, False), (100, 32, True)])
def test_fp8_streaming_group_of_many_tiles(T, E, shared):
    """The register weight-streaming recipe (a few rows per expert) with a
    group of more than one 32-row tile: local expert 3 on every token (128,
    300 or 45 rows in balanced tiles of up to 32), or the shared expert's T
    rows."""
    wl = make_workload("fp8", seed=33, T=T, H=512, I=512, E=E, num_local=8,
                       k=4, shared=shared)
    if not shared:
        logits = wl.logits.copy()
        logits[:, 3] += 20.0
        wl._cache["logits"] = logits
    st = complete_check(wl)
    assert st["codes"] > 0


def test_fp8_weights_in_either_storage_order_give_the_same_layer():
    """Weights handed over in the logical layout (W_gate, W_up [H][I],
    W_down [I][H]) or transposed give bit-identical outputs."""
    from .helpers import run_fp8_steps as run
    wl = make_workload("fp8", seed=32, T=96, H=512, I=256, E=16,
                       num_local=8, k=4)
    a = run(wl, layout="kn")
    b = run(wl, layout="nk")
    assert np.array_equal(a["out"], b["out"])
    N = int(a["offsets"][-1])                 # rows past N are not written
    assert np.array_equal(a["h"][:N], b["h"][:N])
    assert np.array_equal(a["h_scales"][:N], b["h_scales"][:N])


def test_fp8_full_all_tokens():
    """The FP8 prefill workload at full size (T = 4096, H = 7168, I = 2048,
    32 of 256 experts, k = 8), every token."""
    st = complete_check(make_workload("fp8", seed=0), workers=16)
    assert st["codes"] > 4000 * 2048


def test_fp8_many_rows_per_expert_sampled():
    """FP8 prefill with 8,192 tokens: about 256 rows per local expert, more
    than one 160-row tile holds, so gate/up and down run the 128 x 128 tiled
    kernel and h goes through the separate quantisation pass; 256 sampled
    tokens at full size (H = 7168, I = 2048)."""
    from .helpers import sample_tokens
    wl = make_workload("fp8", seed=2, T=8192)
    st = complete_check(wl, tokens=sample_tokens(wl.T, 256), workers=16)
    assert st["codes"] > 200 * 2048          # about one local pair a token


def test_matrix_instruction_block_error_within_the_model():
    """The oracle's error model of an FP8 block sum (oracle.moe.C_BLOCK: a
    128-product sum returned with an error of RMS at most C_BLOCK u sum|p|),
    measured through the C ABI: with I = 128 every down-projection output is
    one such block sum times the row scale of h and the weight block scale,
    so y_perm / (s_h s_w) against the exact sum of the h codes times the
    weight codes gives the instruction's error on 1.2 M block sums."""
    wl = make_workload("fp8", seed=33, T=1200, H=1024, I=128, E=8,
                       num_local=8, k=1)
    print(f"layer {wl.describe()}", flush=True)
    got = run_fp8_steps(wl)
    off = got["offsets"]
    ratios = []
    for p in range(wl.num_local):
        rows = np.arange(off[p], off[p + 1])
        if rows.size == 0:
            continue
        wd32 = wl.expert(p)["wd"]                       # [I][H] float32
        codes, s_w = ofp8.quantize_blocks_2d(wd32, 128)  # s_w [1][H/128]
        wv = ofp8.e4m3_decode(codes)                     # [128][H]
        hv = ofp8.e4m3_decode(got["h"][rows])            # [n][128]
        exact = hv @ wv
        absum = np.abs(hv) @ np.abs(wv)
        scale = (got["h_scales"][rows, :1].astype(np.float64) *
                 np.repeat(s_w[0].astype(np.float64), 128)[None, :])
        meas = got["y_perm"][rows].astype(np.float64) / scale
        ok = absum > 0
        ratios.append((np.abs(meas - exact)[ok] /
                       (omoe.U32 * absum[ok])))
    r = np.concatenate(ratios)
    rms = float(np.sqrt(np.mean(r * r)))
    print(f"  block sums {r.size}: error / (u sum|p|) rms {rms:.2f} "
          f"median {np.median(r):.2f} max {r.max():.1f}", flush=True)
    assert r.size > 1_000_000
    assert rms <= omoe.C_BLOCK
