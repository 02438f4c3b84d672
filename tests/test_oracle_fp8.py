"""OCP E4M3 codec and FP8 quantisers of the oracle, pinned to the format's
definition, to a library implementation (torch.float8_e4m3fn) and to the
bounds a correct rounding must meet."""
import numpy as np
import pytest
import torch

from oracle import fp8


def test_special_codes_from_the_definition():
    t = fp8.e4m3_decode_table()
    assert t[0x00] == 0.0 and t[0x80] == 0.0 and np.signbit(t[0x80])
    assert t[0x01] == 2.0 ** -9            # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9        # largest subnormal
    assert t[0x08] == 2.0 ** -6            # smallest normal
    assert t[0x38] == 1.0                  # exponent field 7 = bias
    assert t[0x7E] == 448.0                # largest finite
    assert t[0xFE] == -448.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.all(np.diff(t[:127]) > 0)    # codes 0..126 increase


def test_decode_table_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = fp8.e4m3_decode_table()
    both_nan = np.isnan(ref) & np.isnan(mine)
    assert np.all(both_nan | (ref == mine))


def test_round_trip_every_code():
    t = fp8.e4m3_decode_table()
    codes = np.array([c for c in range(256) if not np.isnan(t[c])],
                     dtype=np.uint8)
    assert np.array_equal(fp8.e4m3_encode(t[codes]), codes)


def test_midpoints_round_to_even():
    t = fp8.e4m3_decode_table()
    for c in range(0, 126):
        mid = (t[c] + t[c + 1]) / 2
        want = c if c % 2 == 0 else c + 1
        assert fp8.e4m3_encode(mid) == want, c
        assert fp8.e4m3_encode(-mid) == want | 0x80, c


def test_saturation_above_max():
    assert fp8.e4m3_encode(1e6) == 0x7E
    assert fp8.e4m3_encode(-470.0) == 0xFE
    assert fp8.e4m3_encode(464.0) == 0x7E


def test_encode_matches_torch_in_range():
    rng = np.random.default_rng(7)
    v = np.concatenate([rng.standard_normal(200000) * 50,
                        rng.standard_normal(20000) * 1e-3,
                        rng.uniform(-448, 448, 20000)]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    mine = fp8.e4m3_encode(v)
    # torch may return +0 for tiny negatives where the sign bit is kept here
    ok = (ref == mine) | ((ref & 0x7F) == 0) & ((mine & 0x7F) == 0)
    assert ok.all()


def test_rounding_error_bound():
    rng = np.random.default_rng(3)
    v = rng.uniform(-448, 448, 100000)
    d = fp8.e4m3_decode(fp8.e4m3_encode(v))
    a = np.abs(v)
    # half an ulp: 2^(e-3)/2 for normals, 2^-10 for subnormals
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    assert np.all(np.abs(d - v) <= np.exp2(e - 4) * (1 + 1e-12))


def test_block_quantiser_scales_and_codes():
    rng = np.random.default_rng(11)
    w = (rng.standard_normal((256, 384)) * 0.02).astype(np.float32)
    w[:128, :128] = 0.0                           # a zero block: scale 1
    codes, s = fp8.quantize_blocks_2d(w, 128)
    assert s.shape == (2, 3) and s.dtype == np.float32
    assert s[0, 0] == 1.0 and np.all(codes[:128, :128] & 0x7F == 0)
    for bi in range(2):
        for bj in range(3):
            blk = w[bi*128:(bi+1)*128, bj*128:(bj+1)*128]
            amax = np.abs(blk).max()
            if amax > 0:
                assert s[bi, bj] == np.float32(amax) / np.float32(448)
                # the largest element lands at (or rounds to) the top code
                c = codes[bi*128:(bi+1)*128, bj*128:(bj+1)*128]
                assert (c & 0x7F).max() == 0x7E
    deq = fp8.dequantize_blocks_2d(codes, s, 128)
    rel = np.abs(deq - w) / np.repeat(np.repeat(s, 128, 0), 128, 1)
    assert rel.max() <= 16.0 + 1e-9               # half-ulp at 448 is 16


def test_row_quantiser_groups():
    rng = np.random.default_rng(5)
    a = rng.standard_normal((3, 256)).astype(np.float32)
    codes, s = fp8.quantize_rows(a, 128)
    assert s.shape == (3, 2)
    for r in range(3):
        for g in range(2):
            amax = np.abs(a[r, g*128:(g+1)*128]).max()
            assert s[r, g] == np.float32(amax) / np.float32(448)
    deq = fp8.dequantize_rows(codes, s, 128)
    assert np.all(np.abs(deq - a) <= np.repeat(s, 128, 1) * 16 + 1e-12)
    with pytest.raises(ValueError):
        fp8.quantize_rows(a[:, :100], 128)


# ------------------------------------ codes a float32 evaluation may give
def test_intervals_collapse_without_error():
    """With eps = 0 the scale and code intervals are the quantiser's own
    scale and code."""
    rng = np.random.default_rng(11)
    h = rng.standard_normal((6, 256)) * 0.3
    codes, s = fp8.quantize_rows(h.astype(np.float32), 128)
    h32 = h.astype(np.float32).astype(np.float64)
    z = np.zeros_like(h32)
    s_lo, s_hi = fp8.row_scale_interval(h32, z)
    assert np.array_equal(s_lo, s) and np.array_equal(s_hi, s)
    v_lo, v_hi = fp8.row_code_interval(h32, z, s_lo, s_hi)
    assert np.array_equal(v_lo, fp8.e4m3_decode(codes))
    assert np.array_equal(v_hi, fp8.e4m3_decode(codes))


def test_a_value_at_a_rounding_boundary_has_two_codes():
    """Hand-worked: with scale 1 (group maximum 448), 1.0625 lies half way
    between the E4M3 values 1.0 and 1.125; any error window around it admits
    both, while 1.03 (a quarter step from 1.0) keeps one code for a window
    of 0.01."""
    h = np.zeros((1, 128))
    h[0, 0] = 448.0
    h[0, 1] = 1.0625
    h[0, 2] = 1.03
    eps = np.zeros_like(h)
    eps[0, 1:3] = 0.01
    s_lo, s_hi = fp8.row_scale_interval(h, eps)
    assert s_lo[0, 0] == s_hi[0, 0] == np.float32(1.0)
    v_lo, v_hi = fp8.row_code_interval(h, eps, s_lo, s_hi)
    assert (v_lo[0, 1], v_hi[0, 1]) == (1.0, 1.125)
    assert (v_lo[0, 2], v_hi[0, 2]) == (1.0, 1.0)
    assert (v_lo[0, 0], v_hi[0, 0]) == (448.0, 448.0)


def test_perturbed_quantisations_stay_inside_the_intervals():
    """Brute force: many float32 perturbations of h, each no larger than
    eps, quantised by the oracle's own row quantiser, give scales and codes
    inside the intervals."""
    rng = np.random.default_rng(12)
    h = rng.standard_normal((8, 384))
    eps = np.abs(h) * 1e-3 + 1e-6
    s_lo, s_hi = fp8.row_scale_interval(h, eps)
    v_lo, v_hi = fp8.row_code_interval(h, eps, s_lo, s_hi)
    wide = 0
    for trial in range(40):
        hp = h + eps * rng.uniform(-1.0, 1.0, size=h.shape)
        if trial == 0:
            hp = h + eps                       # the window's ends
        elif trial == 1:
            hp = h - eps
        codes, s = fp8.quantize_rows(hp.astype(np.float32), 128)
        assert np.all((s_lo <= s) & (s <= s_hi))
        v = fp8.e4m3_decode(codes)
        assert np.all((v_lo <= v) & (v <= v_hi))
    wide = np.count_nonzero(v_lo != v_hi)
    assert 0 < wide < h.size // 4


def test_h_bound_covers_a_float32_evaluation():
    """The bound on an evaluation of h = silu(x Wg) * (x Wu) covers an actual
    float32 evaluation (torch float32 matmuls on the CPU, silu in float32),
    and is small against h."""
    from oracle import moe
    rng = np.random.default_rng(13)
    n, K, I = 64, 2048, 256
    x = rng.standard_normal((n, K))
    wg = rng.standard_normal((K, I)) * 0.02
    wu = rng.standard_normal((K, I)) * 0.02
    g, u = x @ wg, x @ wu
    h = moe.silu(g) * u
    eps = moe.h_eval_bound(x, wg, wu, g, u)
    t = lambda a: torch.from_numpy(a.astype(np.float32))
    g32 = t(x) @ t(wg)
    u32 = t(x) @ t(wu)
    h32 = (torch.nn.functional.silu(g32) * u32).double().numpy()
    assert np.all(np.abs(h32 - h) <= eps)
    assert np.median(eps / np.abs(h)) < 1e-2


def test_fp8_layer_allowance_covers_a_float32_evaluation():
    """The FP8 layer evaluated in float32 (torch on the CPU: g and u, h,
    h quantised by the oracle's own row quantiser, down) stays within the
    oracle output plus its allowance, and every h code and scale of that
    evaluation lies in the oracle's intervals."""
    from oracle import moe
    from synth import make_workload
    wl = make_workload("fp8", seed=6, T=48, H=256, I=256, E=8, num_local=4,
                       k=2)
    ex = moe.expert_set_from_workload(wl)
    res = moe.layer_from_workload(wl, ex, fp8_detail=True)
    d = res.disp
    x_rows = moe.activation_rows(wl.x, wl.act, "fp8")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    y = np.zeros((d.N, wl.H))
    for p in range(wl.num_local):
        rows = np.arange(d.offsets[p], d.offsets[p + 1])
        if rows.size == 0:
            continue
        wg, wu, wd = ex.get(p)
        xr = t(x_rows[d.row_token[rows]])
        h32 = (torch.nn.functional.silu(xr @ t(wg)) * (xr @ t(wu))).numpy()
        codes, s = fp8.quantize_rows(h32, 128)
        assert np.all((res.fp8_routed.s_lo[rows] <= s) &
                      (s <= res.fp8_routed.s_hi[rows]))
        v = fp8.e4m3_decode(codes)
        assert np.all((res.fp8_routed.v_lo[rows] <= v) &
                      (v <= res.fp8_routed.v_hi[rows]))
        y[rows] = fp8.dequantize_rows(codes, s, 128) @ wd
    out = moe.combine(y, d.pair_row, res.weights, None, wl.T, wl.H)
    rms = np.sqrt(np.mean(res.out ** 2))
    assert np.all(np.abs(out - res.out) <= res.out_allow + 1e-9 * rms)


def test_h_bound_covers_block_sums_with_the_modelled_error():
    """Brute force of the model behind the bound: every 128-product block
    sum of g and u perturbed by a normal error of RMS C_BLOCK u sum|p| over
    the block (independent between blocks), h recomputed in float64: the
    result stays within the bound."""
    from oracle import moe
    rng = np.random.default_rng(14)
    n, K, I, B = 24, 1024, 128, 128
    x = rng.standard_normal((n, K))
    wg = rng.standard_normal((K, I)) * 0.02
    wu = rng.standard_normal((K, I)) * 0.02
    g, u = x @ wg, x @ wu
    h = moe.silu(g) * u
    eps = moe.h_eval_bound(x, wg, wu, g, u, B)

    def perturbed(w):
        tot = np.zeros((n, I))
        for b in range(K // B):
            xb, wb = x[:, b * B:(b + 1) * B], w[b * B:(b + 1) * B]
            sb = xb @ wb
            rms = moe.C_BLOCK * moe.U32 * (np.abs(xb) @ np.abs(wb))
            tot += sb + rms * rng.standard_normal(sb.shape)
        return tot

    for _ in range(5):
        hp = moe.silu(perturbed(wg)) * perturbed(wu)
        assert np.all(np.abs(hp - h) <= eps)
