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
