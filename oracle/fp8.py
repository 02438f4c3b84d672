"""OCP 8-bit floating point E4M3 ("e4m3fn") and the FP8 quantisers.

Format (OCP 8-bit Floating Point Specification, E4M3): 1 sign bit, 4 exponent
bits with bias 7, 3 mantissa bits; exponent field 0 encodes subnormals
m * 2^-9; S.1111.111 is NaN; there is no infinity; the largest finite value is
S.1111.110 = 1.75 * 2^8 = 448.

Quantisation rule used by the FP8 workload (the infra-guide page, section 3.2,
describes FP8 dispatch of tokens; the workload fixes the granularity):
* weights: one float32 scale per 128x128 block of the stored matrix;
* activations: one float32 scale per token per 128 channels;
* scale s = amax / 448 in float32 (s = 1 where amax = 0);
* code q = round-to-nearest-even(fl32(v / s)), saturated to +-448, the sign
  bit copied from v.
All of it is done in float32, the precision in which the kernels take the same
decisions.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode_table() -> np.ndarray:
    """float64 value of each of the 256 codes (NaN for 0x7F and 0xFF)."""
    vals = np.empty(256, dtype=np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = sign * m * 2.0 ** -9
        else:
            vals[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_TABLE = e4m3_decode_table()
_POS = _TABLE[:127]          # codes 0x00..0x7E, strictly increasing, 0 .. 448


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v) -> np.ndarray:
    """Round float values to the nearest E4M3 code, ties to the even code,
    saturating magnitudes above 448 to 448.  Finite inputs only."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    a_sat = np.minimum(a, E4M3_MAX)
    hi = np.searchsorted(_POS, a_sat, side="left")      # _POS[hi] >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo = a_sat - _POS[lo]
    d_hi = _POS[hi] - a_sat
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a_sat == _POS[hi], hi, code).astype(np.uint8)
    sign = np.signbit(v).astype(np.uint8) << np.uint8(7)
    return (code | sign).astype(np.uint8)


def _scale_from_amax(amax32: np.ndarray) -> np.ndarray:
    amax32 = np.asarray(amax32, dtype=np.float32)
    s = amax32 / np.float32(E4M3_MAX)
    return np.where(amax32 == np.float32(0.0), np.float32(1.0),
                    s).astype(np.float32)


def quantize_blocks_2d(w32: np.ndarray, block: int = 128):
    """Quantise a float32 matrix [R, C] with one scale per block x block tile.

    Returns (codes uint8 [R, C], scales float32 [R/block, C/block])."""
    w32 = np.asarray(w32, dtype=np.float32)
    R, C = w32.shape
    if R % block or C % block:
        raise ValueError("matrix dims must be multiples of the block size")
    t = w32.reshape(R // block, block, C // block, block)
    amax = np.abs(t).max(axis=(1, 3))
    s = _scale_from_amax(amax)
    q32 = (t / s[:, None, :, None]).astype(np.float32)
    codes = e4m3_encode(q32).reshape(R, C)
    return codes, s


def quantize_rows(a32: np.ndarray, group: int = 128):
    """Quantise rows of a float32 matrix [N, K] with one scale per row per
    ``group`` consecutive columns.  Returns (codes [N, K], scales [N, K/group])."""
    a32 = np.asarray(a32, dtype=np.float32)
    N, K = a32.shape
    if K % group:
        raise ValueError("row length must be a multiple of the group size")
    t = a32.reshape(N, K // group, group)
    amax = np.abs(t).max(axis=2)
    s = _scale_from_amax(amax)
    q32 = (t / s[:, :, None]).astype(np.float32)
    return e4m3_encode(q32).reshape(N, K), s


def dequantize_blocks_2d(codes: np.ndarray, scales: np.ndarray,
                         block: int = 128) -> np.ndarray:
    """Exact float64 value of a block-quantised matrix."""
    R, C = codes.shape
    v = e4m3_decode(codes).reshape(R // block, block, C // block, block)
    v = v * scales.astype(np.float64)[:, None, :, None]
    return v.reshape(R, C)


def dequantize_rows(codes: np.ndarray, scales: np.ndarray,
                    group: int = 128) -> np.ndarray:
    N, K = codes.shape
    v = e4m3_decode(codes).reshape(N, K // group, group)
    return (v * scales.astype(np.float64)[:, :, None]).reshape(N, K)


# ------------------------------------- codes a float32 evaluation may give
def row_scale_interval(h64: np.ndarray, eps: np.ndarray, group: int = 128):
    """Range of the per-row, per-``group`` scale fl32(amax/448) when each
    element of h may be off by up to ``eps`` (float64 arrays [N, K]): amax
    lies between max(|h| - eps, 0) and max(|h| + eps) over the group, and
    rounding to float32 and the division are monotone.  Returns float32
    (s_lo, s_hi), each [N, K/group]."""
    N, K = h64.shape
    a = np.abs(h64).reshape(N, K // group, group)
    e = np.asarray(eps, dtype=np.float64).reshape(N, K // group, group)
    lo = np.maximum(a - e, 0.0).max(axis=2)
    hi = (a + e).max(axis=2)
    # amax is itself a float32 value inside [lo, hi]
    lo32 = _round_f32_down(lo)
    hi32 = _round_f32_up(hi)
    return _scale_from_amax(lo32), _scale_from_amax(hi32)


def row_code_interval(h64: np.ndarray, eps: np.ndarray, s_lo: np.ndarray,
                      s_hi: np.ndarray, group: int = 128):
    """Smallest and largest E4M3 value that round-to-nearest-even of
    fl32(v / s) can give for some v in [h - eps, h + eps] and some scale s in
    [s_lo, s_hi] (float32 [N, K/group]).  Division, rounding to float32 and
    the saturating E4M3 rounding are all monotone, so the ends of the
    quotient interval give the ends of the code interval.  Returns float64
    arrays (vmin, vmax) [N, K] of code values (not multiplied by the
    scale)."""
    slo = np.repeat(np.asarray(s_lo, dtype=np.float64), group, axis=1)
    shi = np.repeat(np.asarray(s_hi, dtype=np.float64), group, axis=1)
    e = np.asarray(eps, dtype=np.float64)
    a, b = h64 - e, h64 + e
    qlo = np.where(a >= 0, a / shi, a / slo)          # min of a / s
    qhi = np.where(b >= 0, b / slo, b / shi)          # max of b / s
    # the float64 quotients are widened past their own rounding
    qlo = qlo - np.abs(qlo) * 2.0 ** -50
    qhi = qhi + np.abs(qhi) * 2.0 ** -50
    lo = e4m3_decode(e4m3_encode(qlo.astype(np.float32)))
    hi = e4m3_decode(e4m3_encode(qhi.astype(np.float32)))
    return lo, hi


def _round_f32_down(v: np.ndarray) -> np.ndarray:
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    return np.where(f.astype(np.float64) > v, np.nextafter(f, np.float32(-np.inf)),
                    f).astype(np.float32)


def _round_f32_up(v: np.ndarray) -> np.ndarray:
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    return np.where(f.astype(np.float64) < v, np.nextafter(f, np.float32(np.inf)),
                    f).astype(np.float32)
