"""NVFP4 quantisation: tensor amax -> FP32 global, block amax -> E4M3 scale,
E2M1 encode, pack.  TEST INFRASTRUCTURE ONLY.

Follows [P3] "前提1" and [P1] "접근 방법": 4-bit E2M1 values, one E4M3 scale
per 16 consecutive elements set from the block maximum divided by 6, one FP32
scale per tensor.  Readings where the pages are silent:

  * the 16-element blocks run along the last (reduction, K) axis;
  * g = RNE_fp32(amax / 2688) is the decode-direction global (formats.py);
  * block scale s = RNE_SAT_E4M3(m / (6 g)) with m the block's max |x|, the
    quotient taken exactly and rounded once; s = 0 when m = 0 or g = 0;
  * magnitude code = RNE_SAT_E2M1(|x| / (dec(s) g)), exact quotient, one
    rounding, ties to the even code; 0 when dec(s) = 0;
  * the sign bit is signbit(x) always (so -0.0 and negatives that round to
    zero give code 0b1000);
  * two codes per byte, the even-K element in the low nibble; scales are raw
    E4M3 bytes; both row-major.

Why the float64 tier is exact.  Every decision compares an exact quotient
with a midpoint of a grid.  The numerators (m or |x|) are binary32 values
(<= 24 significant bits) and the denominators 6 g and dec(s) g have <= 26 and
<= 28 significant bits, so both are exact in float64.  If the quotient is not
equal to a midpoint t (<= 5 significant bits), then |num - t den| is a
nonzero multiple of a power of two whose size relative to num is at least
about 2^-33, far above the 2^-53 relative error of one float64 division;
a correctly rounded float64 quotient therefore lies on the same side of t.
If the quotient equals t, the division is exact and the tie is seen.
The same holds for g: A / 2688 either is exact in binary32 or is a
non-terminating binary fraction at relative distance >= 2^-30 from every
binary32 rounding boundary, so rounding once to float64 and then to float32
equals one correct rounding.  tests/test_oracle_pins.py checks this tier
against the Fraction tier below.
"""
from fractions import Fraction

import numpy as np

from .formats import (E2M1_MAG, GLOBAL_DIVISOR, e2m1_rne_sat_exact,
                      e4m3_decode, e4m3_rne_sat_exact, fp32_rne_exact,
                      e4m3_decode_table, bf16_rne_from_f64)

BLOCK = 16

_E4M3 = e4m3_decode_table()[:127]                 # codes 0x00..0x7E
_E2M1 = np.array([float(v) for v in E2M1_MAG])    # magnitude codes 0..7


def _rne_sat_codes(v, grid):
    """Vectorised RNE-saturating rounding of v >= 0 (float64) onto `grid`
    (increasing float64, index = code).  Ties go to the even index."""
    lo = np.searchsorted(grid, v, side="right") - 1
    lo = np.clip(lo, 0, len(grid) - 1)
    top = lo == len(grid) - 1
    hi = np.minimum(lo + 1, len(grid) - 1)
    mid = (grid[lo] + grid[hi]) * 0.5              # exact: few-bit values
    code = np.where(v < mid, lo, np.where(v > mid, hi, lo + (lo & 1)))
    return np.where(top, len(grid) - 1, code)


def global_scale(x):
    """FP32 global decode scale of a tensor: RNE_fp32(max|x| / 2688)."""
    x = np.asarray(x, dtype=np.float32)
    a = float(np.max(np.abs(x))) if x.size else 0.0
    return np.float32(a / float(GLOBAL_DIVISOR))


def pack_codes(codes):
    """[rows, K] 4-bit codes -> [rows, K/2] bytes, even K in the low nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def unpack_codes(packed):
    """[rows, K/2] bytes -> [rows, K] 4-bit codes."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty((packed.shape[0], packed.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = packed & 0xF
    out[:, 1::2] = packed >> 4
    return out


def block_scales(m, g):
    """E4M3 block scales for block maxima m (float64 array) under global g:
    RNE_SAT_E4M3(m / (6 g)), 0 where m == 0 or g == 0."""
    m = np.asarray(m, dtype=np.float64)
    gd = float(g)
    if gd <= 0:
        return np.zeros(m.shape, dtype=np.int64)
    s = _rne_sat_codes(m / (6.0 * gd), _E4M3)
    return np.where(m > 0, s, 0)


def encode_elements(x, s, g):
    """4-bit codes of the elements x[..., 16] of blocks with E4M3 scale
    codes s[...] under global g: sign bit | RNE_SAT_E2M1(|x| / (e4m3(s) g)),
    magnitude 0 where e4m3(s) g == 0."""
    x = np.asarray(x, dtype=np.float64)
    den = _E4M3[np.asarray(s, dtype=np.int64)] * float(g)        # exact
    safe = np.where(den > 0, den, 1.0)
    v = np.abs(x) / safe[..., None]
    mag = _rne_sat_codes(v, _E2M1)
    mag = np.where(den[..., None] > 0, mag, 0)
    sign = np.signbit(x).astype(np.int64) << 3
    return (mag | sign).astype(np.uint8)


def quantize(x, g=None, chunk_rows=4096):
    """Quantise a [rows, K] binary32 tensor to NVFP4.

    g=None computes the global from the tensor (self-calibration); otherwise
    g is used as given (a calibrated static global).  Returns
    (codes [rows, K/2] uint8, scales [rows, K/16] uint8, g float32).
    Steps in the order of the definition: global, block maxima, block
    scales, element codes, packing.
    """
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2 or x.shape[1] % BLOCK:
        raise ValueError("x must be [rows, K] with K a multiple of 16")
    if not np.all(np.isfinite(x)):
        raise ValueError("inputs must be finite")
    rows, k = x.shape
    g = global_scale(x) if g is None else np.float32(g)
    if not (np.isfinite(g) and g >= 0):
        raise ValueError("global scale must be finite and >= 0")
    codes = np.empty((rows, k // 2), dtype=np.uint8)
    scales = np.empty((rows, k // BLOCK), dtype=np.uint8)
    for r0 in range(0, rows, chunk_rows):
        xb = x[r0:r0 + chunk_rows].astype(np.float64)
        n = xb.shape[0]
        xb = xb.reshape(n, k // BLOCK, BLOCK)
        m = np.max(np.abs(xb), axis=2)
        s = block_scales(m, g)
        c = encode_elements(xb, s, g).reshape(n, k)
        codes[r0:r0 + n] = pack_codes(c)
        scales[r0:r0 + n] = s.astype(np.uint8)
    return codes, scales, np.float32(g)


def dequantize(codes, scales, g):
    """float64 values sign * E2M1 * E4M3 * g of a packed NVFP4 tensor."""
    c = unpack_codes(codes)
    rows, k = c.shape
    mag = _E2M1[c & 7]
    sgn = np.where(c & 8, -1.0, 1.0)
    sc = e4m3_decode_table()[np.asarray(scales, dtype=np.int64)]
    sc = np.repeat(sc, BLOCK, axis=1)
    return sgn * mag * sc * float(g)


def dequantize_f32(codes, scales, g):
    """binary32 output of the dequantiser: each exact value sign * E2M1 *
    E4M3 * g rounded once to nearest even (numpy's float64 -> float32 cast
    is that rounding; the float64 value is exact, <= 30 significant bits)."""
    return dequantize(codes, scales, g).astype(np.float32)


def dequantize_bf16(codes, scales, g):
    """bfloat16 output of the dequantiser: each exact value rounded once to
    nearest even bfloat16.  Returns the uint16 bit patterns."""
    return bf16_rne_from_f64(dequantize(codes, scales, g))[1]


def error_stats(x, codes, scales, g):
    """Per-row sums behind the A4 / W4 error percentages and the max/RMS
    statistic ([P1] 접근 방법, the input statistics of Table 2; [P3] 前提1
    for max/RMS): float64 [rows, 3] = (sum x^2, sum (x - x_hat)^2, max |x|)
    with x_hat the exact dequantised value.  Relative error of a row or a
    tensor = sqrt(sum of column 1 / sum of column 0); max/RMS of a row =
    column 2 / sqrt(column 0 / K)."""
    x = np.asarray(x, dtype=np.float64)
    d = x - dequantize(codes, scales, g)
    return np.stack([np.sum(x * x, axis=1), np.sum(d * d, axis=1),
                     np.max(np.abs(x), axis=1)], axis=1)


def quantize_exact(x, g=None):
    """Fraction-exact quantisation of a small [rows][K] list of binary32
    values; same outputs as quantize(), computed with no floating point."""
    rows = len(x)
    k = len(x[0]) if rows else 0
    if k % BLOCK:
        raise ValueError("K must be a multiple of 16")
    vals = [[Fraction(float(np.float32(v))) for v in row] for row in x]
    if g is None:
        amax = max((abs(v) for row in vals for v in row), default=Fraction(0))
        g = fp32_rne_exact(amax / GLOBAL_DIVISOR)
    gq = Fraction(float(np.float32(g)))
    codes = []
    scales = []
    for r in range(rows):
        row_codes = []
        row_scales = []
        for b in range(k // BLOCK):
            blk = vals[r][b * BLOCK:(b + 1) * BLOCK]
            m = max(abs(v) for v in blk)
            if m == 0 or gq == 0:
                s = 0
            else:
                s = e4m3_rne_sat_exact(m / (6 * gq))
            d = e4m3_decode(s) * gq
            row_scales.append(s)
            for j, v in enumerate(blk):
                mag = 0 if d == 0 else e2m1_rne_sat_exact(abs(v) / d)
                neg = np.signbit(np.float32(x[r][b * BLOCK + j]))
                row_codes.append(mag | (8 if neg else 0))
        codes.append(row_codes)
        scales.append(row_scales)
    packed = pack_codes(np.array(codes, dtype=np.uint8).reshape(rows, k))
    return packed, np.array(scales, dtype=np.uint8).reshape(rows, k // BLOCK), \
        np.float32(g)
