"""FP8 (OCP E4M3) KV-cache storage with a static per-tensor scale.
TEST INFRASTRUCTURE ONLY (see oracle/__init__.py for the page key).

[P1] 접근 방법 and [P2] abstract: the KV cache is stored in FP8 and a
calibrated static per-tensor scale is shipped with the checkpoint.  The pages
give no formula; readings:

  * E4M3 is the OCP "FN" variant (the one NVFP4 block scales use; max 448);
  * the scale is a decode factor over the calibration data,
    s = RNE_fp32(amax / 448), amax = max |x| over every calibration tensor,
    so the largest calibrated magnitude maps to the largest finite code;
  * stored code = sign(x) | RNE_SAT_E4M3(|x| / s), the quotient exact and
    rounded once, ties to the even code, saturating at 448; magnitude 0
    when s = 0; the sign bit is always copied (so -0.0 gives 0x80);
  * decoded value = e4m3(code) * s.

The float64 tier is exact for the same reason as in quantize.py: |x| has
<= 24 significant bits, s <= 24, an E4M3 midpoint <= 5, so mid * s is exact
in float64 and a quotient that is not a midpoint lies at relative distance
>= 2^-30 from it, far above one float64 division's 2^-53.  amax / 448 =
amax / (7 * 2^6) is either exact in binary32 or a repeating binary fraction
at relative distance >= 2^-30 from every binary32 rounding boundary, so
rounding the float64 quotient to binary32 is one correct rounding.
"""
from fractions import Fraction

import numpy as np

from .formats import e4m3_decode_table, e4m3_rne_sat_exact, fp32_rne_exact

KV_DIVISOR = 448

_E4M3 = e4m3_decode_table()[:127]                 # codes 0x00..0x7E


def kv_amax(tensors):
    """max |x| over a sequence of calibration tensors (binary32 values)."""
    a = 0.0
    for t in tensors:
        t = np.asarray(t, dtype=np.float32)
        if t.size:
            a = max(a, float(np.max(np.abs(t))))
    return np.float32(a)


def kv_scale(amax):
    """Static per-tensor FP8 decode scale RNE_fp32(amax / 448)."""
    return np.float32(float(np.float32(amax)) / float(KV_DIVISOR))


def kv_cast(x, s):
    """FP8 codes (uint8, same shape as x) of binary32 values x under the
    decode scale s: sign | RNE_SAT_E4M3(|x| / s)."""
    x = np.asarray(x, dtype=np.float32)
    s = float(np.float32(s))
    a = np.abs(x.astype(np.float64))
    if s > 0:
        v = a / s
        lo = np.clip(np.searchsorted(_E4M3, v, side="right") - 1, 0, 126)
        hi = np.minimum(lo + 1, 126)
        mid = (_E4M3[lo] + _E4M3[hi]) * 0.5       # exact: few-bit values
        mag = np.where(v < mid, lo, np.where(v > mid, hi, lo + (lo & 1)))
        mag = np.where(lo == 126, 126, mag)
    else:
        mag = np.zeros(x.shape, dtype=np.int64)
    sign = np.signbit(x).astype(np.int64) << 7
    return (mag | sign).astype(np.uint8)


def kv_decode(codes, s):
    """float64 values e4m3(code) * s of FP8 codes."""
    c = np.asarray(codes, dtype=np.int64)
    mag = e4m3_decode_table()[c & 0x7F]
    return np.where(c & 0x80, -1.0, 1.0) * mag * float(np.float32(s))


def kv_cast_exact(x, s):
    """Fraction-exact kv_cast of a small [rows][k] list of binary32 values."""
    sq = Fraction(float(np.float32(s)))
    out = []
    for row in x:
        r = []
        for v in row:
            f = float(np.float32(v))
            mag = 0 if sq == 0 else e4m3_rne_sat_exact(abs(Fraction(f)) / sq)
            r.append(mag | (0x80 if np.signbit(f) else 0))
        out.append(r)
    return out


def kv_scale_exact(amax):
    """Fraction-exact kv_scale."""
    return fp32_rne_exact(Fraction(float(np.float32(amax))) / KV_DIVISOR)
