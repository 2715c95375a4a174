"""Number formats of NVFP4, decoded from their bit layouts, and exact rounding.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py for the page key).

[P3] "前提1" and [P1] "접근 방법" define an NVFP4 tensor as E2M1 4-bit values
(1 sign, 2 exponent, 1 mantissa bit), one E4M3 scale per 16-element block and
one FP32 scale per tensor.  The pages give the bit split but not the decoded
values; they are derived here from the layouts:

  E2M1: exponent bias 1, exponent field 0 is subnormal, no inf/NaN.  The
        magnitudes are {0, 0.5, 1, 1.5, 2, 3, 4, 6}; the largest, 6, is the
        divisor in "block max / 6" of [P3] "前提1".
  E4M3: the OCP "FN" variant (bias 7, subnormals m/8 * 2^-6, no inf, only
        S.1111.111 is NaN, largest finite 448), the variant NVFP4 block scales
        use.  Reading: the pages say "E4M3" only; the FNUZ variant (max 240)
        is not meant.

Rounding (the pages say only "round to 4 bits"; reading): round-to-nearest,
ties to the even code, saturating at the largest finite value.  Exact
versions here work on fractions.Fraction.
"""
from fractions import Fraction

import numpy as np

# Reading of the FP32 per-tensor scale (the pages do not give its formula):
# the stored scale g is a *decode* factor, g = amax / (6 * 448), so that the
# block holding the tensor's largest magnitude gets the largest finite E4M3
# scale and every dequantised value is e2m1 * e4m3 * g.
GLOBAL_DIVISOR = 6 * 448


def e2m1_decode(code):
    """Value of a 4-bit E2M1 code (bit 3 sign, bits 2..1 exponent, bit 0
    mantissa), as a Fraction.  Bit layout from [P3] "前提1"."""
    if not 0 <= code < 16:
        raise ValueError("E2M1 code out of range")
    sign = -1 if code & 8 else 1
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:                      # subnormal: 2^(1-bias) * (m/2), bias 1
        mag = Fraction(m, 2)
    else:
        mag = Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))
    return sign * mag


# Non-negative E2M1 magnitudes indexed by the 3-bit magnitude code.
E2M1_MAG = tuple(e2m1_decode(c) for c in range(8))


def e4m3_decode(byte):
    """Value of an OCP E4M3FN byte as a Fraction; None for the NaN codes."""
    if not 0 <= byte < 256:
        raise ValueError("E4M3 byte out of range")
    sign = -1 if byte & 0x80 else 1
    e = (byte >> 3) & 15
    m = byte & 7
    if e == 15 and m == 7:
        return None
    if e == 0:
        mag = Fraction(m, 8) * Fraction(1, 2 ** 6)
    else:
        mag = (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return sign * mag


# The 127 finite non-negative E4M3 values, indexed by code 0x00..0x7E.
E4M3_POS = tuple(e4m3_decode(b) for b in range(0x7F))


def e4m3_decode_table():
    """float64 array of the 128 non-negative E4M3 codes (NaN at 0x7F)."""
    t = np.array([float(v) for v in E4M3_POS] + [np.nan], dtype=np.float64)
    return t


def _round_to_grid(v, grid):
    """Index of the RNE-saturating rounding of v >= 0 onto `grid`, a tuple of
    increasing Fractions whose index is the code (so "even" = even index)."""
    if v < 0:
        raise ValueError("magnitude must be non-negative")
    if v >= grid[-1]:
        return len(grid) - 1
    lo = 0
    while grid[lo + 1] <= v:
        lo += 1
    below = v - grid[lo]
    above = grid[lo + 1] - v
    if below < above:
        return lo
    if above < below:
        return lo + 1
    return lo if lo % 2 == 0 else lo + 1


def e2m1_rne_sat_exact(v):
    """E2M1 magnitude code (0..7) of the exact non-negative rational v."""
    return _round_to_grid(Fraction(v), E2M1_MAG)


def e4m3_rne_sat_exact(v):
    """E4M3 code (0x00..0x7E) of the exact non-negative rational v."""
    return _round_to_grid(Fraction(v), E4M3_POS)


def _rne_int(q):
    """Round a non-negative Fraction to the nearest integer, ties to even."""
    n = q.numerator // q.denominator
    r = q - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n


def fp32_rne_exact(q):
    """IEEE binary32 round-to-nearest-even of the rational q, with gradual
    underflow; returned as a Python float (binary32 is a subset of binary64).
    Overflow gives +-inf."""
    q = Fraction(q)
    if q == 0:
        return 0.0
    sign = -1.0 if q < 0 else 1.0
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1                       # now 2^e <= a < 2^(e+1)
    quantum_exp = max(e - 23, -149)
    n = _rne_int(a / Fraction(2) ** quantum_exp)
    val = Fraction(n) * Fraction(2) ** quantum_exp
    if val >= Fraction(2) ** 128:
        return sign * float("inf")
    return sign * float(val)


def bf16_rne_from_f64(y):
    """Round float64 values to bfloat16 (8 significant bits, binary32 exponent
    range, gradual underflow to 2^-133), ties to even.  Returns (values as
    float64, bf16 bit patterns as uint16)."""
    y = np.asarray(y, dtype=np.float64)
    _, e = np.frexp(y)                       # y = m * 2^e, 0.5 <= |m| < 1
    qexp = np.maximum(e - 8, -133)
    r = np.ldexp(np.rint(np.ldexp(y, -qexp)), qexp)
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, y), r)
    bits = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return r, bits
