"""Pins of the CPU oracle against what the pages and mathematics fix.

None of these compare the oracle with itself: they use hand-written golden
values, closed forms, invariants stated on the pages, independent library
routines (torch's float8_e4m3fn and bfloat16 casts, scipy's expit) and brute
force in integer arithmetic.  They run on the CPU.
"""
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import importlib
oq = importlib.import_module("oracle.quantize")
from conftest import read_golden
import synth


def _f32(v):
    return float(np.float32(v))


# --------------------------------------------------------------- formats

def test_e2m1_grid_matches_golden():
    for line in read_golden("e2m1_grid.txt"):
        code, val = line.split()
        got = oracle.e2m1_decode(int(code))
        want = Fraction(val.replace("-0", "0") if val == "-0" else val)
        assert got == want, (code, got, want)
    assert oracle.E2M1_MAG[-1] == 6          # the divisor of "block max / 6"


def test_e4m3_decode_matches_golden_and_torch():
    for line in read_golden("e4m3_values.txt"):
        b, val = line.split()
        got = oracle.e4m3_decode(int(b, 16))
        if val == "nan":
            assert got is None
        else:
            assert got == Fraction(val), (b, got, val)
    # every finite non-negative code against torch's float8_e4m3fn decoder
    codes = torch.arange(0, 127, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    table = oracle.e4m3_decode_table()[:127]
    assert np.array_equal(ref, table)
    assert table.max() == 448 and np.isnan(oracle.e4m3_decode_table()[127])


def test_e4m3_rounding_matches_torch_cast():
    """RNE to E4M3 of binary32 values below the saturation point, against
    torch's float -> float8_e4m3fn cast (round to nearest even)."""
    rng = np.random.default_rng(11)
    v = np.concatenate([
        rng.uniform(0, 464, 20000),
        rng.uniform(0, 2.0 ** -5, 20000),
        np.exp(rng.uniform(np.log(2.0 ** -12), np.log(463.9), 20000)),
        # every midpoint between consecutive codes, and its neighbours
        (oracle.e4m3_decode_table()[:126] + oracle.e4m3_decode_table()[1:127])
        / 2,
    ]).astype(np.float32)
    v = np.concatenate([v, np.nextafter(v, np.float32(0)),
                        np.nextafter(v, np.float32(1000))]).astype(np.float32)
    v = v[v < 464]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oq._rne_sat_codes(v.astype(np.float64), oq._E4M3)
    assert np.array_equal(got, ref.astype(np.int64))
    for x in v[::997]:
        assert oracle.e4m3_rne_sat_exact(Fraction(float(x))) == \
            int(torch.tensor([float(x)]).to(torch.float8_e4m3fn)
                .view(torch.uint8)[0])
    # saturation above 464 (where torch's cast makes NaN instead)
    big = np.array([464.0, 465, 1000, 3e38])
    assert np.all(oq._rne_sat_codes(big, oq._E4M3) == 0x7E)
    assert oracle.e4m3_rne_sat_exact(Fraction(464)) == 0x7E   # tie -> 448
    assert oracle.e4m3_rne_sat_exact(Fraction(10 ** 9)) == 0x7E


def test_fp32_rne_exact_against_numpy_cast():
    rng = np.random.default_rng(5)
    xs = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(
        -40, 38, 3000), [1e-46, 7e-46, 2.0 ** -150, 3 * 2.0 ** -151,
                         3.4028235e38, 3.4028236e38]])
    for x in xs:
        with np.errstate(over="ignore"):
            want = float(np.float32(x))      # numpy: RNE double -> single
        assert oracle.fp32_rne_exact(Fraction(float(x))) == want, x


def test_bf16_rne_against_torch():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal(100000) * 10.0 ** rng.integers(-30, 30, 100000)
         ).astype(np.float32)
    # exact ties: bf16 values plus half an ulp
    t = (np.arange(1, 2000, dtype=np.uint32) << 16) | np.uint32(0x8000)
    x = np.concatenate([x, t.view(np.float32), -t.view(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got, bits = oracle.bf16_rne_from_f64(x.astype(np.float64))
    assert np.array_equal(got, ref)
    ref_bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)
    assert np.array_equal(bits, ref_bits)


# ------------------------------------------------------ worked examples

def _parse_block(line):
    head, xs, sc, packed = [p.strip() for p in line.split("|")]
    mode, g = head.split()
    xv = np.array([np.float32(float(v)) for v in xs.split()], dtype=np.float32)
    return mode, float(g), xv, int(sc, 16), bytes(int(b, 16) for b in
                                                  packed.split())


def test_worked_blocks_golden():
    lines = read_golden("worked_blocks.txt")
    assert len(lines) == 9
    for line in lines:
        mode, g, x, sc, packed = _parse_block(line)
        gg = None if mode == "compute" else g
        codes, scales, gout = oracle.quantize(x[None, :], g=gg)
        assert scales[0, 0] == sc, line
        assert bytes(codes[0]) == packed, line
        ce, se, ge = oracle.quantize_exact([list(x)], g=gg)
        assert np.array_equal(ce, codes) and np.array_equal(se, scales)
        assert ge == gout
    # "-0" in the fixture really is a negative zero
    assert np.signbit(_parse_block(lines[0])[2][4])


# ------------------------------------------------ invariants of the pages

def test_scale_tracks_block_max_over_6():
    """[P3] 前提1: the block scale is the block maximum over 6 (times the
    global): within E4M3's relative rounding of 2^-4 while normal and not
    saturated, and the block's maximum element always encodes to +-6."""
    x, _, _ = synth.workload_tensor(2, "x", row_ids=np.arange(64))
    codes, scales, g = oracle.quantize(x)
    m = np.max(np.abs(x.reshape(64, -1, 16)), axis=2)
    d = oracle.e4m3_decode_table()[scales] * float(g)
    normal = (scales >= 8) & (scales < 0x7E)
    rel = np.abs(d - m / 6) / (m / 6)
    assert normal.mean() > 0.99
    assert np.all(rel[normal] <= 2.0 ** -4)
    c = oracle.unpack_codes(codes).reshape(64, -1, 16)
    amax_idx = np.argmax(np.abs(x.reshape(64, -1, 16)), axis=2)
    top = np.take_along_axis(c, amax_idx[..., None], axis=2)[..., 0]
    assert np.all((top & 7) == 7)
    # the tensor's largest block gets the largest finite scale, 448
    assert scales.max() == 0x7E


def test_block_max_over_rms_at_most_4_and_one_hot():
    """[P3] 前提1: inside a 16-element block max/RMS <= sqrt(16) = 4, with
    equality exactly for a one-hot block, which quantises to one +-6 and
    fifteen zeros."""
    x, _, _ = synth.workload_tensor(3, "x", row_ids=np.arange(256))
    b = x.reshape(-1, 16).astype(np.float64)
    ratio = np.max(np.abs(b), axis=1) / np.sqrt(np.mean(b * b, axis=1))
    assert np.all(ratio <= 4.0 + 1e-12)
    one = np.zeros((1, 32), dtype=np.float32)
    one[0, 5] = -3.7
    one[0, 16 + 9] = 120.0
    bb = one.reshape(-1, 16).astype(np.float64)
    r = np.max(np.abs(bb), axis=1) / np.sqrt(np.mean(bb * bb, axis=1))
    assert np.all(r == 4.0)
    codes, scales, g = oracle.quantize(one)
    c = oracle.unpack_codes(codes)[0]
    assert c[5] == 0xF and c[25] == 0x7
    assert np.count_nonzero(c) == 2


def test_outlier_is_local_to_its_block():
    """[P3] 前提1: an outlier can only damage its own block (itself and 15
    neighbours).  With the global held fixed, multiplying one element by 60
    changes only that block's scale and codes."""
    x, _, _ = synth.workload_tensor(2, "x", row_ids=np.arange(8))
    g = oracle.global_scale(x) * np.float32(64)
    c0, s0, _ = oracle.quantize(x, g=g)
    y = x.copy()
    y[3, 1000] *= np.float32(60)
    c1, s1, _ = oracle.quantize(y, g=g)
    u0, u1 = oracle.unpack_codes(c0), oracle.unpack_codes(c1)
    diff_blocks = set(np.nonzero((u0 != u1).reshape(8, -1, 16).any(2)
                                 | (s0 != s1))[1].tolist())
    diff_rows = set(np.nonzero((u0 != u1).any(1) | (s0 != s1).any(1))[0])
    assert diff_rows == {3} and diff_blocks == {1000 // 16}


def test_round_trip_on_grid_values():
    """Values already on the NVFP4 grid, with every block holding a +-6 code
    and the tensor max equal to 2688 * g for g = 2^e, quantise back to the
    same codes, scales and global, bit for bit."""
    rng = np.random.default_rng(3)
    rows, k, e = 8, 256, -7
    s = rng.integers(1, 0x7E, size=(rows, k // 16))
    s[0, 0] = 0x7E
    c = rng.integers(0, 16, size=(rows, k)).astype(np.uint8)
    c.reshape(rows, -1, 16)[:, :, 3] = 7 | (rng.integers(0, 2, (rows, k // 16))
                                           << 3).astype(np.uint8)
    packed = oracle.pack_codes(c)
    g = np.float32(2.0 ** e)
    x = oracle.dequantize(packed, s.astype(np.uint8), g)
    assert np.array_equal(x.astype(np.float32).astype(np.float64), x)
    c2, s2, g2 = oracle.quantize(x.astype(np.float32))
    assert g2 == g
    assert np.array_equal(s2, s.astype(np.uint8))
    # zero magnitudes round-trip to +0 / -0 with their sign
    assert np.array_equal(c2, packed)


# ---------------------------------------------------------- brute force

def _bf16_nonneg_finite():
    bits = np.arange(0, 0x7F80, dtype=np.uint32)
    return (bits << 16).view(np.float32)


def test_e2m1_encode_brute_force_every_bf16_every_scale():
    """Every finite bf16 value (both signs) under every nonzero E4M3 scale
    with g = 1: the code is the nearest of the 8 magnitudes found by
    exhaustive comparison in exact integer arithmetic (ties to the even
    code; beyond 6 saturates)."""
    x = _bf16_nonneg_finite().astype(np.float64)
    mant, ex = np.frexp(x)                      # x = mant * 2^ex
    X = np.rint(np.ldexp(mant, 24)).astype(np.int64)   # x = X * 2^(ex-24)
    halves = np.array([0, 1, 2, 3, 4, 6, 8, 12], dtype=np.int64)
    for s in range(1, 0x7F):
        D = int(oracle.e4m3_decode(s) * 512)     # dec(s) = D * 2^-9
        v = x / (D / 512.0)
        want = np.zeros(x.shape, dtype=np.int64)
        want[v > 64] = 7
        mid = (v >= 2.0 ** -6) & (v <= 64)
        # v = X 2^(ex-24+9) / D; compare 2 v with halves_j:
        # |2 X 2^(ex-15) - h_j D| scaled by 2^sh to integers
        e2 = ex[mid] - 15 + 1
        sh = np.maximum(-e2, 0)
        lhs = X[mid] << np.maximum(e2, 0)
        rhs = halves[None, :] * D * (np.int64(1) << sh)[:, None]
        dist = np.abs(lhs[:, None] - rhs)
        best = np.argmin(dist, axis=1)
        # ties: argmin takes the first (lower) index; move odd winners up
        # when the next grid point is equally near
        nxt = np.minimum(best + 1, 7)
        tie = (dist[np.arange(len(best)), nxt] == dist[np.arange(len(best)),
                                                        best]) & (nxt != best)
        best = np.where(tie & (best % 2 == 1), nxt, best)
        want[mid] = best
        got = oracle.encode_elements(x.reshape(1, -1, 1),
                                     np.full((1, x.size), s), 1.0).reshape(-1)
        assert np.array_equal(got, want), s
        gotn = oracle.encode_elements(-x.reshape(1, -1, 1),
                                      np.full((1, x.size), s), 1.0).reshape(-1)
        assert np.array_equal(gotn, want | 8), s


def test_e4m3_scale_brute_force_every_bf16_max():
    """Every positive finite bf16 block maximum m with g = 1: the scale is
    the nearest of the 127 E4M3 values to m / 6 by exhaustive comparison in
    exact integer arithmetic (ties to even, saturating at 448)."""
    m = _bf16_nonneg_finite()[1:].astype(np.float64)
    mant, ex = np.frexp(m)
    X = np.rint(np.ldexp(mant, 24)).astype(np.int64)   # m = X 2^(ex-24)
    U = np.array([int(v * 512) for v in oracle.formats.E4M3_POS],
                 dtype=np.int64)                       # E4M3 = U 2^-9
    v = m / 6
    want = np.zeros(m.shape, dtype=np.int64)
    want[v > 1024] = 0x7E
    mid = (v >= 2.0 ** -14) & (v <= 1024)
    # compare m/6 with U 2^-9  <=>  X 2^(ex-24+9) with 6 U
    e2 = ex[mid] - 15
    sh = np.maximum(-e2, 0)
    lhs = X[mid] << np.maximum(e2, 0)
    best = np.empty(mid.sum(), dtype=np.int64)
    for i0 in range(0, len(lhs), 4096):
        sl = slice(i0, i0 + 4096)
        rhs = 6 * U[None, :] * (np.int64(1) << sh[sl])[:, None]
        dist = np.abs(lhs[sl, None] - rhs)
        b = np.argmin(dist, axis=1)
        nxt = np.minimum(b + 1, 126)
        r = np.arange(len(b))
        tie = (dist[r, nxt] == dist[r, b]) & (nxt != b)
        best[sl] = np.where(tie & (b % 2 == 1), nxt, b)
    want[mid] = best
    got = oracle.block_scales(m, 1.0)
    assert np.array_equal(got, want)


# --------------------------------------------------- tier cross-checks

def _adversarial_blocks(rng, n):
    """Blocks whose maxima sit on E4M3 midpoints times 6g and whose elements
    sit on E2M1 midpoints times the resulting scale, plus neighbours."""
    out = []
    e4 = oracle.e4m3_decode_table()[:127]
    e2 = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    for _ in range(n):
        g = np.float32(2.0 ** rng.integers(-8, 4))
        j = rng.integers(0, 126)
        m = np.float32(6 * g * (e4[j] + e4[j + 1]) / 2)
        m = [m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(1e9))
             ][rng.integers(0, 3)]
        s = oracle.block_scales(np.array([m]), g)[0]
        d = e4[s] * g
        blk = np.float32(d) * e2[rng.integers(0, 7, 16)].astype(np.float32)
        blk = np.where(rng.random(16) < 0.3, np.nextafter(blk, np.float32(9)),
                       blk)
        blk = blk * np.where(rng.random(16) < 0.5, -1, 1).astype(np.float32)
        blk[rng.integers(0, 16)] = m
        out.append((blk.astype(np.float32), g))
    return out


def test_fast_tier_equals_exact_tier():
    rng = np.random.default_rng(7)
    # random tensors of several magnitudes, self-calibrated and given
    for trial in range(12):
        scale = 10.0 ** rng.uniform(-30, 30)
        x = (rng.standard_normal((3, 32)) * scale).astype(np.float32)
        x[rng.random(x.shape) < 0.1] = 0
        if trial % 3 == 0:
            x[0, :16] = -0.0
        for g in (None, oracle.global_scale(x) * np.float32(
                rng.uniform(0.01, 5))):
            cf, sf, gf = oracle.quantize(x, g=g)
            ce, se, ge = oracle.quantize_exact(x.tolist(), g=g)
            assert np.array_equal(cf, ce) and np.array_equal(sf, se)
            assert gf == ge
    for blk, g in _adversarial_blocks(rng, 300):
        cf, sf, _ = oracle.quantize(blk[None, :], g=g)
        ce, se, _ = oracle.quantize_exact([blk.tolist()], g=g)
        assert np.array_equal(cf, ce) and np.array_equal(sf, se)


def test_global_scale_is_one_correct_rounding():
    rng = np.random.default_rng(9)
    for a in np.concatenate([rng.standard_normal(2000).astype(np.float32)
                             * np.float32(10.0) ** rng.integers(-40, 38, 2000),
                             [2688, 1, 2.0 ** -149, 3e38, 21 * 2.0 ** -100]]):
        a = np.float32(abs(a))
        if not np.isfinite(a):
            continue
        want = oracle.fp32_rne_exact(Fraction(float(a)) / 2688)
        assert float(oracle.global_scale(np.array([a]))) == want


# ------------------------------------------------------------ harmonize

def _fused_group(rng, sizes=(40, 24, 8), k=64, sig=(0.02, 0.05, 0.2)):
    mods = [(rng.standard_normal((r, k)) * s).astype(np.float32)
            for r, s in zip(sizes, sig)]
    q = [oracle.quantize(m) for m in mods]
    codes = np.concatenate([c for c, _, _ in q])
    scales = np.concatenate([s for _, s, _ in q])
    gs = [g for _, _, g in q]
    offs = [0] + list(np.cumsum(sizes))
    return mods, codes, scales, gs, offs


def test_harmonize_identities():
    rng = np.random.default_rng(21)
    _, codes, scales, gs, offs = _fused_group(rng)
    # one module, or all globals equal: nothing changes
    s1, g1 = oracle.harmonize(scales[:40], [0, 40], [gs[0]])
    assert np.array_equal(s1, scales[:40]) and g1 == gs[0]
    s2, g2 = oracle.harmonize(scales, offs, [gs[0]] * 3)
    assert np.array_equal(s2, scales) and g2 == gs[0]
    # ratios that are exact powers of two: scales shift by exact exponents
    # and the dequantised weights are bit-identical
    g = np.float32(0.25)
    sub = scales[:40].copy()
    sub = np.clip(sub, 0x20, 0x60).astype(np.uint8)
    both = np.concatenate([sub, sub])
    sh, gstar = oracle.harmonize(both, [0, 40, 80], [g, g * np.float32(4)])
    assert gstar == np.float32(1.0)
    assert np.array_equal(sh[:40], sub - 16)          # /4 = exponent - 2
    assert np.array_equal(sh[40:], sub)
    w_before = oracle.dequantize(codes[:40], sub, g)
    w_after = oracle.dequantize(codes[:40], sh[:40], gstar)
    assert np.array_equal(w_before, w_after)


def test_harmonize_bound_and_mismatch_closed_form():
    rng = np.random.default_rng(22)
    mods, codes, scales, gs, offs = _fused_group(rng)
    new, gstar = oracle.harmonize(scales, offs, gs)
    assert gstar == max(gs)
    # per block, the folded scale moves the dequantised block by at most
    # E4M3's relative rounding (2^-4) while normal
    e4 = oracle.e4m3_decode_table()
    for i in range(3):
        r = slice(offs[i], offs[i + 1])
        before = e4[scales[r]] * float(gs[i])
        after = e4[new[r]] * float(gstar)
        ok = new[r] >= 8
        assert np.all(np.abs(after[ok] - before[ok]) <= 2.0 ** -4 *
                      before[ok])
    # the bug the fix repairs: serving module i's unfolded scales with the
    # shared global multiplies its outputs by exactly g*/g_i
    x = rng.standard_normal((4, 64)).astype(np.float32)
    xc, xs, xg = oracle.quantize(x)
    wrong = oracle.gemm_exact_int(xc, xs, xg, codes, scales, gstar)
    right_i = [oracle.gemm_exact_int(xc, xs, xg, codes[offs[i]:offs[i + 1]],
                                     scales[offs[i]:offs[i + 1]], gs[i])
               for i in range(3)]
    for i in range(3):
        ratio = wrong[:, offs[i]:offs[i + 1]] / right_i[i]
        assert np.allclose(ratio, float(gstar) / float(gs[i]), rtol=1e-12)
    # after the fix the fused GEMM agrees with the per-module GEMMs up to
    # the one scale rounding (<= 2^-4 per block, far less on average)
    fixed = oracle.gemm_exact_int(xc, xs, xg, codes, new, gstar)
    ref = np.concatenate(right_i, axis=1)
    err = np.linalg.norm(fixed - ref) / np.linalg.norm(ref)
    assert err < 2.0 ** -5


def test_harmonize_fast_equals_exact():
    rng = np.random.default_rng(23)
    for _ in range(5):
        _, _, scales, gs, offs = _fused_group(
            rng, sizes=(3, 2, 4), k=32,
            sig=tuple(10.0 ** rng.uniform(-3, 1, 3)))
        a, ga = oracle.harmonize(scales, offs, gs)
        b, gb = oracle.harmonize_exact(scales, offs, gs)
        assert np.array_equal(a, b) and ga == gb
    # adversarial: every scale byte against ratios that put products on
    # E4M3 midpoints
    allb = np.arange(0, 0x7F, dtype=np.uint8).reshape(1, -1)
    for gi in (np.float32(0.5), np.float32(0.75), np.float32(0.5625),
               np.float32(1 / 3)):
        sc = np.concatenate([allb, allb])
        a, _ = oracle.harmonize(sc, [0, 1, 2], [gi, np.float32(1)])
        b, _ = oracle.harmonize_exact(sc, [0, 1, 2], [gi, np.float32(1)])
        assert np.array_equal(a, b)


# ------------------------------------------------------------------ gemm

def test_gemm_unit_scales_is_integer_matmul():
    """All block scales 1.0 and globals 1: the W4A4 GEMM reduces to a matrix
    product of the E2M1 values, checked against a plain triple loop."""
    rng = np.random.default_rng(31)
    m, n, k = 5, 7, 48
    ca = rng.integers(0, 16, (m, k)).astype(np.uint8)
    cb = rng.integers(0, 16, (n, k)).astype(np.uint8)
    one = np.full((m, k // 16), 0x38, np.uint8)
    oneb = np.full((n, k // 16), 0x38, np.uint8)
    y = oracle.gemm_exact_int(oracle.pack_codes(ca), one, 1.0,
                              oracle.pack_codes(cb), oneb, 1.0)
    val = [float(oracle.e2m1_decode(c)) for c in range(16)]
    for i in range(m):
        for j in range(n):
            ref = sum(val[ca[i, t]] * val[cb[j, t]] for t in range(k))
            assert y[i, j] == ref


def test_gemm_int_equals_f64_blas_and_concatenation():
    rng = np.random.default_rng(32)
    x = (rng.standard_normal((16, 256))).astype(np.float32)
    w1 = (rng.standard_normal((24, 256)) * 0.02).astype(np.float32)
    w2 = (rng.standard_normal((40, 256)) * 0.02).astype(np.float32)
    xq = oracle.quantize(x)
    g = oracle.global_scale(np.concatenate([w1, w2]))
    q1 = oracle.quantize(w1, g=g)
    q2 = oracle.quantize(w2, g=g)
    yi = oracle.gemm_exact_int(*xq, *q1)
    yf = oracle.gemm_f64(*xq, *q1)
    assert np.max(np.abs(yi - yf)) <= 1e-12 * np.max(np.abs(yi))
    # dequantise-then-matmul (a library matmul on the decoded values)
    ref = oracle.dequantize(*xq) @ oracle.dequantize(*q1).T
    assert np.allclose(yi, ref, rtol=1e-12, atol=0)
    # concatenating weights that share a global concatenates the outputs
    cat = oracle.gemm_exact_int(*xq, np.concatenate([q1[0], q2[0]]),
                                np.concatenate([q1[1], q2[1]]), g)
    y2 = oracle.gemm_exact_int(*xq, *q2)
    assert np.array_equal(cat, np.concatenate([yi, y2], axis=1))
    # sampled rows/columns equal the full product's entries
    sub = oracle.gemm_f64_rows_cols(*xq, *q1, [3, 9], [0, 5, 23])
    assert np.array_equal(sub, yf[np.ix_([3, 9], [0, 5, 23])])


def test_gemm_row_blocks_cover_the_exact_product():
    """The row-block generator used for full-size checks yields every row
    once, in order, each block within float64 accumulation error of the
    exact integer product (and ragged last block included)."""
    rng = np.random.default_rng(33)
    x = rng.standard_normal((37, 512)).astype(np.float32)
    w = (rng.standard_normal((21, 512)) * 0.05).astype(np.float32)
    xq, wq = oracle.quantize(x), oracle.quantize(w)
    yi = oracle.gemm_exact_int(*xq, *wq)
    seen = []
    for r0, yb in oracle.gemm_f64_row_blocks(*xq, *wq, rows_per_block=8):
        seen.append((r0, yb.shape[0]))
        assert np.max(np.abs(yb - yi[r0:r0 + yb.shape[0]])) <= \
            1e-12 * np.max(np.abs(yi))
    assert seen == [(0, 8), (8, 8), (16, 8), (24, 8), (32, 5)]


def test_gates_closed_forms():
    """[P3] 前提2: alpha goes through softplus and exp, beta through a
    sigmoid.  alpha = exp(-softplus(y)) = sigmoid(-y) = 1 - beta; both are
    1/2 at 0 and monotone; checked against scipy's expit."""
    y = np.linspace(-40, 40, 20001)
    a = oracle.gate_alpha(y)
    b = oracle.gate_beta(y)
    assert np.allclose(a, scipy.special.expit(-y), rtol=1e-13, atol=0)
    assert np.allclose(b, scipy.special.expit(y), rtol=1e-13, atol=0)
    assert np.max(np.abs(a + b - 1)) < 1e-15
    assert oracle.gate_alpha(0.0) == 0.5 and oracle.gate_beta(0.0) == 0.5
    assert np.all(np.diff(a) <= 0) and np.all(np.diff(b) >= 0)
    inner = np.abs(y[:-1]) < 20
    assert np.all(np.diff(a)[inner] < 0) and np.all(np.diff(b)[inner] > 0)


def test_sanity_band_of_round_trip_error():
    """Not a gate: the NVFP4 round-trip relative error on these synthetic
    activations is of the order the pages report for real GDN inputs
    (a few to ten percent)."""
    x, _, _ = synth.workload_tensor(2, "x", row_ids=np.arange(128))
    q = oracle.quantize(x)
    err = np.linalg.norm(oracle.dequantize(*q) - x) / np.linalg.norm(x)
    assert 0.03 < err < 0.15


# ------------------------------------------------- dequantise and error stats

def _exact_values(codes, scales, g):
    """Fraction value of every element, from the bit layouts alone."""
    c = oracle.unpack_codes(codes)
    out = []
    for r in range(c.shape[0]):
        row = []
        for i in range(c.shape[1]):
            code = int(c[r, i])
            mag = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2),
                   Fraction(2), Fraction(3), Fraction(4), Fraction(6)][code & 7]
            sb = int(scales[r, i // 16])
            e, mnt = sb >> 3, sb & 7
            sc = (Fraction(mnt, 8) * Fraction(2) ** -6 if e == 0
                  else (1 + Fraction(mnt, 8)) * Fraction(2) ** (e - 7))
            row.append((-1 if code & 8 else 1) * mag * sc * Fraction(float(g)))
        out.append(row)
    return out


def _bf16_rne_fraction(q):
    """Nearest-even bfloat16 of a rational (8 significant bits, quantum
    floor 2^-133), as a Fraction; written from the format, not the oracle."""
    if q == 0:
        return Fraction(0)
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    quantum = Fraction(2) ** max(e - 7, -133)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return (1 if q > 0 else -1) * fl * quantum


@pytest.mark.parametrize("g", [0.011, 2.0 ** -140, 3.0e-41, 1.25e30])
def test_dequantize_roundings_against_fractions(g):
    """binary32 and bfloat16 outputs are single roundings of the exact
    products, including products in the subnormal range."""
    rng = np.random.default_rng(17)
    rows, k = 3, 64
    codes = rng.integers(0, 256, size=(rows, k // 2)).astype(np.uint8)
    scales = rng.integers(0, 0x7F, size=(rows, k // 16)).astype(np.uint8)
    g = np.float32(g)
    exact = _exact_values(codes, scales, g)
    f32 = oracle.dequantize_f32(codes, scales, g)
    b16 = oracle.dequantize_bf16(codes, scales, g)
    for r in range(rows):
        for i in range(k):
            assert float(f32[r, i]) == oq.fp32_rne_exact(exact[r][i]) or \
                (exact[r][i] == 0 and f32[r, i] == 0)
            want = _bf16_rne_fraction(exact[r][i])
            got = (np.uint32(b16[r, i]) << 16).view(np.float32)
            assert Fraction(float(got)) == want


def test_error_stats_against_fractions_and_invariants():
    """Row sums equal their Fraction-exact values; values on the grid have
    zero error; a one-hot row of one block has max/RMS exactly 4."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((4, 32)) * 3).astype(np.float32)
    c, s, g = oracle.quantize(x)
    st = oracle.error_stats(x, c, s, g)
    xh = _exact_values(c, s, g)
    for r in range(4):
        xs = [Fraction(float(v)) for v in x[r]]
        sx = sum(v * v for v in xs)
        se = sum((v - w) ** 2 for v, w in zip(xs, xh[r]))
        assert abs(Fraction(st[r, 0]) - sx) <= sx * Fraction(1, 2 ** 50)
        assert abs(Fraction(st[r, 1]) - se) <= se * Fraction(1, 2 ** 40)
        assert st[r, 2] == max(abs(float(v)) for v in x[r])
    g2 = np.float32(2.0 ** -7)   # products exact in binary32
    xg = oracle.dequantize(c, s, g2)
    assert np.array_equal(xg.astype(np.float32).astype(np.float64), xg)
    assert np.all(oracle.error_stats(xg.astype(np.float32), c, s, g2)[:, 1] == 0.0)
    one = np.zeros((1, 16), dtype=np.float32)
    one[0, 5] = -3.5
    c1, s1, g1 = oracle.quantize(one)
    st1 = oracle.error_stats(one, c1, s1, g1)
    assert st1[0, 2] / np.sqrt(st1[0, 0] / 16) == 4.0


def test_gdn_gates_closed_forms_and_scalar_math():
    """The full gate pair: with A_log = dt_bias = 0 alpha is the
    exp(-softplus) gate; point values against Python's math module term by
    term; limits and monotonicity in A_log and dt_bias."""
    import math
    rng = np.random.default_rng(2)
    y = rng.standard_normal((5, 7)) * 4
    b0, a0 = oracle.gdn_gates(y, 3, np.zeros(4), np.zeros(4))
    assert np.array_equal(a0, oracle.gate_alpha(y[:, 3:]))
    assert np.allclose(b0, scipy.special.expit(y[:, :3]), rtol=1e-15, atol=0)
    a_log = np.array([-1.5, 0.0, 0.7, 2.0])
    dt = np.array([0.3, -2.0, 1.1, 0.0])
    _, a = oracle.gdn_gates(y, 3, a_log, dt)
    for i in range(5):
        for j in range(4):
            x = y[i, 3 + j] + dt[j]
            sp = x + math.log1p(math.exp(-x)) if x > 0 else math.log1p(math.exp(x))
            want = math.exp(-math.exp(a_log[j]) * sp)
            assert abs(a[i, j] - want) <= 1e-14 * want
    _, half = oracle.gdn_gates(np.zeros((1, 2)), 1, np.zeros(1), np.zeros(1))
    assert half[0, 0] == 0.5
    _, near1 = oracle.gdn_gates(np.zeros((1, 2)), 1, np.array([-60.0]), np.zeros(1))
    assert 1 - 1e-12 < near1[0, 0] <= 1.0
    _, lo = oracle.gdn_gates(y, 3, a_log, dt)
    _, hi = oracle.gdn_gates(y, 3, a_log + 0.5, dt)
    assert np.all(hi <= lo)          # larger A_log forgets faster
    _, more = oracle.gdn_gates(y, 3, a_log, dt + 0.5)
    assert np.all(more <= lo)        # larger bias forgets faster


# --------------------------------------------------- FP8 KV static scales

def test_kv_cast_matches_torch_float8_in_range():
    """With s = 2^e the codes are torch's float8_e4m3fn cast of x / 2^e
    (exact scaling), for every in-range bf16 value and both signs."""
    mags = _bf16_nonneg_finite()
    for e in (0, -5, 7):
        s = np.float32(2.0 ** e)
        v = mags[mags <= 448 * float(s)]
        x = np.concatenate([v, -v]).astype(np.float32)
        ref = torch.from_numpy(x / np.float32(s)).to(torch.float8_e4m3fn) \
            .view(torch.uint8).numpy()
        got = oracle.kv_cast(x, s)
        # torch keeps -0 as 0x80 like the oracle; compare everything
        assert np.array_equal(got, ref), e


def test_kv_cast_fast_equals_exact_with_midpoints_and_saturation():
    rng = np.random.default_rng(8)
    s = np.float32(0.0137)
    mids = [(oracle.e4m3_decode(c) + oracle.e4m3_decode(c + 1)) / 2
            for c in range(0, 126, 7)]
    x = [float(np.float32(float(m) * float(s))) for m in mids]
    x += list((rng.standard_normal(200) * 3).astype(np.float32))
    x += [1e6, -1e6, 0.0, -0.0, 448 * float(s), 1e-30]
    x = np.array(x, dtype=np.float32)[None, :]
    assert np.array_equal(oracle.kv_cast(x, s),
                          np.array(oracle.kv_cast_exact(x.tolist(), s), dtype=np.uint8))
    c = oracle.kv_cast(x, s)[0]
    assert c[-6] == 0x7E and c[-5] == 0xFE and c[-4] == 0x00 and c[-3] == 0x80
    assert np.all(oracle.kv_cast(x, 0.0) & 0x7F == 0)


def test_kv_scale_is_one_correct_rounding_and_maps_amax_to_448():
    rng = np.random.default_rng(4)
    a = np.concatenate([rng.random(2000) * 1e3, rng.random(200) * 1e-40,
                        [448.0, 1.0, 3.0 * 2 ** -140]]).astype(np.float32)
    for v in a:
        assert float(oracle.kv_scale(v)) == oracle.kv_scale_exact(v)
    x = (rng.standard_normal((16, 64)) * 5).astype(np.float32)
    s = oracle.kv_scale(oracle.kv_amax([x[:8], x[8:]]))
    assert oracle.kv_amax([x[:8], x[8:]]) == np.max(np.abs(x))
    c = oracle.kv_cast(x, s)
    assert np.max(c & 0x7F) == 0x7E               # the largest magnitude saturates at 448
    rel = np.linalg.norm(oracle.kv_decode(c, s) - x) / np.linalg.norm(x)
    assert rel < 2 ** -4                           # 3 mantissa bits
