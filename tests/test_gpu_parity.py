"""Parity of the HIP library (through its C ABI) with the CPU oracle.

Bars: NVFP4 codes, scales and globals bit-exact; GEMM fp32 output within
relative Frobenius error 1e-5 of the exact oracle; bf16 output within one
bf16 ulp of the oracle rounded to bf16; gates within 1e-5 relative
Frobenius.  Small cases are compared element by element in full; the
full-size workloads run in the launch configuration the benchmark uses and
are checked on sampled rows/columns that the oracle computes one by one.
"""
import functools

import numpy as np
import pytest
import torch

import nvfp4_w4a4_quantized_03_amd as nv
import oracle
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 1e-5


def _say(*a):
    print("[gpu-parity]", *a, flush=True)


def up(vals, bits, dtype):
    """Host tensor -> device tensor with identical bits."""
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(vals)).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)) \
        .to(DEV).view(torch.bfloat16)


def bf16_dev(vals):
    bits = synth.bf16_bits_from_f32(vals)
    return synth.f32_from_bf16_bits(bits), up(None, bits, "bf16")


def host(t):
    return t.cpu().numpy()


@functools.lru_cache(maxsize=None)
def workload(w, name):
    vals, bits, dt = synth.workload_tensor(w, name)
    return vals, bits, dt


def check_quant(x_vals, q, g=None, rows=None):
    """Compare a device NVFP4 result with the oracle (optionally on sampled
    rows; then the global is checked against the oracle's full-tensor g)."""
    if g is None:
        g_ref = oracle.global_scale(x_vals)
    else:
        g_ref = np.float32(g)
    g_dev = np.float32(host(q.global_scale)[0])
    assert g_dev.view(np.uint32) == g_ref.view(np.uint32), (g_dev, g_ref)
    sel = slice(None) if rows is None else rows
    c_ref, s_ref, _ = oracle.quantize(x_vals[sel], g=g_ref)
    c_dev = host(q.codes)[sel]
    s_dev = host(q.scales)[sel]
    bad_s = np.nonzero(s_dev != s_ref)
    assert bad_s[0].size == 0, ("scales differ", bad_s[0][:5], bad_s[1][:5])
    bad_c = np.nonzero(c_dev != c_ref)
    assert bad_c[0].size == 0, ("codes differ", bad_c[0][:5], bad_c[1][:5],
                                c_dev[bad_c][:5], c_ref[bad_c][:5])


def sample_rows(n, count, seed):
    rng = np.random.default_rng(seed)
    r = set(rng.choice(n, size=min(count, n), replace=False).tolist())
    r |= {0, n - 1, min(255, n - 1), min(256, n - 1)}
    return np.array(sorted(r))


def rel_frob(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def check_bf16_within_one_ulp(y_dev_bf16, y_ref):
    ref16, _ = oracle.bf16_rne_from_f64(y_ref)
    got = host(y_dev_bf16.float()).astype(np.float64)
    mag = np.maximum(np.abs(ref16), np.abs(got))
    _, e = np.frexp(np.where(mag > 0, mag, 1.0))
    ulp = np.ldexp(1.0, np.maximum(e - 8, -133))
    assert np.all(np.abs(got - ref16) <= ulp)


# ------------------------------------------------------------- quantize

def test_quantize_tiny_fp32_compute():
    for name in ("x", "w"):
        vals, bits, dt = workload(1, name)
        _say("quantize tiny", name, vals.shape)
        q = nv.quantize(up(vals, bits, dt))
        check_quant(vals, q)


def test_quantize_worked_blocks_golden(golden):
    for line in golden("worked_blocks.txt"):
        head, xs, sc, packed = [p.strip() for p in line.split("|")]
        mode, g = head.split()
        x = np.array([np.float32(float(v)) for v in xs.split()],
                     dtype=np.float32)[None, :]
        gt = None if mode == "compute" else torch.tensor(
            [float(g)], dtype=torch.float32, device=DEV)
        for dt in ("f32", "bf16"):
            bits = synth.bf16_bits_from_f32(x)
            if dt == "bf16" and not np.array_equal(
                    synth.f32_from_bf16_bits(bits), x):
                continue
            q = nv.quantize(up(x, bits, dt), global_scale=gt)
            assert host(q.scales)[0, 0] == int(sc, 16), (line, dt)
            assert bytes(host(q.codes)[0]) == bytes(
                int(b, 16) for b in packed.split()), (line, dt)


def _adversarial(rng, rows, k):
    """Values on and next to every E2M1 midpoint times a block scale times
    the global, block maxima on E4M3 midpoints, zeros of both signs,
    sub-normal and huge magnitudes."""
    e4 = oracle.e4m3_decode_table()[:127]
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, 0.0])
    g = np.float32(2.0 ** rng.integers(-12, 6))
    x = np.zeros((rows, k), dtype=np.float32)
    for r in range(rows):
        for b in range(k // 16):
            j = rng.integers(1, 126)
            m = np.float32(6 * g * (e4[j] + e4[j + 1]) / 2)
            m = [m, np.nextafter(m, np.float32(0)),
                 np.nextafter(m, np.float32(np.inf)),
                 np.float32(6 * g * e4[j])][rng.integers(0, 4)]
            s = oracle.block_scales(np.array([m]), g)[0]
            d = np.float32(e4[s] * g)
            blk = d * mids[rng.integers(0, len(mids), 16)].astype(np.float32)
            nudge = rng.integers(-1, 2, 16)
            blk = np.where(nudge < 0, np.nextafter(blk, np.float32(0)),
                           np.where(nudge > 0,
                                    np.nextafter(blk, np.float32(np.inf)),
                                    blk)).astype(np.float32)
            blk *= np.where(rng.random(16) < 0.5, -1, 1).astype(np.float32)
            blk[rng.integers(0, 16)] = m
            if rng.random() < 0.05:
                blk[:] = 0
                blk[rng.integers(0, 16)] = -0.0
            x[r, b * 16:(b + 1) * 16] = blk
    return x, g


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_quantize_adversarial_ties_fp32(seed):
    rng = np.random.default_rng(100 + seed)
    x, g = _adversarial(rng, 64, 256)
    _say("quantize adversarial seed", seed, "g", g)
    xd = up(x, None, "f32")
    check_quant(x, nv.quantize(xd, global_scale=torch.tensor(
        [g], dtype=torch.float32, device=DEV)), g=g)
    check_quant(x, nv.quantize(xd))


def test_quantize_adversarial_bf16():
    rng = np.random.default_rng(7)
    x, g = _adversarial(rng, 64, 256)
    xb, xd = bf16_dev(x)
    check_quant(xb, nv.quantize(xd))
    check_quant(xb, nv.quantize(xd, global_scale=torch.tensor(
        [g], dtype=torch.float32, device=DEV)), g=g)


@pytest.mark.parametrize("g", [0.0, 1e-45, 1e-40, 3e-38, 1e-30, 1e-3, 1.0,
                               7.3e5, 1e30, 1e35])
def test_quantize_given_global_extremes(g):
    """Given globals across the binary32 range, including 0 and
    subnormals, on data of several magnitudes (saturating and underflowing
    blocks included)."""
    rng = np.random.default_rng(int(abs(np.log10(g + 1e-50)) * 10))
    x = (rng.standard_normal((16, 128)) *
         np.float32(10.0) ** rng.integers(-38, 37, (16, 1))).astype(
             np.float32)
    x[3, 5] = -0.0
    x[4, :16] = 0
    x[5, 16:32] = np.float32(1e-45)
    x[6, 32] = np.float32(3.3e38)
    gt = torch.tensor([g], dtype=torch.float32, device=DEV)
    _say("quantize given global", g)
    check_quant(x, nv.quantize(up(x, None, "f32"), global_scale=gt),
                g=np.float32(g))
    xb, xd = bf16_dev(x)
    check_quant(xb, nv.quantize(xd, global_scale=gt), g=np.float32(g))


def test_quantize_degenerate_tensors():
    zeros = np.zeros((3, 32), dtype=np.float32)
    q = nv.quantize(up(zeros, None, "f32"))
    check_quant(zeros, q)
    assert host(q.global_scale)[0] == 0
    negz = -zeros
    check_quant(negz, nv.quantize(up(negz, None, "f32")))
    tiny = np.full((2, 16), np.float32(1e-45), dtype=np.float32)
    check_quant(tiny, nv.quantize(up(tiny, None, "f32")))   # g underflows
    huge = np.full((2, 16), np.float32(3.3e38), dtype=np.float32)
    huge[1, 3] = -1.0
    check_quant(huge, nv.quantize(up(huge, None, "f32")))
    one = np.zeros((1, 16), dtype=np.float32)
    one[0, 7] = 5.0
    check_quant(one, nv.quantize(up(one, None, "f32")))


@pytest.mark.parametrize("rows,k,pad", [(1, 16, 0), (3, 48, 8), (257, 272, 0),
                                        (5, 5136, 24), (130, 4096, 64)])
def test_quantize_ragged_and_strided(rows, k, pad):
    rng = np.random.default_rng(rows * 7 + k)
    full = rng.standard_normal((rows, k + pad)).astype(np.float32)
    x = full[:, :k]
    _say("quantize ragged", rows, k, pad)
    xd = up(full, None, "f32")[:, :k]
    check_quant(x, nv.quantize(xd))
    fb, fd = bf16_dev(full)
    check_quant(fb[:, :k], nv.quantize(fd[:, :k]))


@pytest.mark.parametrize("w,name", [(2, "x"), (2, "w"), (5, "x"),
                                    (5, "x_dec"), (3, "w_a")])
def test_quantize_full_size(w, name):
    vals, bits, dt = workload(w, name)
    _say("quantize full size", w, name, vals.shape)
    xd = up(vals, bits, dt)
    rows = sample_rows(vals.shape[0], 192, w)
    check_quant(vals, nv.quantize(xd), rows=rows)
    g = np.float32(oracle.global_scale(vals) * np.float32(1.5))
    check_quant(vals, nv.quantize(xd, global_scale=torch.tensor(
        [g], dtype=torch.float32, device=DEV)), g=g, rows=rows)


# ------------------------------------------------------------ harmonize

def test_harmonize_every_scale_byte():
    allb = np.arange(0, 0x7F, dtype=np.uint8)
    sc = np.tile(allb, (6, 1)).reshape(6, 127)
    sc = np.concatenate([sc, np.zeros((6, 1), np.uint8)], axis=1)  # k=2048
    for ratios in ([0.5, 1.0, 0.75], [1 / 3, 0.5625, 1.0],
                   [1e-3, 1.0, 0.999], [0.0, 1.0, 0.3]):
        gs = [np.float32(r) for r in ratios]
        offs = [0, 2, 4, 6]
        ref, gstar = oracle.harmonize(sc, offs, gs)
        d = torch.from_numpy(sc.copy()).to(DEV)
        gd = torch.tensor(gs, dtype=torch.float32, device=DEV)
        out = nv.harmonize_group(d, 2048, offs, gd)
        assert host(out)[0] == gstar
        assert np.array_equal(host(d), ref), ratios


@pytest.mark.parametrize("scale", [1.0, 2.0 ** 110, 2.0 ** -110])
def test_harmonize_ragged_modules(scale):
    """Rows of 5 scale bytes (k = 80) and modules of 1-3 rows, so a lane's
    bytes straddle module boundaries and the array ends in a partial word; a
    module with global 0 and two with the shared maximum; shared globals
    beyond 2^100 or below 2^-100 (float64 path)."""
    rng = np.random.default_rng(41)
    rows_per = [1, 3, 1, 2, 1, 4, 2]
    offs = [0] + list(np.cumsum(rows_per))
    k = 80
    sc = rng.integers(0, 0x7F, (offs[-1], k // 16)).astype(np.uint8)
    gs = [np.float32(v * scale) for v in (0.3, 1.7, 0.0, 1.7, 1e-3, 0.999, 1.25)]
    ref, gstar = oracle.harmonize(sc, offs, gs)
    buf = torch.full((sc.size + 16,), 0xA5, dtype=torch.uint8, device=DEV)
    d = buf[:sc.size].view(sc.shape)
    d.copy_(torch.from_numpy(sc))
    _say("harmonize ragged", scale)
    out = nv.harmonize_group(d, k, offs, torch.tensor(gs, dtype=torch.float32, device=DEV))
    assert host(out)[0] == gstar
    assert np.array_equal(host(d), ref)
    assert np.all(host(buf[sc.size:]) == 0xA5)   # nothing past the array


def test_harmonize_rejects_unaligned_scales():
    """A scale array that is not 16-byte aligned is refused before any
    device work (no byte-wise path), and left untouched."""
    sc = np.arange(12 * 5, dtype=np.uint8).reshape(12, 5)
    buf = torch.zeros(sc.size + 16, dtype=torch.uint8, device=DEV)
    d = buf[8:8 + sc.size].view(sc.shape)
    d.copy_(torch.from_numpy(sc))
    gs = torch.tensor([0.5, 1.0], dtype=torch.float32, device=DEV)
    with pytest.raises(nv.NVFP4Error, match="MISALIGNED"):
        nv.harmonize_group(d, 80, [0, 8, 12], gs)
    assert np.array_equal(host(d), sc)


def test_harmonize_most_modules():
    """64 modules (the most the call takes) of one row of 5 scale bytes
    each, with distinct globals: a boundary falls inside almost every
    lane's 4 bytes."""
    rng = np.random.default_rng(43)
    n_mod, k = 64, 80
    offs = list(range(n_mod + 1))
    sc = rng.integers(0, 0x7F, (n_mod, k // 16)).astype(np.uint8)
    gs = [np.float32(v) for v in rng.uniform(0.01, 2.0, n_mod)]
    ref, gstar = oracle.harmonize(sc, offs, gs)
    d = torch.from_numpy(sc.copy()).to(DEV)
    out = nv.harmonize_group(d, k, offs, torch.tensor(gs, dtype=torch.float32, device=DEV))
    assert host(out)[0] == gstar
    assert np.array_equal(host(d), ref)


def test_harmonize_fused_group_full_size():
    """Three modules with different per-module globals quantised into row
    slices of one fused buffer, then harmonised (the fused qkv|z style
    group of the pages)."""
    mods = ["w1", "w2", "w3"]
    sizes = [synth.workload_shape(4, m)[0] for m in mods]
    k = 5120
    offs = [0] + list(np.cumsum(sizes))
    n_tot = offs[-1]
    codes = torch.empty((n_tot, k // 2), dtype=torch.uint8, device=DEV)
    scales = torch.empty((n_tot, k // 16), dtype=torch.uint8, device=DEV)
    gdev = torch.empty(3, dtype=torch.float32, device=DEV)
    ref_scales, ref_g = [], []
    for i, mname in enumerate(mods):
        vals, bits, dt = workload(4, mname)
        q = nv.quantize(up(vals, bits, dt), out=(codes[offs[i]:offs[i + 1]],
                                                 scales[offs[i]:offs[i + 1]]))
        gdev[i:i + 1].copy_(q.global_scale)
        rows = sample_rows(sizes[i], 64, i)
        check_quant(vals, q, rows=rows)
        ref_g.append(oracle.global_scale(vals))
        _, s_ref, _ = oracle.quantize(vals[rows], g=ref_g[-1])
        ref_scales.append((rows + offs[i], s_ref))
    gstar = nv.harmonize_group(scales, k, offs, gdev)
    all_rows = np.concatenate([r for r, _ in ref_scales])
    all_s = np.concatenate([s for _, s in ref_scales])
    # the oracle's harmonisation of the same sampled rows
    sub_offs = [0] + list(np.cumsum([len(r) for r, _ in ref_scales]))
    want, g_ref = oracle.harmonize(all_s, sub_offs, ref_g)
    assert host(gstar)[0] == g_ref
    assert np.array_equal(host(scales)[all_rows], want)
    assert len(set(float(g) for g in ref_g)) == 3


# ------------------------------------------------------------------ gemm

def _quant_pair(xv, xd, wv, wd):
    qa, qb = nv.quantize(xd), nv.quantize(wd)
    return qa, qb


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_gemm_tiny_exact(out_dtype):
    xv, xb, xt = workload(1, "x")
    wv, wb, wt = workload(1, "w")
    qa = nv.quantize(up(xv, xb, xt))
    qb = nv.quantize(up(wv, wb, wt))
    check_quant(xv, qa)
    check_quant(wv, qb)
    ref = oracle.gemm_exact_int(*oracle.quantize(xv), *oracle.quantize(wv))
    y = nv.gemm(qa, qb, out_dtype=out_dtype)
    if out_dtype == torch.float32:
        assert rel_frob(host(y).astype(np.float64), ref) <= TOL
    else:
        check_bf16_within_one_ulp(y, ref)


@pytest.mark.parametrize("m,n,k", [(1, 1, 16), (33, 65, 48), (300, 130, 272),
                                   (17, 300, 5136), (257, 513, 1024),
                                   (64, 64, 4096), (300, 20, 1024),
                                   (40, 1000, 512), (1000, 50, 256),
                                   (7, 777, 384), (513, 257, 640),
                                   (300, 200, 128), (130, 300, 256),
                                   (200, 129, 384), (33, 700, 640),
                                   (136, 264, 768), (130, 200, 1664)])
def test_gemm_ragged_shapes(m, n, k):
    rng = np.random.default_rng(m * 31 + n * 7 + k)
    xv = rng.standard_normal((m, k)).astype(np.float32)
    wv = (rng.standard_normal((n, k)) * 0.05).astype(np.float32)
    _say("gemm ragged", m, n, k)
    qa = nv.quantize(up(xv, None, "f32"))
    qb = nv.quantize(up(wv, None, "f32"))
    ref = oracle.gemm_exact_int(*oracle.quantize(xv), *oracle.quantize(wv))
    y = host(nv.gemm(qa, qb, out_dtype=torch.float32)).astype(np.float64)
    assert rel_frob(y, ref) <= TOL
    check_bf16_within_one_ulp(nv.gemm(qa, qb, out_dtype=torch.bfloat16), ref)
    ya = host(nv.gemm(qa, qb, out_dtype=torch.float32, epilogue="alpha"))
    assert rel_frob(ya.astype(np.float64), oracle.gate_alpha(ref)) <= TOL
    yb = host(nv.gemm(qa, qb, out_dtype=torch.float32, epilogue="beta"))
    assert rel_frob(yb.astype(np.float64), oracle.gate_beta(ref)) <= TOL


@pytest.mark.parametrize("m,n,k", [(32, 300, 512), (300, 40, 256),
                                   (200, 300, 384)])
def test_gemm_rejects_unaligned_scale_arrays(m, n, k):
    """Scale arrays at an odd byte offset are refused with MISALIGNED on
    the host (no kernel runs); the output buffer stays as it was."""
    rng = np.random.default_rng(m + 3 * n + k)
    xv = rng.standard_normal((m, k)).astype(np.float32)
    wv = (rng.standard_normal((n, k)) * 0.05).astype(np.float32)
    _say("gemm unaligned scales refused", m, n, k)
    qa = nv.quantize(up(xv, None, "f32"))
    qb = nv.quantize(up(wv, None, "f32"))

    def shifted(t):
        buf = torch.empty(t.numel() + 1, dtype=torch.uint8, device=DEV)
        v = buf[1:].view(t.shape)
        v.copy_(t)
        assert v.data_ptr() % 2 == 1
        return v
    y = torch.full((m, n), 5.0, dtype=torch.float32, device=DEV)
    for a, b in ((nv.NVFP4(qa.codes, shifted(qa.scales), qa.global_scale), qb),
                 (qa, nv.NVFP4(qb.codes, shifted(qb.scales), qb.global_scale))):
        with pytest.raises(nv.NVFP4Error, match="MISALIGNED"):
            nv.gemm(a, b, out_dtype=torch.float32, out=y)
    assert torch.all(y == 5.0)


# (m, n, k): one operand of at most 64 rows (L) and k a whole number of
# 512-K stages (L <= 32 rows) or 256-K stages (33..64 rows), so w4a4_gemm
# streams the other operand (S); S sized so that every S-rows-per-workgroup
# choice (16, 24, 32, 40, 64, 128: about one workgroup per CU) and every L
# padding (16, 32, 64) is taken, S = B (decode) and S = A (gate
# projections), each with a ragged last workgroup.
STREAM_SHAPES = [(7, 4109, 512),      # S rows per workgroup 24, L 16
                 (32, 5120, 1024),    # 24, L 32
                 (48, 6001, 512),     # 24, L 64, 512-K stages
                 (64, 2100, 256),     # 16, L 64, 256-K stages
                 (20, 8000, 512),     # 32, L 32
                 (3, 10007, 512),     # 40, L 16
                 (33, 12000, 256),    # 64, L 64, 256-K stages
                 (16, 20003, 512),    # 128, L 16
                 (6001, 48, 256),     # S = A: 24, L 64, 256-K stages
                 (12000, 40, 512),    # S = A: 64, L 64, 512-K stages
                 (20000, 64, 512),    # S = A: 128, L 64, 256-K stages
                 (20000, 32, 512),    # S = A: 128, L 32
                 (4100, 8, 1024),     # S = A: 24, L 16
                 (5, 40, 1024),       # both small: L = A (5 rows), one 40-row S slice
                 (64, 64, 512),       # both 64: L = A, 512-K stages for 64-row L
                 (1, 3, 512)]         # one output row, three columns


@pytest.mark.parametrize("m,n,k", STREAM_SHAPES)
def test_gemm_streaming_configurations(m, n, k):
    """Every output of the streaming GEMM's configurations against the
    exact product, fp32 and bf16, and the beta gate."""
    rng = np.random.default_rng(7 * m + 5 * n + k)
    xv = rng.standard_normal((m, k)).astype(np.float32)
    wv = (rng.standard_normal((n, k)) * 0.05).astype(np.float32)
    _say("gemm streaming", m, n, k)
    qa = nv.quantize(up(xv, None, "f32"))
    qb = nv.quantize(up(wv, None, "f32"))
    ref = oracle.gemm_f64(*oracle.quantize(xv), *oracle.quantize(wv))
    y = host(nv.gemm(qa, qb, out_dtype=torch.float32)).astype(np.float64)
    assert rel_frob(y, ref) <= TOL
    assert np.all(np.abs(y - ref) <= 1e-4 * np.max(np.abs(ref)))
    check_bf16_within_one_ulp(nv.gemm(qa, qb, out_dtype=torch.bfloat16), ref)
    yb = host(nv.gemm(qa, qb, out_dtype=torch.float32, epilogue="beta"))
    assert rel_frob(yb.astype(np.float64), oracle.gate_beta(ref)) <= TOL


@pytest.mark.parametrize("m,n,k", [(5 * 256 + 17, 8 * 256, 384),    # 6 x 8 tiles
                                   (11 * 256 + 1, 2 * 256, 256),    # 12 x 2 tiles
                                   (5 * 256 + 17, 8 * 256, 400),    # ragged k: staged
                                   (11 * 256 + 1, 2 * 256, 272)])
def test_gemm_xcd_tile_order_partial_group(m, n, k):
    """Tile counts divisible by 8 (the XCD-aware tile order) with a tile
    row count that leaves the last group of 8 M-tiles partial, for the
    pipelined kernel (k % 128 == 0) and the staged one (ragged k); every
    output compared."""
    rng = np.random.default_rng(m + n + k)
    xv = rng.standard_normal((m, k)).astype(np.float32)
    wv = (rng.standard_normal((n, k)) * 0.05).astype(np.float32)
    tiles_m, tiles_n = -(-m // 256), -(-n // 256)
    assert (tiles_m * tiles_n) % 8 == 0 and tiles_m % 8 != 0
    _say("gemm xcd tile order", m, n, k, tiles_m, tiles_n)
    qa = nv.quantize(up(xv, None, "f32"))
    qb = nv.quantize(up(wv, None, "f32"))
    ref = oracle.gemm_f64(*oracle.quantize(xv), *oracle.quantize(wv))
    y = host(nv.gemm(qa, qb, out_dtype=torch.float32)).astype(np.float64)
    assert rel_frob(y, ref) <= TOL
    # every element, not just the norm: a misplaced tile fails here
    assert np.all(np.abs(y - ref) <= 1e-4 * np.max(np.abs(ref)))
    check_bf16_within_one_ulp(nv.gemm(qa, qb, out_dtype=torch.bfloat16), ref)


def test_gemm_strided_output():
    rng = np.random.default_rng(3)
    xv = rng.standard_normal((40, 256)).astype(np.float32)
    wv = rng.standard_normal((24, 256)).astype(np.float32)
    qa = nv.quantize(up(xv, None, "f32"))
    qb = nv.quantize(up(wv, None, "f32"))
    big = torch.full((40, 64), 7.0, dtype=torch.float32, device=DEV)
    nv.gemm(qa, qb, out_dtype=torch.float32, out=big[:, 8:32])
    ref = oracle.gemm_exact_int(*oracle.quantize(xv), *oracle.quantize(wv))
    got = host(big)
    assert rel_frob(got[:, 8:32].astype(np.float64), ref) <= TOL
    assert np.all(got[:, :8] == 7.0) and np.all(got[:, 32:] == 7.0)


@pytest.mark.parametrize("m,n", [(512, 512), (600, 520)])
@pytest.mark.parametrize("col0,ld", [(8, 528), (2, 528), (8, 532)])
def test_gemm_bf16_tiles_into_wider_output(m, n, col0, ld):
    """bf16 output of the pipelined kernel (m, n > 64) written into a wider
    buffer: full tiles at a 16-byte aligned start with a row stride of whole
    16-byte pieces go through the LDS-staged store; a 4-byte aligned start
    or another stride, and partial tiles, take the per-element store.  The
    rest of the buffer stays untouched."""
    k = 256
    rng = np.random.default_rng(m + n + col0 + ld)
    xv = rng.standard_normal((m, k)).astype(np.float32)
    wv = (rng.standard_normal((n, k)) * 0.05).astype(np.float32)
    _say("gemm bf16 wide output", m, n, col0, ld)
    qa = nv.quantize(up(xv, None, "f32"))
    qb = nv.quantize(up(wv, None, "f32"))
    ref = oracle.gemm_exact_int(*oracle.quantize(xv), *oracle.quantize(wv))
    for epi, f in (("none", lambda r: r), ("alpha", oracle.gate_alpha),
                   ("beta", oracle.gate_beta)):
        big = torch.full((m, ld), 3.0, dtype=torch.bfloat16, device=DEV)
        view = big[:, col0:col0 + n]
        nv.gemm(qa, qb, out_dtype=torch.bfloat16, epilogue=epi, out=view)
        check_bf16_within_one_ulp(view, f(ref))
        got = host(big.float())
        assert np.all(got[:, :col0] == 3.0) and np.all(got[:, col0 + n:] == 3.0)


def _sampled_gemm_check(xv, qa, wv, qb, rows, cols, y_dev, out_dtype,
                        epilogue="none"):
    ca, sa, ga = oracle.quantize(xv[rows], g=oracle.global_scale(xv))
    cb, sb, gb = oracle.quantize(wv[cols], g=oracle.global_scale(wv))
    ref = oracle.gemm_f64(ca, sa, ga, cb, sb, gb)
    if epilogue == "alpha":
        ref = oracle.gate_alpha(ref)
    elif epilogue == "beta":
        ref = oracle.gate_beta(ref)
    got = y_dev[torch.from_numpy(rows).to(DEV)][:, torch.from_numpy(cols)
                                                 .to(DEV)]
    if out_dtype == torch.float32:
        err = rel_frob(host(got).astype(np.float64), ref)
        _say("sampled rel-Frob", err)
        assert err <= TOL
    else:
        check_bf16_within_one_ulp(got, ref)


def test_gemm_gdn_in_proj_full_size():
    xv, xb, xt = workload(2, "x")
    wv, wb, wt = workload(2, "w")
    _say("gemm in_proj 4096x12288x5120")
    qa = nv.quantize(up(xv, xb, xt))
    qb = nv.quantize(up(wv, wb, wt))
    rows = sample_rows(4096, 96, 21)
    cols = sample_rows(12288, 96, 22)
    for od in (torch.bfloat16, torch.float32):
        y = nv.gemm(qa, qb, out_dtype=od)
        _sampled_gemm_check(xv, qa, wv, qb, rows, cols, y, od)


def test_gemm_gate_projections_full_size():
    xv, xb, xt = workload(3, "x")
    _say("gemm gates 32768x64x5120")
    qa = nv.quantize(up(xv, xb, xt))
    rows = sample_rows(32768, 256, 31)
    cols = np.arange(64)
    for name, epi in (("w_a", "alpha"), ("w_b", "beta")):
        wv, wb, wt = workload(3, name)
        qb = nv.quantize(up(wv, wb, wt))
        y = nv.gemm(qa, qb, out_dtype=torch.float32, epilogue=epi)
        _sampled_gemm_check(xv, qa, wv, qb, rows, cols, y, torch.float32, epi)
        y = nv.gemm(qa, qb, out_dtype=torch.float32)
        _sampled_gemm_check(xv, qa, wv, qb, rows, cols, y, torch.float32)


def test_gemm_fused_group_after_harmonize():
    mods = ["w1", "w2", "w3"]
    sizes = [synth.workload_shape(4, m)[0] for m in mods]
    k = 5120
    offs = [0] + list(np.cumsum(sizes))
    codes = torch.empty((offs[-1], k // 2), dtype=torch.uint8, device=DEV)
    scales = torch.empty((offs[-1], k // 16), dtype=torch.uint8, device=DEV)
    gdev = torch.empty(3, dtype=torch.float32, device=DEV)
    wvals = []
    for i, mname in enumerate(mods):
        vals, bits, dt = workload(4, mname)
        wvals.append(vals)
        q = nv.quantize(up(vals, bits, dt), out=(codes[offs[i]:offs[i + 1]],
                                                 scales[offs[i]:offs[i + 1]]))
        gdev[i:i + 1].copy_(q.global_scale)
    gstar = nv.harmonize_group(scales, k, offs, gdev)
    xv, xb, xt = workload(4, "x")
    qa = nv.quantize(up(xv, xb, xt))
    y = nv.gemm(qa, nv.NVFP4(codes, scales, gstar), out_dtype=torch.float32)
    # oracle: quantise each module with its own global, harmonise, GEMM
    rows = sample_rows(8192, 64, 41)
    cols_per = [sample_rows(s, 40, 42 + i) for i, s in enumerate(sizes)]
    ca, sa, ga = oracle.quantize(xv[rows], g=oracle.global_scale(xv))
    gs = [oracle.global_scale(v) for v in wvals]
    parts = [oracle.quantize(v[c], g=g) for v, c, g in zip(wvals, cols_per,
                                                           gs)]
    bc = np.concatenate([p[0] for p in parts])
    bs = np.concatenate([p[1] for p in parts])
    sub_offs = [0] + list(np.cumsum([len(c) for c in cols_per]))
    bs_h, g_ref = oracle.harmonize(bs, sub_offs, gs)
    ref = oracle.gemm_f64(ca, sa, ga, bc, bs_h, g_ref)
    cols = np.concatenate([c + offs[i] for i, c in enumerate(cols_per)])
    got = host(y[torch.from_numpy(rows).to(DEV)][:, torch.from_numpy(cols)
                                                 .to(DEV)])
    assert rel_frob(got.astype(np.float64), ref) <= TOL


def test_gemm_prefill_and_decode_full_size():
    xv, xb, xt = workload(5, "x")
    dv, db, dt_ = workload(5, "x_dec")
    wv, wb, wt = workload(5, "w")
    _say("gemm prefill 32768x10240x5120 + decode 32")
    qb = nv.quantize(up(wv, wb, wt))
    qa = nv.quantize(up(xv, xb, xt))
    rows = sample_rows(32768, 64, 51)
    cols = sample_rows(10240, 64, 52)
    y = nv.gemm(qa, qb, out_dtype=torch.bfloat16)
    _sampled_gemm_check(xv, qa, wv, qb, rows, cols, y, torch.bfloat16)
    del y
    y = nv.gemm(qa, qb, out_dtype=torch.float32)
    _sampled_gemm_check(xv, qa, wv, qb, rows, cols, y, torch.float32)
    del y
    qd = nv.quantize(up(dv, db, dt_))
    check_quant(dv, qd)
    yd = nv.gemm(qd, qb, out_dtype=torch.float32)
    cols = sample_rows(10240, 512, 53)
    _sampled_gemm_check(dv, qd, wv, qb, np.arange(32), cols, yd,
                        torch.float32)
    ydb = nv.gemm(qd, qb, out_dtype=torch.bfloat16)
    _sampled_gemm_check(dv, qd, wv, qb, np.arange(32), cols, ydb,
                        torch.bfloat16)


def test_gemm_repeated_launches_bit_identical():
    """Every wave of a pipelined-GEMM workgroup fills rows that the others
    read, so a missing wait or barrier shows as run-to-run differences:
    back-to-back launches (full-size prefill, and a small-K shape whose
    tiles are mostly prologue and epilogue) must give identical bits."""
    xv, xb, xt = workload(5, "x")
    wv, wb, wt = workload(5, "w")
    qa = nv.quantize(up(xv, xb, xt))
    qb = nv.quantize(up(wv, wb, wt))
    for od, reps in ((torch.bfloat16, 12), (torch.float32, 4)):
        _say("gemm repeat prefill", od, reps)
        ref = nv.gemm(qa, qb, out_dtype=od)
        out = torch.empty_like(ref)
        ibits = torch.int16 if od == torch.bfloat16 else torch.int32
        for i in range(reps):
            nv.gemm(qa, qb, out_dtype=od, out=out)
            assert torch.equal(out.view(ibits), ref.view(ibits)), i
        del ref, out
    rng = np.random.default_rng(12)
    m, n, k = 4160, 4224, 640
    qa = nv.quantize(up(rng.standard_normal((m, k)).astype(np.float32), None, "f32"))
    qb = nv.quantize(up(rng.standard_normal((n, k)).astype(np.float32), None, "f32"))
    _say("gemm repeat", m, n, k)
    ref = nv.gemm(qa, qb, out_dtype=torch.bfloat16)
    out = torch.empty_like(ref)
    for i in range(50):
        nv.gemm(qa, qb, out_dtype=torch.bfloat16, out=out)
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), i


def test_calls_on_a_side_stream():
    rng = np.random.default_rng(8)
    xv = rng.standard_normal((64, 512)).astype(np.float32)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        xd = up(xv, None, "f32")
        q = nv.quantize(xd)
        y = nv.gemm(q, q, out_dtype=torch.float32)
    s.synchronize()
    check_quant(xv, q)
    ref = oracle.gemm_exact_int(*oracle.quantize(xv), *oracle.quantize(xv))
    assert rel_frob(host(y).astype(np.float64), ref) <= TOL


# ----------------------------------------- gate pair of a fused b|a projection

def _gate_params(n_alpha, seed):
    rng = np.random.default_rng(seed)
    a_log = rng.uniform(-2.0, 1.5, n_alpha).astype(np.float32)
    dt = rng.uniform(-3.0, 3.0, n_alpha).astype(np.float32)
    return a_log, dt, torch.from_numpy(a_log).to(DEV), torch.from_numpy(dt).to(DEV)


# k % 256 == 0 (% 512 for n <= 32) with n = n_beta + n_alpha <= 64 takes the
# streaming GEMM (S = the tokens; L of 16, 32 or 64 rows), other shapes the
# skinny kernel
@pytest.mark.parametrize("m,n_beta,n_alpha,k", [(1, 16, 16, 128), (37, 64, 64, 5120),
                                                (300, 32, 48, 384), (513, 100, 120, 256),
                                                (64, 0, 20, 128), (40, 24, 0, 256),
                                                (70, 128, 128, 640),
                                                (1000, 64, 64, 512), (20000, 64, 64, 256),
                                                (33, 0, 40, 512), (5000, 20, 12, 1024),
                                                (3000, 60, 4, 256), (4100, 7, 9, 512),
                                                (1, 8, 8, 512), (2, 0, 64, 1024)])
def test_gdn_gates(m, n_beta, n_alpha, k):
    rng = np.random.default_rng(m + n_beta + 3 * n_alpha + k)
    xv = rng.standard_normal((m, k)).astype(np.float32)
    wv = (rng.standard_normal((n_beta + n_alpha, k)) * 0.05).astype(np.float32)
    _say("gdn gates", m, n_beta, n_alpha, k)
    a_log, dt, a_dev, dt_dev = _gate_params(n_alpha, k)
    qa = nv.quantize(up(xv, None, "f32"))
    qb = nv.quantize(up(wv, None, "f32"))
    y = oracle.gemm_exact_int(*oracle.quantize(xv), *oracle.quantize(wv))
    beta_ref, alpha_ref = oracle.gdn_gates(y, n_beta, a_log, dt)
    beta, alpha = nv.gdn_gates(qa, qb, n_beta, a_dev, dt_dev)
    if n_beta:
        assert rel_frob(host(beta).astype(np.float64), beta_ref) <= TOL
    if n_alpha:
        assert rel_frob(host(alpha).astype(np.float64), alpha_ref) <= TOL
    # element by element, within what fp32 accumulation and evaluation allow
    from test_gpu_fullsize import abs_product, check_gate
    oq = (oracle.quantize(xv), oracle.quantize(wv))
    sabs = abs_product(*oq)
    if n_beta:
        check_gate(host(beta), "beta", y[:, :n_beta], sabs[:, :n_beta], k)
    if n_alpha:
        check_gate(host(alpha), "gdn_alpha", y[:, n_beta:], sabs[:, n_beta:], k, a_log, dt)


def test_gdn_gates_harmonized_group_full_size():
    """32768 tokens x hidden 5120 through the b|a group (64 + 64 heads), the
    two weights quantised with their own globals and harmonised into one
    fused buffer; sampled rows against the oracle."""
    k, nb, na = 5120, 64, 64
    xv, xb, xt = workload(3, "x")
    wav, wab, wat = workload(3, "w_a")
    wbv, wbb, wbt = workload(3, "w_b")
    _say("gdn gates full size 32768x128x5120")
    codes = torch.empty((nb + na, k // 2), dtype=torch.uint8, device=DEV)
    scales = torch.empty((nb + na, k // 16), dtype=torch.uint8, device=DEV)
    gdev = torch.empty(2, dtype=torch.float32, device=DEV)
    for i, (v, b, t, lo, hi) in enumerate(((wbv, wbb, wbt, 0, nb), (wav, wab, wat, nb, nb + na))):
        q = nv.quantize(up(v, b, t), out=(codes[lo:hi], scales[lo:hi]))
        gdev[i:i + 1].copy_(q.global_scale)
    gstar = nv.harmonize_group(scales, k, [0, nb, nb + na], gdev)
    qa = nv.quantize(up(xv, xb, xt))
    a_log, dt, a_dev, dt_dev = _gate_params(na, 77)
    beta, alpha = nv.gdn_gates(qa, nv.NVFP4(codes, scales, gstar), nb, a_dev, dt_dev)
    rows = sample_rows(32768, 128, 43)
    ca, sa, ga = oracle.quantize(xv[rows], g=oracle.global_scale(xv))
    gs = [oracle.global_scale(wbv), oracle.global_scale(wav)]
    pb, pa = oracle.quantize(wbv, g=gs[0]), oracle.quantize(wav, g=gs[1])
    bs_h, g_ref = oracle.harmonize(np.concatenate([pb[1], pa[1]]), [0, nb, nb + na], gs)
    y = oracle.gemm_f64(ca, sa, ga, np.concatenate([pb[0], pa[0]]), bs_h, g_ref)
    beta_ref, alpha_ref = oracle.gdn_gates(y, nb, a_log, dt)
    sel = torch.from_numpy(rows).to(DEV)
    assert rel_frob(host(beta[sel]).astype(np.float64), beta_ref) <= TOL
    assert rel_frob(host(alpha[sel]).astype(np.float64), alpha_ref) <= TOL


# ------------------------------------------------------ degenerate and limits

def test_gemm_zero_operand_and_zero_global():
    """An all-zero activation tensor quantises to g = 0 and zero scales; the
    product is exactly +0 everywhere (pipelined and skinny shapes)."""
    rng = np.random.default_rng(6)
    for m, n, k in ((300, 200, 256), (16, 500, 512)):
        xz = np.zeros((m, k), dtype=np.float32)
        wv = rng.standard_normal((n, k)).astype(np.float32)
        qa, qb = nv.quantize(up(xz, None, "f32")), nv.quantize(up(wv, None, "f32"))
        assert host(qa.global_scale)[0] == 0.0
        y = host(nv.gemm(qa, qb, out_dtype=torch.float32))
        assert np.all(y == 0.0)


@pytest.mark.parametrize("k", [1 << 22, (1 << 22) + 256])
def test_gemm_longest_k_sparse_blocks(k):
    """k at and past the largest K of the pipelined kernel's 32-bit tile
    offsets (2^22; beyond it the staged kernel runs).  Random codes, block
    scales zero except in a few blocks spread over K (first, middle, last),
    so the exact reference only needs those blocks."""
    m = n = 65
    rng = np.random.default_rng(k)
    _say("gemm longest k", k)
    ac = rng.integers(0, 256, (m, k // 2), dtype=np.uint8)
    bc = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    kb = k // 16
    live = np.array(sorted({0, 1, 7, kb // 2, kb // 2 + 1, (1 << 18) - 1,
                            min(1 << 18, kb - 1), kb - 2, kb - 1}))
    as_ = np.zeros((m, kb), dtype=np.uint8)
    bs = np.zeros((n, kb), dtype=np.uint8)
    as_[:, live] = rng.integers(1, 0x7F, (m, live.size))
    bs[:, live] = rng.integers(1, 0x7F, (n, live.size))
    ga, gb = np.float32(0.01), np.float32(0.003)

    def dev(c, s, g):
        return nv.NVFP4(torch.from_numpy(c).to(DEV), torch.from_numpy(s).to(DEV),
                        torch.tensor([g], dtype=torch.float32, device=DEV))
    y = host(nv.gemm(dev(ac, as_, ga), dev(bc, bs, gb), out_dtype=torch.float32))
    cols = (live[:, None] * 8 + np.arange(8)[None, :]).ravel()     # code bytes of live blocks
    ref = oracle.gemm_f64(ac[:, cols], as_[:, live], ga, bc[:, cols], bs[:, live], gb)
    assert rel_frob(y.astype(np.float64), ref) <= TOL
