"""Seeded random sweeps through the C ABI, against the oracle.

GEMM: shapes that fall on every kernel the library picks (skinny tiles for
m or n up to 64 with either K-group size, the pipelined kernel, the staged
kernel for ragged k), with ragged edges, both output types, the gate
epilogues and strided outputs; scale arrays at an odd address are refused
(MISALIGNED) before any launch.  Bars as in
test_gpu_parity: fp32 output within relative Frobenius error 1e-5 of the
exact product (gated: of the gate of it); bf16 output within one bf16 ulp
of the exact value rounded to bf16; output columns past n untouched.

Quantise -> dequantise -> error statistics: random shapes, row strides,
input types, global modes and value mixes (normal with outlier channels,
log-uniform magnitudes over 1e-20..1e20, sparse, values near E2M1
midpoints).  Codes, scales, globals and dequantised values bit-exact; the
statistics' maxima exact and sums within 1e-12 relative.

FP8 KV cache: calibration over several strided slabs and the cast into a
strided output, amax, scale and every code bit-exact.  GDN gate pair:
random token counts, head counts and per-head parameters, gates within
1e-5 relative Frobenius error of the oracle's gates of the exact product.
Fused small-M quantise + GEMM: random m <= 64, n, k, input types and
global modes, bit-identical to the two separate calls.
"""
import numpy as np
import pytest
import torch

import nvfp4_w4a4_quantized_03_amd as nv
import oracle
import synth
from test_gpu_parity import DEV, TOL, check_bf16_within_one_ulp, host, rel_frob, up

pytestmark = pytest.mark.gpu

GATES = {"none": lambda y: y, "alpha": oracle.gate_alpha, "beta": oracle.gate_beta}


def _say(*a):
    print("[gpu-sweep]", *a, flush=True)


def _dim(rng):
    """Small (skinny kernel), just past 64, or a few tiles with a ragged edge."""
    kind = rng.integers(0, 3)
    if kind == 0:
        return int(rng.integers(1, 65))
    if kind == 1:
        return int(rng.integers(65, 130))
    return int(rng.integers(130, 560))


def _cases(count, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        m, n = _dim(rng), _dim(rng)
        if rng.random() < 0.7:
            k = 128 * int(rng.integers(1, 12))          # whole stages (skinny / pipelined)
        else:
            k = 16 * int(rng.integers(1, 90))           # ragged k (staged)
        cases.append(dict(
            m=m, n=n, k=k,
            out=("f32", "bf16")[int(rng.integers(0, 2))],
            epi=("none", "alpha", "beta")[int(rng.integers(0, 3))],
            pad=int(rng.choice([0, 0, 8, 24])),
            odd_scales=bool(rng.random() < 0.15),
            seed=int(rng.integers(0, 2**31)),
        ))
    return cases


def _shifted(t):
    """The same bytes at an odd address (the ABI requires 16-byte aligned
    scale arrays and refuses others)."""
    buf = torch.empty(t.numel() + 1, dtype=torch.uint8, device=DEV)
    v = buf[1:].view(t.shape)
    v.copy_(t)
    return v


@pytest.mark.parametrize("case", _cases(56, 20261208), ids=lambda c: "%(m)dx%(n)dx%(k)d-%(out)s-%(epi)s" % c)
def test_gemm_random_shape(case):
    m, n, k = case["m"], case["n"], case["k"]
    _say(case)
    rng = np.random.default_rng(case["seed"])
    xv = rng.standard_normal((m, k)).astype(np.float32)
    xv[:, rng.integers(0, k, 2)] *= np.float32(30.0)
    wv = (rng.standard_normal((n, k)) * 0.05).astype(np.float32)
    qa = nv.quantize(up(xv, None, "f32"))
    qb = nv.quantize(up(wv, None, "f32"))
    od = torch.float32 if case["out"] == "f32" else torch.bfloat16
    if case["odd_scales"]:
        odd = nv.NVFP4(qa.codes, _shifted(qa.scales), qa.global_scale)
        with pytest.raises(nv.NVFP4Error, match="MISALIGNED"):
            nv.gemm(odd, qb, out_dtype=od)
    pad = case["pad"]
    big = torch.full((m, n + pad), -3.0, dtype=od, device=DEV)
    y = big[:, :n]
    nv.gemm(qa, qb, out_dtype=od, epilogue=case["epi"], out=y)
    ref = GATES[case["epi"]](oracle.gemm_exact_int(*oracle.quantize(xv), *oracle.quantize(wv)))
    if od == torch.float32:
        assert rel_frob(host(y).astype(np.float64), ref) <= TOL
    else:
        check_bf16_within_one_ulp(y, ref)
    if pad:
        assert torch.all(big[:, n:] == -3.0)


# ------------------------------------------------- quantise / dequantise

def _values(rng, rows, k, kind):
    """Seeded inputs of several magnitude mixes."""
    if kind == "normal":
        x = rng.standard_normal((rows, k))
        x[:, rng.integers(0, k, max(1, k // 100))] *= 60.0        # outlier channels
    elif kind == "loguniform":
        x = np.exp(rng.uniform(np.log(1e-20), np.log(1e20), (rows, k)))
        x *= rng.choice([-1.0, 1.0], (rows, k))
    elif kind == "sparse":
        x = rng.standard_normal((rows, k)) * (rng.random((rows, k)) < 0.1)
    else:                                                           # "grid": near E2M1 midpoints
        mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
        x = rng.choice(mids, (rows, k)) * np.exp2(rng.integers(-3, 4, (rows, 1)))
        x *= 1.0 + rng.choice([0.0, 2.0 ** -20, -(2.0 ** -20)], (rows, k))
    return x.astype(np.float32)


def _qcases(count, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        out.append(dict(rows=int(rng.integers(1, 300)), k=16 * int(rng.integers(1, 200)),
                        pad=int(rng.choice([0, 0, 8, 40])),
                        dtype=("f32", "bf16")[int(rng.integers(0, 2))],
                        mode=("compute", "given")[int(rng.integers(0, 2))],
                        kind=("normal", "loguniform", "sparse", "grid")[int(rng.integers(0, 4))],
                        seed=int(rng.integers(0, 2**31))))
    return out


@pytest.mark.parametrize("case", _qcases(40, 20261209),
                         ids=lambda c: "%(rows)dx%(k)d+%(pad)d-%(dtype)s-%(mode)s-%(kind)s" % c)
def test_quantize_dequantize_random(case):
    """Quantise (codes, scales and global bit-exact with the oracle),
    then dequantise (each output one rounding of the exact value) and the
    error statistics of the same tensors, on a strided input."""
    _say(case)
    rng = np.random.default_rng(case["seed"])
    rows, k, pad = case["rows"], case["k"], case["pad"]
    full = _values(rng, rows, k + pad, case["kind"])
    if case["dtype"] == "bf16":
        bits = synth.bf16_bits_from_f32(full)
        full = synth.f32_from_bf16_bits(bits)
        fd = torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    else:
        fd = up(full, None, "f32")
    x, xd = full[:, :k], fd[:, :k]
    g_ref = oracle.global_scale(x)
    gt = None
    if case["mode"] == "given":
        g_ref = np.float32(g_ref * np.float32(rng.uniform(0.5, 2.0)))
        gt = torch.tensor([g_ref], dtype=torch.float32, device=DEV)
    q = nv.quantize(xd, global_scale=gt)
    c_ref, s_ref, _ = oracle.quantize(x, g=g_ref)
    assert np.float32(host(q.global_scale)[0]).view(np.uint32) == np.float32(g_ref).view(np.uint32)
    assert np.array_equal(host(q.scales), s_ref)
    assert np.array_equal(host(q.codes), c_ref)
    f32 = host(nv.dequantize(q, torch.float32))
    assert np.array_equal(f32.view(np.uint32), oracle.dequantize_f32(c_ref, s_ref, g_ref).view(np.uint32))
    b16 = host(nv.dequantize(q, torch.bfloat16).view(torch.int16)).view(np.uint16)
    assert np.array_equal(b16, oracle.dequantize_bf16(c_ref, s_ref, g_ref))
    st = host(nv.error_stats(xd, q))
    ref = oracle.error_stats(x, c_ref, s_ref, g_ref)
    assert np.array_equal(st[:, 2], ref[:, 2])
    for col in (0, 1):
        assert np.all(np.abs(st[:, col] - ref[:, col]) <= 1e-12 * np.abs(ref[:, col]) + 1e-300)


# ------------------------------------------------------------- FP8 KV cache

def _kvcases(count, seed):
    rng = np.random.default_rng(seed)
    return [dict(rows=int(rng.integers(1, 300)), k=16 * int(rng.integers(1, 160)),
                 pad=int(rng.choice([0, 0, 16, 48])), opad=int(rng.choice([0, 16])),
                 dtype=("f32", "bf16")[int(rng.integers(0, 2))],
                 kind=("normal", "loguniform", "sparse")[int(rng.integers(0, 3))],
                 parts=int(rng.integers(1, 4)), seed=int(rng.integers(0, 2**31)))
            for _ in range(count)]


@pytest.mark.parametrize("case", _kvcases(24, 20261210),
                         ids=lambda c: "%(rows)dx%(k)d+%(pad)d-%(dtype)s-%(kind)s-%(parts)d" % c)
def test_fp8_kv_random(case):
    """Calibration over 1-3 strided slabs (running amax and scale
    bit-exact), then the cast of a fresh strided slab into a strided
    output (every code bit-exact, padding untouched)."""
    _say(case)
    rng = np.random.default_rng(case["seed"])
    rows, k, pad, opad = case["rows"], case["k"], case["pad"], case["opad"]

    def slab():
        full = _values(rng, rows, k + pad, case["kind"])
        if case["dtype"] == "bf16":
            bits = synth.bf16_bits_from_f32(full)
            full = synth.f32_from_bf16_bits(bits)
            fd = torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
        else:
            fd = up(full, None, "f32")
        return full[:, :k], fd[:, :k]
    parts = [slab() for _ in range(case["parts"])]
    scale, amax = nv.fp8_kv_calibrate([d for _, d in parts])
    a_ref = oracle.kv_amax([v for v, _ in parts])
    s_ref = oracle.kv_scale(a_ref)
    assert np.float32(host(amax)[0]).view(np.uint32) == a_ref.view(np.uint32)
    assert np.float32(host(scale)[0]).view(np.uint32) == s_ref.view(np.uint32)
    xv, xd = slab()
    big = torch.full((rows, k + opad), 0xA5, dtype=torch.uint8, device=DEV)
    nv.fp8_kv_cast(xd, scale, out=big[:, :k])
    got = host(big)
    assert np.array_equal(got[:, :k], oracle.kv_cast(xv, s_ref))
    assert np.all(got[:, k:] == 0xA5)


# ----------------------------------------------------------- GDN gate pair

def _gcases(count, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        nb = int(rng.choice([0, int(rng.integers(1, 129))]))
        na = int(rng.integers(1 if nb == 0 else 0, 129))
        out.append(dict(m=int(rng.integers(1, 600)), nb=nb, na=na,
                        k=128 * int(rng.integers(1, 24)), seed=int(rng.integers(0, 2**31))))
    return out


@pytest.mark.parametrize("case", _gcases(16, 20261211),
                         ids=lambda c: "%(m)dx(%(nb)d+%(na)d)x%(k)d" % c)
def test_gdn_gates_random(case):
    """The gate pair of a fused b|a projection on random shapes and
    per-head parameters, against the oracle's gates of the exact product."""
    _say(case)
    rng = np.random.default_rng(case["seed"])
    m, nb, na, k = case["m"], case["nb"], case["na"], case["k"]
    xv = rng.standard_normal((m, k)).astype(np.float32)
    wv = (rng.standard_normal((nb + na, k)) * 0.05).astype(np.float32)
    a_log = rng.uniform(-2.0, 1.5, na).astype(np.float32)
    dt = rng.uniform(-3.0, 3.0, na).astype(np.float32)
    qa = nv.quantize(up(xv, None, "f32"))
    qb = nv.quantize(up(wv, None, "f32"))
    y = oracle.gemm_exact_int(*oracle.quantize(xv), *oracle.quantize(wv))
    beta_ref, alpha_ref = oracle.gdn_gates(y, nb, a_log, dt)
    beta, alpha = nv.gdn_gates(qa, qb, nb, torch.from_numpy(a_log).to(DEV),
                               torch.from_numpy(dt).to(DEV))
    if nb:
        assert rel_frob(host(beta).astype(np.float64), beta_ref) <= TOL
    if na:
        assert rel_frob(host(alpha).astype(np.float64), alpha_ref) <= TOL


# ------------------------------------------ fused small-M quantise + GEMM

def _fcases(count, seed):
    rng = np.random.default_rng(seed)
    return [dict(m=int(rng.integers(1, 65)), n=int(rng.integers(1, 3000)),
                 k=128 * int(rng.integers(1, 20)),
                 dtype=("f32", "bf16")[int(rng.integers(0, 2))],
                 mode=("compute", "given")[int(rng.integers(0, 2))],
                 out=("f32", "bf16")[int(rng.integers(0, 2))],
                 seed=int(rng.integers(0, 2**31)))
            for _ in range(count)]


@pytest.mark.parametrize("case", _fcases(16, 20261212),
                         ids=lambda c: "%(m)dx%(n)dx%(k)d-%(dtype)s-%(mode)s-%(out)s" % c)
def test_fused_quantize_gemm_random(case):
    """One-launch quantise + GEMM on random small-M shapes: X's NVFP4 form
    and Y bit-identical to the two separate calls, Y against the exact
    product of the oracle's quantisation."""
    _say(case)
    rng = np.random.default_rng(case["seed"])
    m, n, k = case["m"], case["n"], case["k"]
    xv = rng.standard_normal((m, k)).astype(np.float32)
    xv[:, rng.integers(0, k, 2)] *= np.float32(40.0)
    wv = (rng.standard_normal((n, k)) * 0.05).astype(np.float32)
    if case["dtype"] == "bf16":
        bits = synth.bf16_bits_from_f32(xv)
        xv = synth.f32_from_bf16_bits(bits)
        xd = torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    else:
        xd = up(xv, None, "f32")
    qw = nv.quantize(up(wv, None, "f32"))
    g_ref = oracle.global_scale(xv)
    gt = None
    if case["mode"] == "given":
        g_ref = np.float32(g_ref * np.float32(1.5))
        gt = torch.tensor([g_ref], dtype=torch.float32, device=DEV)
    od = torch.float32 if case["out"] == "f32" else torch.bfloat16
    qx, y = nv.gemm_quantize_a(xd, qw, global_scale=gt, out_dtype=od)
    qs = nv.quantize(xd, global_scale=gt)
    for a, b in ((qx.codes, qs.codes), (qx.scales, qs.scales), (qx.global_scale, qs.global_scale)):
        assert torch.equal(a, b)
    ys = nv.gemm(qs, qw, out_dtype=od)
    ib = torch.int16 if od == torch.bfloat16 else torch.int32
    assert torch.equal(y.view(ib), ys.view(ib)), "fused Y differs from quantize + gemm"
    ref = oracle.gemm_exact_int(*oracle.quantize(xv, g=g_ref), *oracle.quantize(wv))
    if od == torch.float32:
        assert rel_frob(host(y).astype(np.float64), ref) <= TOL
    else:
        check_bf16_within_one_ulp(y, ref)
