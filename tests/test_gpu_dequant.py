"""Parity of nvfp4_dequantize and nvfp4_error_stats (through the C ABI)
with the CPU oracle.

Bars: dequantised binary32 and bfloat16 outputs bit-exact (both sides round
the exact value once); error statistics: max |x| exact, the float64 sums
within 1e-12 relative (summation order differs).  Small cases element by
element, the full-size activation tensor on sampled rows.
"""
import numpy as np
import pytest
import torch

import nvfp4_w4a4_quantized_03_amd as nv
import oracle
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(*a):
    print("[gpu-dequant]", *a, flush=True)


def host(t):
    return t.cpu().numpy()


def _random_nvfp4(rows, k, g, seed):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(rows, k // 2)).astype(np.uint8)
    scales = rng.integers(0, 0x7F, size=(rows, k // 16)).astype(np.uint8)
    g = np.float32(g)
    dev = nv.NVFP4(torch.from_numpy(codes).to(DEV),
                   torch.from_numpy(scales).to(DEV),
                   torch.tensor([g], dtype=torch.float32, device=DEV))
    return codes, scales, g, dev


@pytest.mark.parametrize("rows,k", [(1, 16), (7, 48), (300, 272), (33, 5136)])
@pytest.mark.parametrize("g", [0.0173, 2.0 ** -140, 3.0e-41, 1.25e30, 0.0])
def test_dequantize_bit_exact(rows, k, g):
    _say("dequantize", rows, k, g)
    codes, scales, g, q = _random_nvfp4(rows, k, g, rows * 7 + k)
    f32 = host(nv.dequantize(q, torch.float32))
    ref = oracle.dequantize_f32(codes, scales, g)
    assert np.array_equal(f32.view(np.uint32), ref.view(np.uint32))
    b16 = host(nv.dequantize(q, torch.bfloat16).view(torch.int16)).view(np.uint16)
    assert np.array_equal(b16, oracle.dequantize_bf16(codes, scales, g))


def test_dequantize_strided_output():
    codes, scales, g, q = _random_nvfp4(40, 256, 0.5, 3)
    big = torch.full((40, 320), 7.0, dtype=torch.float32, device=DEV)
    nv.dequantize(q, torch.float32, out=big[:, 32:288])
    got = host(big)
    assert np.array_equal(got[:, 32:288].view(np.uint32),
                          oracle.dequantize_f32(codes, scales, g).view(np.uint32))
    assert np.all(got[:, :32] == 7.0) and np.all(got[:, 288:] == 7.0)


def test_dequantize_strided_bf16_output():
    codes, scales, g, q = _random_nvfp4(40, 256, 0.0625, 4)
    big = torch.zeros((40, 320), dtype=torch.bfloat16, device=DEV)
    nv.dequantize(q, torch.bfloat16, out=big[:, 48:304])
    got = host(big.view(torch.int16)).view(np.uint16)
    assert np.array_equal(got[:, 48:304], oracle.dequantize_bf16(codes, scales, g))
    assert not got[:, :48].any() and not got[:, 304:].any()


def _bf16_midpoint_cases(count, seed):
    """(code nibble, scale byte, g) with fp32(e2m1 * e4m3 * g) exactly on a
    bfloat16 midpoint while the exact product is not: the only products for
    which rounding the binary32 value again to bfloat16 gives another
    result than one rounding of the exact value."""
    rng = np.random.default_rng(seed)
    e2m1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    e4m3 = oracle.e4m3_decode_table()
    cases = []
    while len(cases) < count:
        code, sbyte = int(rng.integers(1, 8)), int(rng.integers(1, 127))
        v = e2m1[code] * float(e4m3[sbyte])
        target = np.array([(int(rng.integers(0x2000, 0x5000)) << 16) | 0x8000],
                          dtype=np.uint32).view(np.float32)[0]
        g = np.float32(float(target) / v)
        if not np.isfinite(g) or g <= 0:
            continue
        exact = v * float(g)                    # exact in float64
        f = np.float32(exact)
        if (int(f.view(np.uint32)) & 0xFFFF) == 0x8000 and float(f) != exact:
            cases.append((code, sbyte, g))
    return cases


def test_dequantize_bf16_at_binary32_midpoints():
    """Products whose binary32 rounding lands on a bfloat16 midpoint: the
    device must round the exact product, not the binary32 value."""
    naive_wrong = 0
    for i, (code, sbyte, g) in enumerate(_bf16_midpoint_cases(48, 11)):
        codes = np.zeros((1, 16), dtype=np.uint8)
        codes[0, :8] = code | (code << 4)                  # block 0: +v
        codes[0, 8:] = (code | 8) | ((code | 8) << 4)      # block 1: -v
        scales = np.array([[sbyte, sbyte]], dtype=np.uint8)
        q = nv.NVFP4(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV),
                     torch.tensor([g], dtype=torch.float32, device=DEV))
        want = oracle.dequantize_bf16(codes, scales, g)
        got = host(nv.dequantize(q, torch.bfloat16).view(torch.int16)).view(np.uint16)
        assert np.array_equal(got, want), (i, code, sbyte, float(g))
        twice = oracle.bf16_rne_from_f64(
            oracle.dequantize(codes, scales, g).astype(np.float32).astype(np.float64))[1]
        naive_wrong += int(np.any(twice != want))
    assert naive_wrong > 0   # the cases do separate the two roundings


def test_fake_quantize_round_trip():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((64, 512)) * 2).astype(np.float32)
    y = host(nv.fake_quantize(torch.from_numpy(x).to(DEV)))
    ref = oracle.dequantize_f32(*oracle.quantize(x))
    assert np.array_equal(y.view(np.uint32), ref.view(np.uint32))


def _check_stats(got, ref):
    assert np.array_equal(got[:, 2], ref[:, 2])
    for c in (0, 1):
        assert np.all(np.abs(got[:, c] - ref[:, c]) <= 1e-12 * np.abs(ref[:, c]) + 1e-300)


@pytest.mark.parametrize("rows,k,dtype", [(1, 16, "f32"), (37, 80, "bf16"),
                                          (300, 1040, "f32"), (5, 5120, "bf16")])
def test_error_stats_small(rows, k, dtype):
    _say("error_stats", rows, k, dtype)
    rng = np.random.default_rng(rows + k)
    x = (rng.standard_normal((rows, k)) * 1.5).astype(np.float32)
    if dtype == "bf16":
        bits = synth.bf16_bits_from_f32(x)
        x = synth.f32_from_bf16_bits(bits)
        xd = torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    else:
        xd = torch.from_numpy(x).to(DEV)
    q = nv.quantize(xd)
    g = np.float32(host(q.global_scale)[0])
    got = host(nv.error_stats(xd, q))
    c, s, _ = oracle.quantize(x, g=g)
    _check_stats(got, oracle.error_stats(x, c, s, g))


def test_error_stats_and_dequantize_full_size():
    """32768 x 5120 bf16 activations (the long-prefill workload) in the
    benchmark's configuration; sampled rows against the oracle."""
    vals, bits, _ = synth.workload_tensor(5, "x")
    _say("full size 32768x5120")
    xd = torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    q = nv.quantize(xd)
    g = np.float32(host(q.global_scale)[0])
    st = host(nv.error_stats(xd, q))
    y = nv.dequantize(q, torch.bfloat16)
    rows = np.array(sorted({0, 1, 255, 4096, 20000, 32767} |
                           set(np.random.default_rng(9).choice(32768, 40, replace=False).tolist())))
    c, s, _ = oracle.quantize(vals[rows], g=g)
    _check_stats(st[rows], oracle.error_stats(vals[rows], c, s, g))
    yb = host(y[torch.from_numpy(rows).to(DEV)].view(torch.int16)).view(np.uint16)
    assert np.array_equal(yb, oracle.dequantize_bf16(c, s, g))
    rel = np.sqrt(st[:, 1].sum() / st[:, 0].sum())
    _say("A4 relative error %.4f" % rel)
    assert 0.01 < rel < 0.2
