"""Parity of the FP8 KV-cache calls (through the C ABI) with the CPU
oracle: the running amax and the static scale bit-exact, every cast code
bit-exact (both sides decide each rounding exactly)."""
import numpy as np
import pytest
import torch

import nvfp4_w4a4_quantized_03_amd as nv
import oracle
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(*a):
    print("[gpu-fp8kv]", *a, flush=True)


def host(t):
    return t.cpu().numpy()


def _dev(x, dtype):
    if dtype == "bf16":
        bits = synth.bf16_bits_from_f32(x)
        return synth.f32_from_bf16_bits(bits), \
            torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    return x, torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


@pytest.mark.parametrize("rows,k,dtype", [(1, 16, "f32"), (7, 48, "bf16"),
                                          (300, 272, "bf16"), (33, 1040, "f32")])
def test_calibrate_and_cast(rows, k, dtype):
    _say("calibrate+cast", rows, k, dtype)
    rng = np.random.default_rng(rows * 13 + k)
    parts = [(rng.standard_normal((rows, k)) * 2.0 ** rng.integers(-4, 5)).astype(np.float32)
             for _ in range(3)]
    parts[1][0, 3] = 80.0                                  # an outlier sets the amax
    host_vals, devs = zip(*[_dev(p, dtype) for p in parts])
    scale, amax = nv.fp8_kv_calibrate(list(devs))
    a_ref = oracle.kv_amax(host_vals)
    s_ref = oracle.kv_scale(a_ref)
    assert np.float32(host(amax)[0]).view(np.uint32) == a_ref.view(np.uint32)
    assert np.float32(host(scale)[0]).view(np.uint32) == s_ref.view(np.uint32)
    # cast a fresh tensor (values above the calibrated range saturate)
    x = (rng.standard_normal((rows, k)) * 30).astype(np.float32)
    xv, xd = _dev(x, dtype)
    got = host(nv.fp8_kv_cast(xd, scale))
    assert np.array_equal(got, oracle.kv_cast(xv, s_ref))


@pytest.mark.parametrize("s", [0.0, 2.0 ** -120, 3.7e-3, 1.0, 6.0e25, 2.0 ** 110])
def test_cast_scale_range_midpoints_and_signs(s):
    """Every scale regime (zero, extreme, normal) with values placed exactly
    on E4M3 rounding midpoints, both zeros and saturating values."""
    _say("cast scale", s)
    s = np.float32(s)
    rng = np.random.default_rng(1)
    mids = [(float(oracle.e4m3_decode(c)) + float(oracle.e4m3_decode(c + 1))) / 2
            for c in range(126)]
    vals = [m * float(s) for m in mids] + [0.0, -0.0, 1e30, -1e30]
    vals += list(rng.standard_normal(222) * float(s) * 50.0)
    x = np.array(vals[:256], dtype=np.float32)
    x = np.where(np.isfinite(x), x, 0.0).astype(np.float32).reshape(16, 16)
    got = host(nv.fp8_kv_cast(torch.from_numpy(x).to(DEV),
                              torch.tensor([s], dtype=torch.float32, device=DEV)))
    assert np.array_equal(got, oracle.kv_cast(x, s))


def test_cast_strided_and_full_size():
    """A row-strided output, then a 32768 x 1024 bf16 K-cache slab (the
    long-context shape) checked on sampled rows."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((40, 64)) * 3).astype(np.float32)
    big = torch.full((40, 128), 0xAB, dtype=torch.uint8, device=DEV)
    s = torch.tensor([0.05], dtype=torch.float32, device=DEV)
    nv.fp8_kv_cast(torch.from_numpy(x).to(DEV), s, out=big[:, 32:96])
    got = host(big)
    assert np.array_equal(got[:, 32:96], oracle.kv_cast(x, np.float32(0.05)))
    assert np.all(got[:, :32] == 0xAB) and np.all(got[:, 96:] == 0xAB)
    _say("full size 32768x1024")
    xf = (rng.standard_normal((32768, 1024)) * 1.5).astype(np.float32)
    xv, xd = _dev(xf, "bf16")
    scale, _ = nv.fp8_kv_calibrate([xd])
    c = nv.fp8_kv_cast(xd, scale)
    s_ref = oracle.kv_scale(oracle.kv_amax([xv]))
    assert np.float32(host(scale)[0]) == s_ref
    rows = np.array(sorted({0, 1, 4095, 32767} | set(rng.choice(32768, 60, replace=False).tolist())))
    assert np.array_equal(host(c[torch.from_numpy(rows).to(DEV)]), oracle.kv_cast(xv[rows], s_ref))
