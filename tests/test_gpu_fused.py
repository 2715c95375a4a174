"""Parity of the one-launch small-M activation quantise + GEMM
(w4a4_gemm_quantize_a, through its C ABI) with the CPU oracle and with the
two separate library calls it replaces.

Bars: the NVFP4 form of X (codes, scales, global) bit-exact with the
oracle's quantisation; Y bit-identical to nvfp4_quantize + w4a4_gemm on the
same device (the fused kernel runs the same tiles in the same K order);
against the exact oracle product, Y within relative Frobenius error 1e-5
(fp32) or one bf16 ulp (bf16).
"""
import ctypes

import numpy as np
import pytest
import torch

import nvfp4_w4a4_quantized_03_amd as nv
import oracle
from test_gpu_parity import (DEV, TOL, _sampled_gemm_check, bf16_dev,
                             check_bf16_within_one_ulp, check_quant, host,
                             rel_frob, sample_rows, up, workload)

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[gpu-fused]", *a, flush=True)


def _bits(t):
    """Raw bits of a device tensor, for bit-for-bit comparisons."""
    if t.dtype == torch.bfloat16:
        return host(t.view(torch.int16))
    if t.dtype == torch.float32:
        return host(t.view(torch.int32))
    return host(t)


def _same_bits(a, b):
    return np.array_equal(_bits(a), _bits(b))


def _operands(m, n, k, xdt, seed):
    rng = np.random.default_rng(seed)
    xv = rng.standard_normal((m, k)).astype(np.float32)
    xv[:, rng.integers(0, k, 3)] *= np.float32(40.0)     # outlier channels
    wv = (rng.standard_normal((n, k)) * 0.05).astype(np.float32)
    if xdt == "bf16":
        xv, xd = bf16_dev(xv)
    else:
        xd = up(xv, None, "f32")
    qw = nv.quantize(up(wv, None, "f32"))
    return xv, xd, wv, qw


def _check_against_separate_and_oracle(xv, xd, wv, qw, gt, out_dtype):
    qx, y = nv.gemm_quantize_a(xd, qw, global_scale=gt, out_dtype=out_dtype)
    g_ref = None if gt is None else np.float32(host(gt)[0])
    check_quant(xv, qx, g=g_ref)
    qs = nv.quantize(xd, global_scale=gt)
    assert _same_bits(qx.codes, qs.codes) and _same_bits(qx.scales, qs.scales)
    assert _same_bits(qx.global_scale, qs.global_scale)
    ys = nv.gemm(qs, qw, out_dtype=out_dtype)
    assert _same_bits(y, ys), "fused Y differs from quantize + gemm"
    g_used = oracle.global_scale(xv) if g_ref is None else g_ref
    ref = oracle.gemm_exact_int(*oracle.quantize(xv, g=g_used),
                                *oracle.quantize(wv))
    if out_dtype == torch.float32:
        assert rel_frob(host(y).astype(np.float64), ref) <= TOL
    else:
        check_bf16_within_one_ulp(y, ref)


# k a whole number of streaming stages takes the streaming GEMM's tiles
# (incl. 24-row S slices: (7, 4109, 512), (64, 4100, 1024); 40-row slices:
# (20, 10007, 512); 33-64-row L with 512-K stages: (48, 6001, 512)), other k
# the skinny kernel's
@pytest.mark.parametrize("m,n,k", [(1, 1, 128), (1, 64, 128), (7, 100, 384),
                                   (32, 300, 512), (33, 96, 256),
                                   (64, 130, 640), (17, 33, 1024),
                                   (64, 4100, 1024), (2, 1000, 5120),
                                   (7, 4109, 512), (48, 6001, 512),
                                   (20, 10007, 512)])
@pytest.mark.parametrize("xdt,mode", [("f32", "compute"), ("bf16", "compute"),
                                      ("f32", "given"), ("bf16", "given")])
def test_fused_matches_separate_calls(m, n, k, xdt, mode):
    _say("fused", m, n, k, xdt, mode)
    xv, xd, wv, qw = _operands(m, n, k, xdt, m * 131 + n * 7 + k)
    gt = None
    if mode == "given":
        g = np.float32(oracle.global_scale(xv) * np.float32(1.25))
        gt = torch.tensor([g], dtype=torch.float32, device=DEV)
    for od in (torch.float32, torch.bfloat16):
        _check_against_separate_and_oracle(xv, xd, wv, qw, gt, od)


def test_fused_decode_full_size():
    """The decode projection: 32 x 5120 bf16 activations, 10240 x 5120
    weights, in the launch configuration the benchmark times."""
    dv, db, dt_ = workload(5, "x_dec")
    wv, wb, wt = workload(5, "w")
    _say("fused decode 32x10240x5120")
    qw = nv.quantize(up(wv, wb, wt))
    xd = up(dv, db, dt_)
    for od in (torch.bfloat16, torch.float32):
        qx, y = nv.gemm_quantize_a(xd, qw, out_dtype=od)
        check_quant(dv, qx)
        qs = nv.quantize(xd)
        assert _same_bits(y, nv.gemm(qs, qw, out_dtype=od))
        cols = sample_rows(10240, 512, 54)
        _sampled_gemm_check(dv, qx, wv, qw, np.arange(32), cols, y, od)


def test_fused_more_tiles_than_resident_workgroups():
    """n = 80000: 2500 output tiles, more than the device holds at once, so
    every workgroup loops over several tiles after the barrier."""
    m, n, k = 32, 80000, 256
    xv, xd, wv, qw = _operands(m, n, k, "bf16", 77)
    _say("fused wide", m, n, k)
    qx, y = nv.gemm_quantize_a(xd, qw, out_dtype=torch.float32)
    check_quant(xv, qx)
    assert _same_bits(y, nv.gemm(nv.quantize(xd), qw, out_dtype=torch.float32))
    cols = sample_rows(n, 256, 78)
    _sampled_gemm_check(xv, qx, wv, qw, np.arange(m), cols, y, torch.float32)


def test_fused_reuses_output_buffers():
    """Two calls in a row on the same output buffers, the second with
    fewer rows and other data: nothing stale from the first is read."""
    k, n = 512, 200
    lib = nv.library()
    xc = torch.empty((64, k // 2), dtype=torch.uint8, device=DEV)
    xs = torch.empty((64, k // 16), dtype=torch.uint8, device=DEV)
    xg = torch.empty(1, dtype=torch.float32, device=DEV)
    y = torch.empty((64, n), dtype=torch.float32, device=DEV)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for m, seed in ((64, 1), (20, 2)):
        xv, xd, wv, qw = _operands(m, n, k, "f32", 900 + seed)
        _say("fused reuse", m)
        rc = lib.w4a4_gemm_quantize_a(
            xd.data_ptr(), nv.DTYPE_F32, m, k, k, xc.data_ptr(), xs.data_ptr(),
            xg.data_ptr(), nv.GLOBAL_COMPUTE, qw.codes.data_ptr(),
            qw.scales.data_ptr(), qw.global_scale.data_ptr(), n, y.data_ptr(),
            nv.DTYPE_F32, n, stream)
        assert rc == 0, lib.nvfp4_status_string(rc)
        check_quant(xv, nv.NVFP4(xc[:m], xs[:m], xg))
        ref = oracle.gemm_exact_int(*oracle.quantize(xv), *oracle.quantize(wv))
        assert rel_frob(host(y[:m]).astype(np.float64), ref) <= TOL


def test_fused_zero_activations():
    """X = 0: g = 0, every scale and code 0, Y exactly +0."""
    m, n, k = 5, 70, 256
    _, _, wv, qw = _operands(m, n, k, "f32", 5)
    xd = torch.zeros((m, k), dtype=torch.float32, device=DEV)
    qx, y = nv.gemm_quantize_a(xd, qw, out_dtype=torch.float32)
    assert host(qx.global_scale)[0] == 0
    assert not host(qx.codes).any() and not host(qx.scales).any()
    assert not _bits(y).any()


@pytest.mark.parametrize("xdt", ["f32", "bf16"])
def test_fused_strided_activations(xdt):
    """X as a column slice of a wider tensor (row stride 400 > k = 384): the
    quantise phase takes the strided block addressing."""
    m, n, k, ld = 20, 150, 384, 400
    rng = np.random.default_rng(31)
    full = rng.standard_normal((m, ld)).astype(np.float32)
    wv = (rng.standard_normal((n, k)) * 0.05).astype(np.float32)
    qw = nv.quantize(up(wv, None, "f32"))
    if xdt == "bf16":
        fv, fd = bf16_dev(full)
    else:
        fv, fd = full, up(full, None, "f32")
    xv, xd = fv[:, :k], fd[:, :k]
    _say("fused strided", xdt)
    for gt in (None, torch.tensor([np.float32(oracle.global_scale(xv) * 2)],
                                  dtype=torch.float32, device=DEV)):
        _check_against_separate_and_oracle(xv, xd, wv, qw, gt, torch.float32)
