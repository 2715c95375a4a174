"""Full-size parity with the CPU oracle, every element compared.

For the four hidden-5120 workloads (in_proj 4096 x 12288, the gate
projections 32768 x 64 and their fused b|a pair, the harmonised fused group
8192 x 17536, long prefill 32768 x 10240 and its 32-row decode batch), at
their full shapes and in the launch configuration the benchmark times:

  * every code byte, scale byte and global of every tensor, bit-exact
    (self-calibrated globals, as the benchmark's given globals are);
  * every byte of the harmonised fused-group scales;
  * every GEMM output: fp32 output within relative Frobenius error 1e-5 of
    the oracle over the whole of Y; bf16 output within one bf16 ulp of the
    oracle rounded to bf16, element by element; gate outputs element by
    element within the bound that fp32 accumulation and fp32 evaluation
    of the gate allow (gate_bound below), and within 1e-5 rel-Frob.

The oracle's operands come from oracle.quantize of the same seeded inputs
(never from the device); its GEMM runs in float64 blocks of rows.
"""
import functools

import numpy as np
import pytest
import torch

import nvfp4_w4a4_quantized_03_amd as nv
import oracle
import synth
from test_gpu_parity import DEV, TOL, host, up, workload

pytestmark = pytest.mark.gpu
U = 2.0 ** -24          # binary32 unit roundoff


def _say(*a):
    print("[gpu-fullsize]", *a, flush=True)


@functools.lru_cache(maxsize=None)
def oracle_q(w, name):
    """The oracle's NVFP4 form of a workload tensor (its own global)."""
    return oracle.quantize(workload(w, name)[0])


ALL_TENSORS = [(w, n) for w in (2, 3, 4, 5)
               for (n, *_rest) in synth.WORKLOADS[w]["tensors"]]


def assert_same_bytes(dev, ref, what):
    bad = np.nonzero(dev != ref)
    assert bad[0].size == 0, (what, "first differing (row, byte)",
                              list(zip(bad[0][:5].tolist(), bad[1][:5].tolist())),
                              dev[bad][:5], ref[bad][:5], bad[0].size)


@pytest.mark.parametrize("w,name", ALL_TENSORS, ids=lambda v: str(v))
def test_quantize_every_element(w, name):
    vals, bits, dt = workload(w, name)
    _say("quantize every element", w, name, vals.shape)
    q = nv.quantize(up(vals, bits, dt))
    rc, rs, rg = oracle_q(w, name)
    g_dev = np.float32(host(q.global_scale)[0])
    assert g_dev.view(np.uint32) == np.float32(rg).view(np.uint32), (g_dev, rg)
    assert_same_bytes(host(q.scales), rs, "scales")
    assert_same_bytes(host(q.codes), rc, "codes")


def ulp_check_block(got16, ref):
    """bf16 output (as float64) within one bf16 ulp of bf16(ref)."""
    ref16, _ = oracle.bf16_rne_from_f64(ref)
    mag = np.maximum(np.abs(ref16), np.abs(got16))
    _, e = np.frexp(np.where(mag > 0, mag, 1.0))
    ulp = np.ldexp(1.0, np.maximum(e - 8, -133))
    bad = np.abs(got16 - ref16) > ulp
    assert not bad.any(), ("bf16 beyond one ulp at", np.argwhere(bad)[:5],
                           got16[bad][:5], ref16[bad][:5])


def compare_full(ref_blocks, y32=None, y16=None):
    """Every row block of the oracle's product against the device outputs:
    fp32 by relative Frobenius error over the whole matrix, bf16 element by
    element.  Returns the fp32 relative error (or None)."""
    num = den = 0.0
    for r0, yb in ref_blocks:
        n = yb.shape[0]
        if y32 is not None:
            got = host(y32[r0:r0 + n]).astype(np.float64)
            num += float(np.sum((got - yb) ** 2))
            den += float(np.sum(yb ** 2))
        if y16 is not None:
            ulp_check_block(host(y16[r0:r0 + n].float()).astype(np.float64), yb)
    if y32 is None:
        return None
    err = (num / max(den, 1e-300)) ** 0.5
    _say("full rel-Frob", err)
    assert err <= TOL
    return err


def abs_product(qa, qb):
    """sum_k |A_hat[i, k]| |B_hat[j, k]| g_a g_b, float64 (the magnitude that
    bounds fp32 accumulation error of y[i, j])."""
    b = np.abs(oracle.decoded_units(qb[0], qb[1])).astype(np.float64).T * 2.0 ** -10
    out = np.empty((qa[0].shape[0], b.shape[1]))
    for r0 in range(0, qa[0].shape[0], 4096):
        a = np.abs(oracle.decoded_units(qa[0][r0:r0 + 4096], qa[1][r0:r0 + 4096])
                   ).astype(np.float64) * 2.0 ** -10
        out[r0:r0 + a.shape[0]] = a @ b
    return out * float(qa[2]) * float(qb[2])


def gate_bound(kind, y, sabs, k, a_log=None, dt_bias=None):
    """Reference gate value and an elementwise bound on |device - reference|.

    y is the exact product and sabs the sum of |terms|.  The device's fp32
    y carries at most (k/16 + 16) roundings of partial sums (one per 16-K
    MFMA step, the cross-wave sums and the global factor), so
    |y_dev - y| <= ey = (k/16 + 16) u sabs.  The gate then moves by at most
    |f'(y)| ey e^(L ey), L bounding |d ln|f'| / dy| (1 for the sigmoids,
    1 + e^A_log for alpha = exp(-e^A_log softplus(y + dt_bias)), whose fp32
    sum y + dt_bias adds u |y + dt_bias| to ey), plus the fp32 evaluation
    error of the gate itself, u (8 + 4 |ln f|) f, plus the smallest normal
    binary32 for results that underflow."""
    ey = (k / 16.0 + 16.0) * U * sabs
    if kind == "beta":
        f = oracle.gate_beta(y)
        fp, lip = f * (1.0 - f), 1.0
    elif kind == "alpha":
        f = oracle.gate_alpha(y)
        fp, lip = f * (1.0 - f), 1.0
    else:
        c = np.exp(np.asarray(a_log, dtype=np.float64))[None, :]
        x = y + np.asarray(dt_bias, dtype=np.float64)[None, :]
        _, f = oracle.gdn_gates(y, 0, a_log, dt_bias)
        ey = ey + U * np.abs(x)
        fp, lip = c * oracle.gate_beta(x) * f, 1.0 + c
    with np.errstate(divide="ignore"):
        lnf = np.where(f > 0, np.abs(np.log(np.where(f > 0, f, 1.0))), 0.0)
    bound = fp * ey * np.exp(np.minimum(lip * ey, 50.0)) + U * (8.0 + 4.0 * lnf) * f \
        + 2.0 ** -126
    return f, bound


def check_gate(got, kind, y, sabs, k, a_log=None, dt_bias=None):
    f, bound = gate_bound(kind, y, sabs, k, a_log, dt_bias)
    got = np.asarray(got, dtype=np.float64)
    bad = np.abs(got - f) > bound
    assert not bad.any(), (kind, "gate beyond its bound at", np.argwhere(bad)[:5],
                           got[bad][:5], f[bad][:5], bound[bad][:5])
    err = float(np.linalg.norm(got - f) / np.linalg.norm(f))
    assert err <= TOL, err
    rel = np.abs(got - f) / np.maximum(np.abs(f), 2.0 ** -126)
    _say(kind, "rel-Frob", err, "max elementwise relative error", float(rel.max()))


# ----------------------------------------------------------------- GEMMs

def test_gemm_in_proj_every_output():
    """in_proj X[4096x5120] x W[12288x5120] -> bf16 and fp32, all of Y."""
    _say("gemm in_proj 4096x12288x5120 every output")
    xv, xb, xt = workload(2, "x")
    wv, wb, wt = workload(2, "w")
    qa, qb = nv.quantize(up(xv, xb, xt)), nv.quantize(up(wv, wb, wt))
    y16 = nv.gemm(qa, qb, out_dtype=torch.bfloat16)
    y32 = nv.gemm(qa, qb, out_dtype=torch.float32)
    compare_full(oracle.gemm_f64_row_blocks(*oracle_q(2, "x"), *oracle_q(2, "w")),
                 y32, y16)


def test_gemm_prefill_and_decode_every_output():
    """Long prefill X[32768x5120] and decode X[32x5120] against
    W[10240x5120]: the benchmark's calls (activation quantised with its
    global given, bf16 out), plus fp32 out; all of Y."""
    _say("gemm prefill 32768x10240x5120 + decode 32 every output")
    xv, xb, xt = workload(5, "x")
    dv, db, dt_ = workload(5, "x_dec")
    wv, wb, wt = workload(5, "w")
    qb = nv.quantize(up(wv, wb, wt))
    xd = up(xv, xb, xt)
    gx = nv.quantize(xd).global_scale.clone()
    qa = nv.quantize(xd, global_scale=gx)             # the benchmark's call
    del xd
    ra, rb = oracle_q(5, "x"), oracle_q(5, "w")
    assert_same_bytes(host(qa.codes), ra[0], "codes (given global)")
    y16 = nv.gemm(qa, qb, out_dtype=torch.bfloat16)
    y32 = nv.gemm(qa, qb, out_dtype=torch.float32)
    compare_full(oracle.gemm_f64_row_blocks(*ra, *rb), y32, y16)
    del y16, y32
    qd = nv.quantize(up(dv, db, dt_))
    yd16 = nv.gemm(qd, qb, out_dtype=torch.bfloat16)
    yd32 = nv.gemm(qd, qb, out_dtype=torch.float32)
    compare_full(oracle.gemm_f64_row_blocks(*oracle_q(5, "x_dec"), *rb), yd32, yd16)


def test_fused_group_every_scale_and_output():
    """Three modules with their own globals quantised into row slices of
    one fused buffer, harmonised to one global (every scale byte and every
    code byte compared), then the GEMM with X[8192x5120] (all of Y)."""
    _say("fused group 12288|5120|128 harmonise + gemm 8192x17536x5120")
    mods = ["w1", "w2", "w3"]
    sizes = [synth.workload_shape(4, m)[0] for m in mods]
    k = 5120
    offs = [0] + [int(v) for v in np.cumsum(sizes)]
    codes = torch.empty((offs[-1], k // 2), dtype=torch.uint8, device=DEV)
    scales = torch.empty((offs[-1], k // 16), dtype=torch.uint8, device=DEV)
    gdev = torch.empty(3, dtype=torch.float32, device=DEV)
    for i, mname in enumerate(mods):
        vals, bits, dt = workload(4, mname)
        q = nv.quantize(up(vals, bits, dt), out=(codes[offs[i]:offs[i + 1]],
                                                 scales[offs[i]:offs[i + 1]]))
        gdev[i:i + 1].copy_(q.global_scale)
    gstar = nv.harmonize_group(scales, k, offs, gdev)
    parts = [oracle_q(4, m) for m in mods]
    rc = np.concatenate([p[0] for p in parts])
    rs, g_ref = oracle.harmonize(np.concatenate([p[1] for p in parts]), offs,
                                 [p[2] for p in parts])
    assert np.float32(host(gstar)[0]).view(np.uint32) == np.float32(g_ref).view(np.uint32)
    assert_same_bytes(host(scales), rs, "harmonised scales")
    assert_same_bytes(host(codes), rc, "fused codes")
    xv, xb, xt = workload(4, "x")
    qa = nv.quantize(up(xv, xb, xt))
    wq = nv.NVFP4(codes, scales, gstar)
    y16 = nv.gemm(qa, wq, out_dtype=torch.bfloat16)
    y32 = nv.gemm(qa, wq, out_dtype=torch.float32)
    compare_full(oracle.gemm_f64_row_blocks(*oracle_q(4, "x"), rc, rs, g_ref), y32, y16)


def test_gate_projections_every_output():
    """X[32768x5120] x W_a / W_b [64x5120]: fp32 y and the alpha / beta
    epilogues on every element."""
    xv, xb, xt = workload(3, "x")
    qa = nv.quantize(up(xv, xb, xt))
    ra = oracle_q(3, "x")
    for name, epi in (("w_a", "alpha"), ("w_b", "beta")):
        _say("gate projection 32768x64x5120", name, epi)
        wv, wb, wt = workload(3, name)
        qb = nv.quantize(up(wv, wb, wt))
        rb = oracle_q(3, name)
        y = oracle.gemm_f64(*ra, *rb)
        sabs = abs_product(ra, rb)
        y32 = nv.gemm(qa, qb, out_dtype=torch.float32)
        compare_full([(0, y)], y32)
        g = nv.gemm(qa, qb, out_dtype=torch.float32, epilogue=epi)
        check_gate(host(g), epi, y, sabs, 5120)


def test_gdn_gate_pair_every_output():
    """The fused b|a group (64 + 64 heads, harmonised) through the gate-pair
    call: every beta and alpha against the oracle's gates of the exact
    product, element by element."""
    _say("gdn gate pair 32768x(64+64)x5120 every output")
    k, nb, na = 5120, 64, 64
    xv, xb, xt = workload(3, "x")
    codes = torch.empty((nb + na, k // 2), dtype=torch.uint8, device=DEV)
    scales = torch.empty((nb + na, k // 16), dtype=torch.uint8, device=DEV)
    gdev = torch.empty(2, dtype=torch.float32, device=DEV)
    for i, (name, lo, hi) in enumerate((("w_b", 0, nb), ("w_a", nb, nb + na))):
        v, b, t = workload(3, name)
        q = nv.quantize(up(v, b, t), out=(codes[lo:hi], scales[lo:hi]))
        gdev[i:i + 1].copy_(q.global_scale)
    gstar = nv.harmonize_group(scales, k, [0, nb, nb + na], gdev)
    qa = nv.quantize(up(xv, xb, xt))
    rng = np.random.default_rng(77)
    a_log = rng.uniform(-2.0, 1.5, na).astype(np.float32)
    dtb = rng.uniform(-3.0, 3.0, na).astype(np.float32)
    beta, alpha = nv.gdn_gates(qa, nv.NVFP4(codes, scales, gstar), nb,
                               torch.from_numpy(a_log).to(DEV),
                               torch.from_numpy(dtb).to(DEV))
    pb, pa = oracle_q(3, "w_b"), oracle_q(3, "w_a")
    bs_h, g_ref = oracle.harmonize(np.concatenate([pb[1], pa[1]]), [0, nb, nb + na],
                                   [pb[2], pa[2]])
    rw = (np.concatenate([pb[0], pa[0]]), bs_h, g_ref)
    ra = oracle_q(3, "x")
    y = oracle.gemm_f64(*ra, *rw)
    sabs = abs_product(ra, rw)
    check_gate(host(beta), "beta", y[:, :nb], sabs[:, :nb], k)
    check_gate(host(alpha), "gdn_alpha", y[:, nb:], sabs[:, nb:], k, a_log, dtb)
