"""Seeded random sweep of W4A4 GEMM shapes through the C ABI, against the
exact oracle product.  The shapes fall on every kernel the library picks
(skinny tiles for m or n up to 64 with either K-group size, the pipelined
kernel, the staged kernel for ragged k or unaligned scale arrays), with
ragged edges, both output types, the gate epilogues and strided outputs.

Bars as in test_gpu_parity: fp32 output within relative Frobenius error
1e-5 of the exact product (gated: of the gate of it); bf16 output within
one bf16 ulp of the exact value rounded to bf16; output columns past n
untouched.
"""
import numpy as np
import pytest
import torch

import nvfp4_w4a4_quantized_03_amd as nv
import oracle
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
    """The same bytes at an odd address (scale arrays have no alignment
    requirement in the ABI; misaligned ones take the guarded kernel)."""
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
    if case["odd_scales"]:
        qa = nv.NVFP4(qa.codes, _shifted(qa.scales), qa.global_scale)
        qb = nv.NVFP4(qb.codes, _shifted(qb.scales), qb.global_scale)
    od = torch.float32 if case["out"] == "f32" else torch.bfloat16
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
