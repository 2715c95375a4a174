"""The hot path inside a captured HIP graph (torch.cuda.CUDAGraph on ROCm):
the decode step (activation quantisation with a given global, then the
streaming GEMM), the self-calibrated quantisation chain (init, amax,
finalise, quantise) followed by the GEMM, and a pipelined-GEMM shape.  The
library records no memset, allocation or synchronisation, so a serving loop
can replay these launches without host work.  Each graph is replayed
several times on new input data, with eager library calls and
synchronisations between replays, and every replay is compared bit for bit
with eager calls on the same data.
"""
import numpy as np
import pytest
import torch

import nvfp4_w4a4_quantized_03_amd as nv
from test_gpu_parity import DEV

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[gpu-graph]", *a, flush=True)


def _same(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def _data(rng, shape, scale=1.0):
    v = rng.standard_normal(shape).astype(np.float32) * np.float32(scale)
    return torch.from_numpy(v).to(DEV).to(torch.bfloat16)


@pytest.mark.parametrize("m,n,k,mode", [(32, 10240, 5120, "given"), (32, 4096, 1024, "compute"),
                                        (300, 320, 256, "given")])
def test_quantize_and_gemm_replayed_from_a_graph(m, n, k, mode):
    _say("graph", m, n, k, mode)
    rng = np.random.default_rng(m + n + k)
    x = _data(rng, (m, k))
    qw = nv.quantize(_data(rng, (n, k), 0.05))
    gx = nv.quantize(x).global_scale.clone()
    codes = torch.empty((m, k // 2), dtype=torch.uint8, device=DEV)
    scales = torch.empty((m, k // 16), dtype=torch.uint8, device=DEV)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)

    def step():
        q = nv.quantize(x, global_scale=gx if mode == "given" else None, out=(codes, scales))
        nv.gemm(q, qw, out_dtype=torch.bfloat16, out=y)
        return q

    # warm-up on a side stream, as torch's capture expects, then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        qg = step()
    torch.cuda.synchronize()

    for trial in range(4):
        x.copy_(_data(rng, (m, k), 1.0 + trial))   # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        q_ref = nv.quantize(x, global_scale=gx if mode == "given" else None)
        y_ref = nv.gemm(q_ref, qw, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert _same(codes, q_ref.codes) and _same(scales, q_ref.scales), trial
        assert _same(qg.global_scale, q_ref.global_scale), trial
        assert _same(y, y_ref), trial
