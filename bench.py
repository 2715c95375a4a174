"""Benchmark of the NVFP4 W4A4 hot path on one MI355X.

One step = the long-prefill + decode workload at hidden size 5120:
  quantize X[32768 x 5120] bf16 to NVFP4 with a calibrated (given) global,
  W4A4 GEMM against the pre-quantized weight W[10240 x 5120] -> bf16,
  quantize X[32 x 5120] (decode batch), W4A4 GEMM -> bf16.
Inputs are seeded synthetic tensors (synth.py) already resident in HBM when
the timed region starts; the weight is quantised once before timing.

Prints one JSON line: whole-step throughput (TFLOP/s over 2 K N (M + M_dec)
flops), per-kernel HIP-event timings on the launch stream, the GEMM's
roofline fraction against the dense fp16/bf16 MFMA peak, the quantiser's
against HBM, and the CPU oracle timed on a bounded sample of the same work.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--no-cpu-baseline]
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("W4A4 GEMM TFLOP/s + NVFP4 quantize GB/s at K=5120, "
          "as % of MI355X peak")
PEAK_MFMA_TFLOPS = 2500.0        # MI355X dense fp16/bf16 MFMA
PEAK_HBM_GBPS = 8000.0           # MI355X HBM3E
M, M_DEC, N, K = 32768, 32, 10240, 5120
WORKLOAD = 5
KERNEL_SOURCES = ["gemm.hip", "gemm_stream.hip", "quantize.hip", "quant_device.h"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calibration", action="store_true",
                   help="after the timed steps, copy a 512 MiB device buffer "
                   "once (a known-size kernel for scaling HBM counters)")
    p.add_argument("--workloads", action=argparse.BooleanOptionalAction,
                   default=True, help="also time the other four workloads "
                   "once each (reported, not part of the step)")
    return p.parse_args()


def source_hash(name):
    path = os.path.join(ROOT, "nvfp4_w4a4_quantized_03_amd", "csrc", name)
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def measured_traffic(kernel_file, per_launch_units):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", kernel_file)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    src = re.search(r"source_sha256_16:\s*(\w+)", text)
    byt = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    kern = re.search(r"kernel_source:\s*(\S+)", text)
    if not (src and byt and kern) or src.group(1) != source_hash(kern.group(1)):
        return None
    return float(byt.group(1))


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline():
    """The oracle, as it stands, on a bounded sample of the step's work
    (about 10 s of CPU time): quantize 16384 rows of X (numpy, one core)
    and the W4A4 GEMM of 8192 of those rows against all 10240 weight rows
    (float64 BLAS on the decoded operands, all BLAS threads).  Each tensor
    gets its own self-calibrated global, as the GPU step's given globals
    are.  Scaled to the whole step's flops."""
    import oracle
    import synth
    from threadpoolctl import threadpool_info
    GQ, GM, GN = 16384, 8192, N
    xv, _, _ = synth.workload_tensor(WORKLOAD, "x", row_ids=np.arange(GQ))
    wv, _, _ = synth.workload_tensor(WORKLOAD, "w", row_ids=np.arange(GN))
    gx = oracle.global_scale(xv)
    t0 = time.perf_counter()
    qa = oracle.quantize(xv, g=gx)
    tq = time.perf_counter() - t0
    qb = oracle.quantize(wv)
    qa = tuple(t[:GM] if t.ndim else t for t in qa)
    t0 = time.perf_counter()
    oracle.gemm_f64(*qa, *qb)
    tg = time.perf_counter() - t0
    # per-element quantize time and per-flop GEMM time, scaled to one step
    q_elems = (M + M_DEC) * K
    t_step = tq / xv.size * q_elems + tg / (2.0 * GM * GN * K) * \
        (2.0 * (M + M_DEC) * N * K)
    blas = [d for d in threadpool_info() if d.get("user_api") == "blas"]
    blas_threads = max([d.get("num_threads", 1) for d in blas] or [1])
    blas_lib = ", ".join(sorted({"%s %s (%s)" % (d.get("internal_api", "?"),
                                                 d.get("version", "?"),
                                                 os.path.basename(d.get("filepath", "?")))
                                 for d in blas})) or "unknown"
    host_cores = len(os.sched_getaffinity(0))
    return {
        "value": 2.0 * (M + M_DEC) * N * K / t_step / 1e12,
        "unit": "TFLOP/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": ("oracle.quantize of X rows 0..%d (%.2f s, 1 core) and "
                   "oracle.gemm_f64 %dx%dx%d (%.2f s, %d BLAS threads), "
                   "scaled per element / per flop to one step "
                   "(quantize 32800x5120 + GEMM 32800x10240x5120)"
                   % (GQ - 1, tq, GM, GN, K, tg, blas_threads)),
        "quantize_gbps": xv.size * 2.5625 / tq / 1e9,
        "quantize_cores": 1,
        "gemm_tflops": 2.0 * GM * GN * K / tg / 1e12,
        "gemm_cores": int(blas_threads),
        "host_cores": host_cores,
        "cpu_model": _cpu_model(),
        "blas": blas_lib,
        "blas_threads": int(blas_threads),
    }


MALL_BYTES = 256 * 2 ** 20   # MI355X memory-side (infinity) cache


def _time(fn, reps, stream, runs=20):
    """Median GPU time (us) of one call of fn() (HIP events on the launch
    stream): one warm-up call, then `runs` timed batches of calls, a batch
    long enough (>= ~200 us) that the event pair's own cost is small.  fn may
    be a list of equivalent calls on different buffers, used in turn (to
    keep inputs that fit the memory-side cache from being timed warm).
    `reps` is kept for callers and ignored (the batch size is chosen here)."""
    import torch
    fns = fn if isinstance(fn, (list, tuple)) else [fn]
    fns[0]()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    fns[1 % len(fns)]()
    e1.record(stream)
    torch.cuda.synchronize()
    one = max(e0.elapsed_time(e1) * 1e3, 1.0)
    batch = int(min(64, max(1, np.ceil(200.0 / one))))
    times, i = [], 0
    for _ in range(runs):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(batch):
            fns[i % len(fns)]()
            i += 1
        b.record(stream)
        times.append((a, b))
    torch.cuda.synchronize()
    return float(np.median([x.elapsed_time(y) * 1e3 / batch for x, y in times]))


def _copies(nbytes):
    """How many copies of an nbytes input to rotate through so that they
    exceed twice the memory-side cache."""
    return int(max(1, np.ceil(2 * MALL_BYTES / nbytes)))


def other_workloads(nv, synth, dev, stream, reps=10):
    """Kernel timings of the other workloads at hidden size 5120 (inputs
    resident in HBM): in_proj 4096x12288, gate projections 32768x64 with
    alpha/beta epilogues and as one fused b|a GEMM with the full gate pair,
    a harmonised fused group (N = 17536), the tiny
    16x128x256 case, the self-calibrated (COMPUTE) activation quantize, and
    dequantisation to bf16 plus per-row error statistics of the 32768x5120
    activations, the decode projection's activation quantisation + GEMM as
    two calls and as one fused launch, and the FP8 KV-cache scale
    calibration and cast of a 32768x1024 bf16 slab.  Each figure is the
    median of 20 timed batches of calls; bandwidth-bound calls whose inputs
    fit the memory-side cache rotate over copies of them."""
    import numpy as np
    import torch

    def up(w, name):
        v, b, dt = synth.workload_tensor(w, name)
        if dt == "f32":
            return torch.from_numpy(v).to(dev)
        return torch.from_numpy(b.view(np.int16)).to(dev).view(torch.bfloat16)

    out = {}
    # in_proj: X[4096x5120], W[12288x5120]; both quantisations rotate over
    # copies of their input and output (together over twice the memory-side
    # cache), so that no call finds them cached
    x, w = up(2, "x"), up(2, "w")
    qx, qw = nv.quantize(x), nv.quantize(w)
    gx = qx.global_scale.clone()
    nxc = _copies(4096 * 5120 * 2.5625)
    xs = [x.clone() for _ in range(nxc)]
    qxs = [(torch.empty_like(qx.codes), torch.empty_like(qx.scales)) for _ in range(nxc)]
    t_q = _time([lambda i=i: nv.quantize(xs[i], global_scale=gx, out=qxs[i]) for i in range(nxc)],
                reps, stream)
    del xs, qxs
    nwc = _copies(12288 * 5120 * 4.5625)
    ws = [w.clone() for _ in range(nwc)]
    qws = [(torch.empty_like(qw.codes), torch.empty_like(qw.scales)) for _ in range(nwc)]
    t_qw = _time([lambda i=i: nv.quantize(ws[i], out=qws[i]) for i in range(nwc)], reps, stream)
    del ws, qws
    y = torch.empty((4096, 12288), dtype=torch.bfloat16, device=dev)
    t_g = _time(lambda: nv.gemm(qx, qw, out_dtype=torch.bfloat16, out=y), reps, stream)
    fl = 2.0 * 4096 * 12288 * 5120
    out["in_proj_4096x12288x5120"] = {
        "quantize_x_us": t_q, "quantize_x_gbps": 4096 * 5120 * 2.5625 / t_q / 1e3,
        "quantize_w_compute_us": t_qw,
        "gemm_us": t_g, "gemm_tflops": fl / t_g / 1e6}
    del x, w, qx, qw, y
    # gate projections: X[32768x5120], W_a/W_b[64x5120], fp32 out + gates;
    # the 94 MB of quantised activations fit the memory-side cache, so the
    # calls rotate over copies of them
    x = up(3, "x")
    qx = nv.quantize(x)
    nqc = _copies(32768 * 5120 * 0.5625)
    qxs = [nv.NVFP4(qx.codes.clone(), qx.scales.clone(), qx.global_scale) for _ in range(nqc)]
    res = {}
    for name, epi in (("w_a", "alpha"), ("w_b", "beta")):
        qw = nv.quantize(up(3, name))
        y = torch.empty((32768, 64), dtype=torch.float32, device=dev)
        t = _time([lambda q=q: nv.gemm(q, qw, out_dtype=torch.float32, epilogue=epi, out=y)
                   for q in qxs], reps, stream)
        byts = 32768 * 5120 * 0.5625 + 64 * 5120 * 0.5625 + 32768 * 64 * 4
        res[name + "_" + epi] = {"gemm_us": t, "gbps": byts / t / 1e3,
                                 "frac_hbm_peak": byts / t / 1e3 / PEAK_HBM_GBPS}
    out["gate_proj_32768x64x5120"] = res
    # the same two projections as one fused b|a GEMM with the full gate pair
    codes = torch.empty((128, 2560), dtype=torch.uint8, device=dev)
    scales = torch.empty((128, 320), dtype=torch.uint8, device=dev)
    gmod = torch.empty(2, dtype=torch.float32, device=dev)
    for i, name in enumerate(("w_b", "w_a")):
        q = nv.quantize(up(3, name), out=(codes[64 * i:64 * (i + 1)], scales[64 * i:64 * (i + 1)]))
        gmod[i:i + 1].copy_(q.global_scale)
    wba = nv.NVFP4(codes, scales, nv.harmonize_group(scales, 5120, [0, 64, 128], gmod))
    a_log = torch.linspace(-2.0, 1.5, 64, device=dev)
    dt_bias = torch.linspace(-3.0, 3.0, 64, device=dev)
    gb = (torch.empty((32768, 64), dtype=torch.float32, device=dev),
          torch.empty((32768, 64), dtype=torch.float32, device=dev))
    t = _time([lambda q=q: nv.gdn_gates(q, wba, 64, a_log, dt_bias, out=gb) for q in qxs],
              reps, stream)
    byts = 32768 * 5120 * 0.5625 + 128 * 5120 * 0.5625 + 32768 * 128 * 4
    out["gdn_gates_fused_ba_32768x128x5120"] = {
        "gemm_us": t, "gbps": byts / t / 1e3,
        "frac_hbm_peak": byts / t / 1e3 / PEAK_HBM_GBPS}
    del x, qx, qxs
    # harmonised fused group 12288|5120|128 with X[8192x5120]
    sizes = [12288, 5120, 128]
    offs = [0, 12288, 17408, 17536]
    codes = torch.empty((17536, 2560), dtype=torch.uint8, device=dev)
    scales = torch.empty((17536, 320), dtype=torch.uint8, device=dev)
    gmod = torch.empty(3, dtype=torch.float32, device=dev)
    for i, nm in enumerate(("w1", "w2", "w3")):
        q = nv.quantize(up(4, nm), out=(codes[offs[i]:offs[i + 1]], scales[offs[i]:offs[i + 1]]))
        gmod[i:i + 1].copy_(q.global_scale)
    saved = scales.clone()

    def harm():
        scales.copy_(saved)
        return nv.harmonize_group(scales, 5120, offs, gmod)
    t_copy = _time(lambda: scales.copy_(saved), reps, stream)
    t_h = _time(harm, reps, stream) - t_copy
    gstar = harm()
    x = up(4, "x")
    qx = nv.quantize(x)
    y = torch.empty((8192, 17536), dtype=torch.bfloat16, device=dev)
    wq = nv.NVFP4(codes, scales, gstar)
    t_g = _time(lambda: nv.gemm(qx, wq, out_dtype=torch.bfloat16, out=y), reps, stream)
    out["fused_group_8192x17536x5120"] = {
        "harmonize_us": t_h, "gemm_us": t_g,
        "gemm_tflops": 2.0 * 8192 * 17536 * 5120 / t_g / 1e6}
    del x, qx, y, codes, scales
    # tiny: 16x128x256 fp32
    x, w = up(1, "x"), up(1, "w")
    qx, qw = nv.quantize(x), nv.quantize(w)
    t_q = _time(lambda: nv.quantize(x), reps, stream)
    t_g = _time(lambda: nv.gemm(qx, qw, out_dtype=torch.float32), reps, stream)
    out["tiny_16x128x256"] = {"quantize_compute_us": t_q, "gemm_us": t_g}
    # self-calibrated quantize of the long-prefill activations
    xv = up(5, "x")
    q = nv.quantize(xv)
    t_c = _time(lambda: nv.quantize(xv, out=(q.codes, q.scales)), reps, stream)
    out["quantize_compute_32768x5120"] = {
        "us": t_c, "gbps_4.5625B_per_elem": 32768 * 5120 * 4.5625 / t_c / 1e3}
    # dequantise (fake-quant half) to bf16 and per-row error statistics
    yb = torch.empty((32768, 5120), dtype=torch.bfloat16, device=dev)
    t_d = _time(lambda: nv.dequantize(q, torch.bfloat16, out=yb), reps, stream)
    del yb
    yf = torch.empty((32768, 5120), dtype=torch.float32, device=dev)
    t_f = _time(lambda: nv.dequantize(q, torch.float32, out=yf), reps, stream)
    del yf
    t_e = _time(lambda: nv.error_stats(xv, q), reps, stream)
    elems = 32768 * 5120
    out["dequantize_error_stats_32768x5120"] = {
        "dequantize_bf16_us": t_d,
        "dequantize_gbps_2.5625B_per_elem": elems * 2.5625 / t_d / 1e3,
        "dequantize_frac_hbm_peak": elems * 2.5625 / t_d / 1e3 / PEAK_HBM_GBPS,
        "dequantize_f32_us": t_f,
        "dequantize_f32_gbps_4.5625B_per_elem": elems * 4.5625 / t_f / 1e3,
        "dequantize_f32_frac_hbm_peak": elems * 4.5625 / t_f / 1e3 / PEAK_HBM_GBPS,
        "error_stats_us": t_e,
        "error_stats_gbps_2.5625B_per_elem": elems * 2.5625 / t_e / 1e3,
        "error_stats_frac_hbm_peak": elems * 2.5625 / t_e / 1e3 / PEAK_HBM_GBPS}
    del q, xv
    # decode projection 32 x 10240 x 5120: activation quantisation + GEMM as
    # two library calls and as the one-launch fused call, with COMPUTE
    # (self-calibrated) and GIVEN globals.  Direct C-ABI calls with
    # pre-marshalled arguments keep the Python wrappers' host time out of
    # the GPU timing of these short kernels.
    import ctypes
    lib = nv.library()
    xd, qw = up(5, "x_dec"), nv.quantize(up(5, "w"))
    qd = nv.quantize(xd)
    g_given = qd.global_scale.clone()
    g_out = torch.empty(1, dtype=torch.float32, device=dev)
    yd = torch.empty((32, 10240), dtype=torch.bfloat16, device=dev)
    sv = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    dec = {}
    for mode, g in (("compute", g_out), ("given", g_given)):
        mcode = nv.GLOBAL_COMPUTE if mode == "compute" else nv.GLOBAL_GIVEN
        qargs = (P(xd), nv.DTYPE_BF16, 32, 5120, 5120, P(qd.codes), P(qd.scales), P(g),
                 mcode, sv)
        gargs = (P(qd.codes), P(qd.scales), P(g), 32, P(qw.codes), P(qw.scales),
                 P(qw.global_scale), 10240, 5120, P(yd), nv.DTYPE_BF16, 10240, 0, sv)
        fargs = (P(xd), nv.DTYPE_BF16, 32, 5120, 5120, P(qd.codes), P(qd.scales), P(g),
                 mcode, P(qw.codes), P(qw.scales), P(qw.global_scale), 10240, P(yd),
                 nv.DTYPE_BF16, 10240, sv)
        assert lib.nvfp4_quantize(*qargs) == 0 and lib.w4a4_gemm(*gargs) == 0
        assert lib.w4a4_gemm_quantize_a(*fargs) == 0

        def separate():
            lib.nvfp4_quantize(*qargs)
            lib.w4a4_gemm(*gargs)
        t_sep = _time(separate, 4 * reps, stream)
        t_fus = _time(lambda: lib.w4a4_gemm_quantize_a(*fargs), 4 * reps, stream)
        dec[mode] = {"separate_quantize_gemm_us": t_sep, "fused_us": t_fus,
                     "fused_speedup": t_sep / t_fus}
    out["decode_quantize_gemm_32x10240x5120"] = dec
    del xd, qw, qd, yd
    # FP8 KV cache: calibrate a static scale, cast a 32768 x 1024 bf16 slab
    kvx = torch.randn((32768, 1024), device=dev).to(torch.bfloat16)
    scale, amax = nv.fp8_kv_calibrate([kvx])
    # 67 MB of input: rotated over copies, as above
    nkc = _copies(32768 * 1024 * 3)
    kvs = [kvx.clone() for _ in range(nkc)]
    kvos = [torch.empty((32768, 1024), dtype=torch.uint8, device=dev) for _ in range(nkc)]
    t_a = _time([lambda i=i: nv.fp8_kv_calibrate([kvs[i]], amax=amax) for i in range(nkc)],
                reps, stream)
    t_k = _time([lambda i=i: nv.fp8_kv_cast(kvs[i], scale, out=kvos[i]) for i in range(nkc)],
                reps, stream)
    del kvs, kvos
    kv_el = 32768 * 1024
    out["fp8_kv_32768x1024_bf16"] = {
        "calibrate_us": t_a, "calibrate_gbps_2B_per_elem": kv_el * 2 / t_a / 1e3,
        "cast_us": t_k, "cast_gbps_3B_per_elem": kv_el * 3 / t_k / 1e3,
        "cast_frac_hbm_peak": kv_el * 3 / t_k / 1e3 / PEAK_HBM_GBPS}
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the NVFP4 W4A4 path here is "
              "single-GPU (no collectives); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import nvfp4_w4a4_quantized_03_amd as nv
    import oracle
    import synth

    dev = torch.device("cuda:0")
    print("[bench] generating synthetic inputs", file=sys.stderr, flush=True)
    xv, xbits, _ = synth.workload_tensor(WORKLOAD, "x")
    dv, dbits, _ = synth.workload_tensor(WORKLOAD, "x_dec")
    wv, wbits, _ = synth.workload_tensor(WORKLOAD, "w")

    def upload(bits):
        return torch.from_numpy(bits.view(np.int16)).to(dev).view(
            torch.bfloat16)

    x, xd, w = upload(xbits), upload(dbits), upload(wbits)
    del xbits, dbits, wbits
    stream = torch.cuda.current_stream(dev)

    # weights are pre-quantised (offline); activation globals are the
    # calibrated static values (here: the tensors' own amax-derived g)
    qw = nv.quantize(w)
    gx = nv.quantize(x).global_scale.clone()
    gd = nv.quantize(xd).global_scale.clone()
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    yd = torch.empty((M_DEC, N), dtype=torch.bfloat16, device=dev)
    codes = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((M, K // 16), dtype=torch.uint8, device=dev)
    dcodes = torch.empty((M_DEC, K // 2), dtype=torch.uint8, device=dev)
    dscales = torch.empty((M_DEC, K // 16), dtype=torch.uint8, device=dev)

    names = ["quantize", "gemm", "quantize_dec", "gemm_dec"]
    ev = {n: [] for n in names}

    def step(record):
        marks = []
        if record:
            marks.append(torch.cuda.Event(enable_timing=True))
            marks[-1].record(stream)
        qa = nv.quantize(x, global_scale=gx, out=(codes, scales))
        if record:
            marks.append(torch.cuda.Event(enable_timing=True))
            marks[-1].record(stream)
        nv.gemm(qa, qw, out_dtype=torch.bfloat16, out=y)
        if record:
            marks.append(torch.cuda.Event(enable_timing=True))
            marks[-1].record(stream)
        qd = nv.quantize(xd, global_scale=gd, out=(dcodes, dscales))
        if record:
            marks.append(torch.cuda.Event(enable_timing=True))
            marks[-1].record(stream)
        nv.gemm(qd, qw, out_dtype=torch.bfloat16, out=yd)
        if record:
            marks.append(torch.cuda.Event(enable_timing=True))
            marks[-1].record(stream)
            for i, nme in enumerate(names):
                ev[nme].append((marks[i], marks[i + 1]))

    print("[bench] warmup", args.warmup, file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()

    # the timed region: exactly K steps, synchronised on both sides
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    print("[bench] timed %d steps in %.3f s" % (args.steps, elapsed),
          file=sys.stderr, flush=True)

    if args.copy_calibration:
        src = torch.ones(512 * 2 ** 20 // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    # mean (the roofline's average launch duration) and median per kernel
    avg_ms = {n: float(np.mean([a.elapsed_time(b) for a, b in ev[n]]))
              for n in names}
    med_ms = {n: float(np.median([a.elapsed_time(b) for a, b in ev[n]]))
              for n in names}
    flops_gemm = 2.0 * M * N * K
    flops_step = 2.0 * (M + M_DEC) * N * K
    ms_step = elapsed * 1e3 / args.steps
    q_bytes = M * K * 2.5625           # bf16 in, codes + scales out
    gemm_tflops = flops_gemm / (avg_ms["gemm"] * 1e-3) / 1e12
    q_gbps = q_bytes / (avg_ms["quantize"] * 1e-3) / 1e9
    dec_bytes = N * K * 0.5625 + M_DEC * K * 0.5625 + M_DEC * N * 2
    # sampled parity of this very run's outputs against the oracle
    rows = np.array([0, 1, 4095, 16384, M - 1])
    cols = np.array([0, 7, 5000, N - 1])
    g_x = np.float32(gx.cpu().numpy()[0])
    ca, sa, _ = oracle.quantize(xv[rows], g=g_x)
    cb, sb, gb = oracle.quantize(wv[cols], g=oracle.global_scale(wv))
    ref = oracle.gemm_f64(ca, sa, g_x, cb, sb, gb)
    got = y[torch.from_numpy(rows).to(dev)][:, torch.from_numpy(cols).to(
        dev)].float().cpu().numpy().astype(np.float64)
    ref16, _ = oracle.bf16_rne_from_f64(ref)
    parity_ok = bool(np.all(np.abs(got - ref16) <= np.abs(ref16) * 2.0 ** -7
                            + 1e-30))

    reported = other_workloads(nv, synth, dev, stream) if args.workloads else {}
    traffic = measured_traffic("w4a4_gemm_prefill_32768x10240x5120_traffic.md",
                               1)
    out = {
        "metric": METRIC,
        "value": flops_step / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4->f16 mfma, f32 acc",
        "data": "synthetic",
        "config": {"workload": "long prefill + decode, hidden 5120: "
                               "X[32768x5120] and X[32x5120] bf16 (1% outlier "
                               "channels x60), W[10240x5120] bf16 N(0,0.02) "
                               "pre-quantized; NVFP4 activation quantize per "
                               "call (given global) + W4A4 GEMM, bf16 out",
                   "M": M, "M_decode": M_DEC, "N": N, "K": K},
        "roofline": {"bound": "mfma", "achieved": gemm_tflops,
                     "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": gemm_tflops / PEAK_MFMA_TFLOPS,
                     "traffic": traffic},
        "kernels": {
            "gemm_prefill": {"us": avg_ms["gemm"] * 1e3,
                             "us_median": med_ms["gemm"] * 1e3,
                             "tflops": gemm_tflops,
                             "frac_mfma_peak": gemm_tflops / PEAK_MFMA_TFLOPS},
            "quantize_prefill": {"us": avg_ms["quantize"] * 1e3,
                                 "us_median": med_ms["quantize"] * 1e3,
                                 "gbps": q_gbps,
                                 "frac_hbm_peak": q_gbps / PEAK_HBM_GBPS,
                                 "bytes": q_bytes},
            "quantize_decode": {"us": avg_ms["quantize_dec"] * 1e3,
                                "us_median": med_ms["quantize_dec"] * 1e3},
            "gemm_decode": {"us": avg_ms["gemm_dec"] * 1e3,
                            "us_median": med_ms["gemm_dec"] * 1e3,
                            "gbps": dec_bytes / (avg_ms["gemm_dec"] * 1e-3)
                            / 1e9,
                            "frac_hbm_peak": dec_bytes /
                            (avg_ms["gemm_dec"] * 1e-3) / 1e9 /
                            PEAK_HBM_GBPS},
        },
        "parity_sample_ok": parity_ok,
        "other_workloads": reported,
        "kernel_sources_sha256_16": {s: source_hash(s)
                                     for s in KERNEL_SOURCES},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr,
              flush=True)
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
