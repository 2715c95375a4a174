"""Seeded synthetic inputs for the NVFP4 W4A4 workloads.

This module only draws random numbers and rounds them to the storage dtype;
it holds none of the quantisation or GEMM arithmetic.  Tests, the benchmark
and the oracle checks all take their inputs from here, so the GPU path and
the CPU oracle see the same bits.

Recipe (shapes from the hidden-5120 Gated DeltaNet projections):
  * generator: numpy PCG64, one stream per (workload, tensor, row-chunk of
    1024 rows): default_rng([workload, tensor, chunk]); fp32 normal draws;
  * "outlier" activations: N(0, 1) with 1 % of the K channels (51 of 5120,
    the same channels for every row, drawn from default_rng([workload,
    tensor, 999999])) multiplied by 60 before rounding;
  * weights: N(0, sigma) with the stated sigma;
  * bf16 tensors are the fp32 draws rounded to nearest-even bf16; the same
    bf16 bits go to the device and to the oracle.
"""
import numpy as np

CHUNK = 1024
OUTLIER_FRACTION = 0.01
OUTLIER_GAIN = 60.0


def bf16_bits_from_f32(f):
    """Round binary32 values to bfloat16, nearest-even; returns uint16 bits."""
    u = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1))) >> 16
    return r.astype(np.uint16)


def f32_from_bf16_bits(b):
    """bfloat16 bits -> binary32 values (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(
        np.float32)


def _outlier_channels(workload, tensor, k):
    n = int(round(OUTLIER_FRACTION * k))
    rng = np.random.default_rng([workload, tensor, 999999])
    return np.sort(rng.choice(k, size=n, replace=False))


def normal_rows(workload, tensor, rows, k, sigma=1.0, outliers=False,
                row_ids=None):
    """fp32 draws for the given rows (all rows by default) of a [rows, k]
    tensor.  Rows are generated chunk by chunk, so a subset of rows can be
    produced without drawing the rest."""
    if row_ids is None:
        row_ids = np.arange(rows)
    row_ids = np.asarray(row_ids, dtype=np.int64)
    out = np.empty((len(row_ids), k), dtype=np.float32)
    chunks = np.unique(row_ids // CHUNK)
    ch_cols = _outlier_channels(workload, tensor, k) if outliers else None
    for c in chunks:
        r0 = c * CHUNK
        n = min(CHUNK, rows - r0)
        rng = np.random.default_rng([workload, tensor, int(c)])
        blk = rng.standard_normal((n, k), dtype=np.float32)
        if sigma != 1.0:
            blk *= np.float32(sigma)
        if outliers:
            blk[:, ch_cols] *= np.float32(OUTLIER_GAIN)
        sel = np.nonzero(row_ids // CHUNK == c)[0]
        out[sel] = blk[row_ids[sel] - r0]
    return out


def tensor(workload, tensor_id, rows, k, sigma=1.0, outliers=False,
           dtype="bf16", row_ids=None):
    """Return (values_f32, device_bits) for one tensor.  For bf16,
    device_bits is a uint16 array of bf16 patterns and values_f32 their
    exact fp32 values; for fp32 both are the same float32 array."""
    f = normal_rows(workload, tensor_id, rows, k, sigma, outliers, row_ids)
    if dtype == "f32":
        return f, f
    bits = bf16_bits_from_f32(f)
    return f32_from_bf16_bits(bits), bits


# The five workloads.  Each tensor: (name, tensor_id, rows, k, sigma,
# outliers, dtype).
WORKLOADS = {
    1: dict(name="tiny W4A4 GEMM 16x128x256 fp32",
            tensors=[("x", 0, 16, 256, 1.0, False, "f32"),
                     ("w", 1, 128, 256, 1.0, False, "f32")]),
    2: dict(name="GDN in_proj 4096x12288x5120",
            tensors=[("x", 0, 4096, 5120, 1.0, True, "bf16"),
                     ("w", 1, 12288, 5120, 0.02, False, "bf16")]),
    3: dict(name="GDN gate projections a/b 32768x64x5120",
            tensors=[("x", 0, 32768, 5120, 1.0, True, "bf16"),
                     ("w_a", 1, 64, 5120, 0.02, False, "bf16"),
                     ("w_b", 2, 64, 5120, 0.02, False, "bf16")]),
    4: dict(name="fused group 12288|5120|128 harmonised, X 8192x5120",
            tensors=[("x", 0, 8192, 5120, 1.0, True, "bf16"),
                     ("w1", 1, 12288, 5120, 0.02, False, "bf16"),
                     ("w2", 2, 5120, 5120, 0.05, False, "bf16"),
                     ("w3", 3, 128, 5120, 0.2, False, "bf16")]),
    5: dict(name="long prefill + decode 32768|32 x 10240 x 5120",
            tensors=[("x", 0, 32768, 5120, 1.0, True, "bf16"),
                     ("x_dec", 4, 32, 5120, 1.0, True, "bf16"),
                     ("w", 1, 10240, 5120, 0.02, False, "bf16")]),
}


def workload_tensor(workload, name, row_ids=None):
    """(values_f32, device_bits, dtype) of a named tensor of a workload."""
    for (n, tid, rows, k, sigma, outl, dt) in WORKLOADS[workload]["tensors"]:
        if n == name:
            vals, bits = tensor(workload, tid, rows, k, sigma, outl, dt,
                                row_ids)
            return vals, bits, dt
    raise KeyError(name)


def workload_shape(workload, name):
    for (n, tid, rows, k, sigma, outl, dt) in WORKLOADS[workload]["tensors"]:
        if n == name:
            return rows, k
    raise KeyError(name)
