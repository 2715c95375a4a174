"""W4A4 GEMM on NVFP4 operands and the gate epilogues.
TEST INFRASTRUCTURE ONLY.

The linear layer of [P3] "前提1" with both operands NVFP4 (W4A4):
    y[i, j] = g_a g_b * sum_k A_hat[i, k] B_hat[j, k]
with A_hat = e2m1(code) * e4m3(scale of its 16-block) and B [N, K] stored
K-major like A.  This is a plain definition (a dot product), so the oracle is
that dot product computed exactly:

  * every decoded operand e2m1 * e4m3 is an integer multiple of 2^-10
    (E2M1 in halves, E4M3 in units of 2^-9) of magnitude <= 6 * 448 * 2^10
    < 2^22, so products are integers in units of 2^-20 below 2^44 and a sum
    over K <= 8192 stays below 2^57: int64 accumulation is exact;
  * the one rounding is the final conversion to float64 and the product with
    the two globals.

gemm_f64 does the same with float64 BLAS on the decoded matrices (products
exact, accumulation error <= K 2^-53 of sum |terms|); it serves the full-size
configurations and is cross-checked against the integer tier.

Gates ([P3] "前提2": alpha from the projection output through softplus and
exp, beta through a sigmoid; the workload's form with no extra parameters):
    alpha = exp(-softplus(y)),  beta = 1 / (1 + exp(-y)).
"""
import numpy as np

from .formats import E2M1_MAG, E4M3_POS
from .quantize import unpack_codes, BLOCK

# E2M1 magnitudes in units of 1/2 and E4M3 values in units of 2^-9.
_E2M1_HALVES = np.array([int(v * 2) for v in E2M1_MAG], dtype=np.int64)
_E4M3_UNITS = np.array([int(v * 512) for v in E4M3_POS] + [0], dtype=np.int64)


def decoded_units(codes, scales):
    """Decoded NVFP4 operand (without the global) as int64 in units of
    2^-10: sign * e2m1_halves * e4m3_units."""
    c = unpack_codes(codes).astype(np.int64)
    s = np.asarray(scales, dtype=np.int64)
    if np.any(s == 0x7F) or np.any(s & 0x80):
        raise ValueError("scales must be non-negative finite E4M3")
    mag = _E2M1_HALVES[c & 7]
    sgn = np.where(c & 8, -1, 1)
    sc = np.repeat(_E4M3_UNITS[s], BLOCK, axis=1)
    return sgn * mag * sc


def gemm_exact_int(a_codes, a_scales, a_global, b_codes, b_scales, b_global):
    """Exact W4A4 GEMM: int64 accumulation, float64 result [M, N]."""
    a = decoded_units(a_codes, a_scales)
    b = decoded_units(b_codes, b_scales)
    if a.shape[1] > 8192:
        raise ValueError("exact int64 tier is bounded to K <= 8192")
    acc = a @ b.T                                   # units of 2^-20, exact
    return acc.astype(np.float64) * 2.0 ** -20 * float(a_global) \
        * float(b_global)


def _decoded_f64(codes, scales):
    return decoded_units(codes, scales).astype(np.float64) * 2.0 ** -10


def gemm_f64(a_codes, a_scales, a_global, b_codes, b_scales, b_global):
    """W4A4 GEMM with float64 BLAS on the exactly decoded operands."""
    a = _decoded_f64(a_codes, a_scales)
    b = _decoded_f64(b_codes, b_scales)
    return (a @ b.T) * float(a_global) * float(b_global)


def gemm_f64_row_blocks(a_codes, a_scales, a_global, b_codes, b_scales,
                        b_global, rows_per_block=2048):
    """gemm_f64 of a tall A, one block of rows at a time: yields
    (first_row, y_block).  B is decoded once; every block is computed
    exactly as gemm_f64 computes those rows (it bounds host memory for the
    full-size configurations, nothing else)."""
    b = _decoded_f64(b_codes, b_scales).T.copy()
    scale = float(a_global) * float(b_global)
    rows = np.asarray(a_codes).shape[0]
    for r0 in range(0, rows, rows_per_block):
        a = _decoded_f64(a_codes[r0:r0 + rows_per_block],
                         a_scales[r0:r0 + rows_per_block])
        yield r0, (a @ b) * scale


def gemm_f64_rows_cols(a_codes, a_scales, a_global, b_codes, b_scales,
                       b_global, rows, cols):
    """The outputs y[rows][:, cols] only (sampled check of a large GEMM)."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    return gemm_f64(np.asarray(a_codes)[rows], np.asarray(a_scales)[rows],
                    a_global, np.asarray(b_codes)[cols],
                    np.asarray(b_scales)[cols], b_global)


def gate_alpha(y):
    """Decay gate alpha = exp(-softplus(y)), float64."""
    y = np.asarray(y, dtype=np.float64)
    return np.exp(-np.logaddexp(0.0, y))


def gate_beta(y):
    """Write-strength gate beta = sigmoid(y), float64."""
    y = np.asarray(y, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-y))


def gdn_gates(y, n_beta, a_log, dt_bias):
    """The gate pair of one Gated DeltaNet layer from the fused b|a
    projection output y [m, n_beta + n_alpha] (float64): beta = sigmoid of
    the first n_beta columns, alpha = exp(-exp(A_log) * softplus(a + dt_bias))
    of the rest, per column ([P3] 前提2: a through softplus and an
    exponential in log space, b through a sigmoid; A_log and dt_bias are
    the per-head log-space parameters).  Returns (beta, alpha)."""
    y = np.asarray(y, dtype=np.float64)
    a_log = np.asarray(a_log, dtype=np.float64)
    dt_bias = np.asarray(dt_bias, dtype=np.float64)
    beta = gate_beta(y[:, :n_beta])
    sp = np.logaddexp(0.0, y[:, n_beta:] + dt_bias[None, :])
    alpha = np.exp(-np.exp(a_log)[None, :] * sp)
    return beta, alpha
